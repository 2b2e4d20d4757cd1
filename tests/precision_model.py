"""The attention layer's backward in plain fp32 arithmetic with io-dtype storage.

Test infrastructure for inputs too ill-conditioned for the layer's fixed
tolerances (the sharp-softmax stress cases): how far does the *same math*,
done plainly in the precision the GPU path works in, land from the fp64
oracle? Whatever that distance is, no implementation in that precision can
be expected to do much better, so it sets the scale of a derived tolerance.

What is modelled, per head (numpy float32 throughout, one head at a time):
  * q, k, v projected and rotated in fp32, stored in the io dtype;
  * S = q k^T / sqrt(d), the softmax and P in fp32, P stored in the io dtype
    before it multiplies V; O = P V stored in the io dtype;
  * dO = dY Wo_h stored in the io dtype; dP = dO V^T, Delta = rowsum(dO O)
    and dS = P (dP - Delta) in fp32, dS stored in the io dtype before its
    products; dq, dk, dv summed in fp32, rotated back and stored in the io
    dtype; the weight gradients and dx summed in fp32 from those.
Nothing here is the GPU path's code or order of operations: it is the
textbook backward, rounded where any implementation storing io-dtype
operands must round. It is not the oracle (``oracle.layer_bwd`` is exact
fp64), and no test compares the GPU with it directly.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from headwise_chunked_attention_amd.synth import round_to_bf16

F32 = np.float32


def _store(a, io):
    a = np.asarray(a, F32)
    return round_to_bf16(a) if io == "bf16" else a


def plain_grads(inp, n_q_heads, n_kv_heads, head_dim, theta, io):
    """(dx, dwq, dwk, dwv, dwo) of the layer (no q/k norm) in fp32 arithmetic
    with io-dtype storage, as float64 arrays."""
    d = head_dim
    x = np.asarray(inp.x, F32)
    dy = np.asarray(inp.dy, F32)
    N = x.shape[0]
    pos = np.arange(N)
    g = n_q_heads // n_kv_heads
    c, s = (a.astype(F32) for a in oracle.rope_cos_sin(pos, d, theta))

    def rope(t):
        u, w = t[:, : d // 2], t[:, d // 2:]
        return np.concatenate([u * c - w * s, w * c + u * s], axis=1)

    def rope_t(t):
        u, w = t[:, : d // 2], t[:, d // 2:]
        return np.concatenate([u * c + w * s, -u * s + w * c], axis=1)

    def rows(w, h):
        return np.asarray(w[h * d:(h + 1) * d], F32)

    rs = F32(1.0 / math.sqrt(d))
    later = np.triu(np.ones((N, N), bool), 1)
    dx = np.zeros(x.shape, F32)
    dwq = np.zeros(np.shape(inp.wq), F32)
    dwk = np.zeros(np.shape(inp.wk), F32)
    dwv = np.zeros(np.shape(inp.wv), F32)
    dwo = np.zeros(np.shape(inp.wo), F32)
    for kh in range(n_kv_heads):
        k = _store(rope(x @ rows(inp.wk, kh).T), io)
        v = _store(x @ rows(inp.wv, kh).T, io)
        dk = np.zeros((N, d), F32)
        dv = np.zeros((N, d), F32)
        for h in range(kh * g, (kh + 1) * g):
            q = _store(rope(x @ rows(inp.wq, h).T), io)
            sc = (q @ k.T) * rs
            sc[later] = -np.inf
            m = sc.max(axis=1, keepdims=True)
            lse = m + np.log(np.exp(sc - m).sum(axis=1, keepdims=True, dtype=F32))
            p = np.exp(sc - lse).astype(F32)
            ps = _store(p, io)
            o = _store(ps @ v, io)
            wo_h = np.asarray(inp.wo[:, h * d:(h + 1) * d], F32)
            do = _store(dy @ wo_h, io)
            dwo[:, h * d:(h + 1) * d] = dy.T @ o
            dp = do @ v.T
            delta = (do * o).sum(axis=1, keepdims=True, dtype=F32)
            ds = _store(p * (dp - delta), io)
            dq = _store(rope_t((ds @ k) * rs), io)
            dk += (ds.T @ q) * rs
            dv += ps.T @ do
            dwq[h * d:(h + 1) * d] = dq.T @ x
            dx += dq @ rows(inp.wq, h)
        dk = _store(rope_t(dk), io)
        dv = _store(dv, io)
        dwk[kh * d:(kh + 1) * d] = dk.T @ x
        dwv[kh * d:(kh + 1) * d] = dv.T @ x
        dx += dk @ rows(inp.wk, kh) + dv @ rows(inp.wv, kh)
    return tuple(a.astype(np.float64) for a in (dx, dwq, dwk, dwv, dwo))
