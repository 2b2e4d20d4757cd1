"""Plain fp64 CPU oracle of one GPU's share of a headwise-chunked attention layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s cpu_baseline leg, never by the product path.

What it computes
----------------
The method (Untied Ulysses, also called UPipe) splits the attention heads that
one GPU owns into small chunks and runs them one after another: each chunk's
Q/K/V are recomputed, its attention is computed, its partial result is stored,
and the next chunk reuses the same buffers ("500 万トークンへの道 — Max Ryabinin
(Together AI) の Untied Ulysses", section "Untied Ulysses (UPipe) — head 単位の
チャンク化"; "Road to 5 Million Tokens: Breaking Barriers in Long Context
Training", section "Primary Contribution"). That is a schedule, not an
approximation: the layer output is the plain causal softmax attention layer.
So this oracle is the plain definition written out in fp64:

    q_h = rope(norm_q(x Wq_h^T)),  k_g = rope(norm_k(x Wk_g^T)),  v_g = x Wv_g^T
    S_h = q_h k_{g(h)}^T / sqrt(d)   with keys j > i masked (causal)
    LSE_h[i] = log sum_{j<=i} exp S_h[i, j],   P_h = exp(S_h - LSE_h)
    O_h = P_h v_{g(h)},   y = sum_h O_h Wo_h^T

and its exact backward. The pages give no formulas, so every convention below
(rotate-half RoPE, contiguous GQA groups, RMSNorm over head_dim before RoPE,
1/sqrt(head_dim) scale, key j visible to query i iff j <= i) is the plainest
reading and is listed with the other readings in the design notes.

Parity pins: every function here is checked in ``tests/test_oracle.py``
against brute force, closed forms, library special cases and finite
differences; none is "parity unpinned".

Layouts match the library: x ``[N][D]``; Wq ``[Hq*d][D]`` (head h = rows
``h*d:(h+1)*d``); Wk, Wv ``[Hkv*d][D]``; Wo ``[D][Hq*d]`` (head h = columns);
lse ``[Hq][N]`` (natural log).
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# chunk plan
# --------------------------------------------------------------------------
def chunk_plan(n_q_heads: int, n_kv_heads: int, chunk_heads: int):
    """List of chunks, each ``(q_heads, kv_heads)`` as ranges.

    Heads of one GPU are taken in contiguous chunks of ``chunk_heads``
    (section "Untied Ulysses (UPipe) — head 単位のチャンク化" of the
    memeeeeeex.com article: the heads owned by a GPU are split into chunks
    iterated over in time). q head h reads kv head ``h // G`` with
    ``G = n_q_heads // n_kv_heads``.
    """
    if n_q_heads % n_kv_heads:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if n_q_heads % chunk_heads:
        raise ValueError("chunk_heads must divide n_q_heads")
    g = n_q_heads // n_kv_heads
    if chunk_heads % g and g % chunk_heads:
        raise ValueError("chunk_heads must divide, or be a multiple of, the GQA group size")
    out = []
    for c0 in range(0, n_q_heads, chunk_heads):
        qs = range(c0, c0 + chunk_heads)
        kvs = range(c0 // g, (c0 + chunk_heads - 1) // g + 1)
        out.append((qs, kvs))
    return out


# --------------------------------------------------------------------------
# RoPE (rotate-half pairing (i, i + d/2), omega_i = theta^(-2i/d))
# --------------------------------------------------------------------------
def rope_cos_sin(positions, head_dim: int, theta: float):
    """cos/sin of the rotary angles ``a[p, i] = p * theta^(-2i/d)``, fp64, ``[P][d/2]``."""
    pos = np.asarray(positions, dtype=F64)
    i = np.arange(head_dim // 2, dtype=F64)
    omega = float(theta) ** (-2.0 * i / head_dim)
    ang = pos[:, None] * omega[None, :]
    return np.cos(ang), np.sin(ang)


def apply_rope(t, positions, theta: float):
    """Rotate each pair ``(t[p, i], t[p, i + d/2])`` by angle ``a[p, i]``."""
    t = np.asarray(t, dtype=F64)
    d = t.shape[-1]
    c, s = rope_cos_sin(positions, d, theta)
    u, w = t[..., : d // 2], t[..., d // 2:]
    return np.concatenate([u * c - w * s, w * c + u * s], axis=-1)


def rope_transpose(dt, positions, theta: float):
    """Adjoint of ``apply_rope``: rotate each pair by ``-a[p, i]``."""
    dt = np.asarray(dt, dtype=F64)
    d = dt.shape[-1]
    c, s = rope_cos_sin(positions, d, theta)
    du, dw = dt[..., : d // 2], dt[..., d // 2:]
    return np.concatenate([du * c + dw * s, -du * s + dw * c], axis=-1)


# --------------------------------------------------------------------------
# per-head RMSNorm over head_dim (Qwen-shaped q/k norm)
# --------------------------------------------------------------------------
def rmsnorm(u, gamma, eps: float):
    """``gamma * u / sqrt(mean(u^2) + eps)`` over the last axis."""
    u = np.asarray(u, dtype=F64)
    r = 1.0 / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)
    return np.asarray(gamma, dtype=F64) * (u * r)


def rmsnorm_bwd(u, gamma, eps: float, dout):
    """Gradients of ``rmsnorm`` w.r.t. u and gamma (gamma grad summed over rows)."""
    u = np.asarray(u, dtype=F64)
    dout = np.asarray(dout, dtype=F64)
    d = u.shape[-1]
    r = 1.0 / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)
    uh = u * r
    gh = np.asarray(gamma, dtype=F64) * dout
    du = r * (gh - uh * np.sum(gh * uh, axis=-1, keepdims=True) / d)
    dgamma = np.sum((dout * uh).reshape(-1, d), axis=0)
    return du, dgamma


# --------------------------------------------------------------------------
# causal attention core (one q head against its kv head)
# --------------------------------------------------------------------------
def _causal_mask(q_pos, k_pos):
    return np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]


def causal_attention(q, k, v, q_pos=None, k_pos=None):
    """Causal softmax attention of one head, fp64.

    ``q [R][d]`` at positions ``q_pos``, ``k, v [M][d]`` at ``k_pos``; key j is
    visible to query i iff ``k_pos[j] <= q_pos[i]``. Returns ``(O, LSE, P)``.
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    if q_pos is None:
        q_pos = np.arange(q.shape[0])
    if k_pos is None:
        k_pos = np.arange(k.shape[0])
    d = q.shape[-1]
    s = (q @ k.T) / math.sqrt(d)
    mask = _causal_mask(q_pos, k_pos)
    s = np.where(mask, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    lse = m[:, 0] + np.log(np.sum(np.exp(s - m), axis=-1))
    p = np.exp(s - lse[:, None])
    return p @ v, lse, p


def causal_attention_bwd(q, k, v, p, do):
    """Exact backward of ``causal_attention`` given its P; returns ``(dq, dk, dv)``.

    dP = dO V^T, Delta_i = sum_j P_ij dP_ij, dS = P (dP - Delta),
    dq = dS k / sqrt(d), dk = dS^T q / sqrt(d), dv = P^T dO.
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    do = np.asarray(do, dtype=F64)
    d = q.shape[-1]
    dp = do @ v.T
    delta = np.sum(p * dp, axis=-1, keepdims=True)
    ds = p * (dp - delta)
    dq = ds @ k / math.sqrt(d)
    dk = ds.T @ q / math.sqrt(d)
    dv = p.T @ do
    return dq, dk, dv


# --------------------------------------------------------------------------
# the layer on one GPU's share
# --------------------------------------------------------------------------
def _proj(x, w, h, d):
    return np.asarray(x, dtype=F64) @ np.asarray(w[h * d:(h + 1) * d], dtype=F64).T


def _qk_heads(x, w, h, d, gamma, eps, theta, positions, use_rope=True):
    """One head's projection -> optional RMSNorm -> RoPE. Returns (final, pre_norm)."""
    u = _proj(x, w, h, d)
    t = rmsnorm(u, gamma, eps) if gamma is not None else u
    if use_rope:
        t = apply_rope(t, positions, theta)
    return t, u


def layer_fwd(x, wq, wk, wv, wo, n_q_heads, n_kv_heads, head_dim, rope_theta,
              chunk_heads, q_norm=None, k_norm=None, eps=1e-6, use_rope=True,
              keep=False):
    """Forward of the layer: ``y [N][D]`` and ``lse [Hq][N]``.

    Heads run chunk by chunk and each chunk's partial output is added into y,
    as the method describes; the sum is exact, so y does not depend on the
    chunk size. With ``keep=True`` also returns the per-head intermediates.
    """
    x = np.asarray(x, dtype=F64)
    N = x.shape[0]
    d = head_dim
    pos = np.arange(N)
    g = n_q_heads // n_kv_heads
    y = np.zeros((N, np.asarray(wo).shape[0]), dtype=F64)
    lse = np.zeros((n_q_heads, N), dtype=F64)
    inter = {"q": {}, "k": {}, "v": {}, "o": {}, "p": {}, "uq": {}, "uk": {}}
    for qs, kvs in chunk_plan(n_q_heads, n_kv_heads, chunk_heads):
        kv = {}
        for kh in kvs:
            k, uk = _qk_heads(x, wk, kh, d, k_norm, eps, rope_theta, pos, use_rope)
            kv[kh] = (k, _proj(x, wv, kh, d))
            inter["k"][kh], inter["v"][kh], inter["uk"][kh] = k, kv[kh][1], uk
        part = np.zeros_like(y)
        for h in qs:
            q, uq = _qk_heads(x, wq, h, d, q_norm, eps, rope_theta, pos, use_rope)
            k, v = kv[h // g]
            o, l_h, p = causal_attention(q, k, v)
            lse[h] = l_h
            part += o @ np.asarray(wo[:, h * d:(h + 1) * d], dtype=F64).T
            if keep:
                inter["q"][h], inter["uq"][h], inter["o"][h], inter["p"][h] = q, uq, o, p
        y += part
    if keep:
        return y, lse, inter
    return y, lse


def layer_bwd(x, wq, wk, wv, wo, dy, n_q_heads, n_kv_heads, head_dim, rope_theta,
              chunk_heads, q_norm=None, k_norm=None, eps=1e-6, use_rope=True):
    """Exact backward of ``layer_fwd`` for upstream gradient ``dy``.

    Returns ``(dx, dwq, dwk, dwv, dwo, dq_norm, dk_norm)``; the norm grads are
    None when the layer has no q/k norm. Per head h of kv group g:
    dO = dY Wo_h, dWo_h = dY^T O_h, attention backward, RoPE transpose,
    RMSNorm backward, dWq_h = dq^T x, dx += dq Wq_h (same for k and v).
    """
    x = np.asarray(x, dtype=F64)
    dy = np.asarray(dy, dtype=F64)
    N = x.shape[0]
    d = head_dim
    pos = np.arange(N)
    g = n_q_heads // n_kv_heads
    _, _, it = layer_fwd(x, wq, wk, wv, wo, n_q_heads, n_kv_heads, head_dim, rope_theta,
                         chunk_heads, q_norm, k_norm, eps, use_rope, keep=True)
    dx = np.zeros_like(x)
    dwq = np.zeros(np.asarray(wq).shape, dtype=F64)
    dwk = np.zeros(np.asarray(wk).shape, dtype=F64)
    dwv = np.zeros(np.asarray(wv).shape, dtype=F64)
    dwo = np.zeros(np.asarray(wo).shape, dtype=F64)
    dqn = np.zeros(d, dtype=F64) if q_norm is not None else None
    dkn = np.zeros(d, dtype=F64) if k_norm is not None else None
    dk_acc = {kh: np.zeros((N, d)) for kh in range(n_kv_heads)}
    dv_acc = {kh: np.zeros((N, d)) for kh in range(n_kv_heads)}
    for qs, _ in chunk_plan(n_q_heads, n_kv_heads, chunk_heads):
        for h in qs:
            kh = h // g
            wo_h = np.asarray(wo[:, h * d:(h + 1) * d], dtype=F64)
            do = dy @ wo_h
            dwo[:, h * d:(h + 1) * d] = dy.T @ it["o"][h]
            dq, dk, dv = causal_attention_bwd(it["q"][h], it["k"][kh], it["v"][kh], it["p"][h], do)
            dk_acc[kh] += dk
            dv_acc[kh] += dv
            if use_rope:
                dq = rope_transpose(dq, pos, rope_theta)
            if q_norm is not None:
                dq, dg = rmsnorm_bwd(it["uq"][h], q_norm, eps, dq)
                dqn += dg
            dwq[h * d:(h + 1) * d] = dq.T @ x
            dx += dq @ np.asarray(wq[h * d:(h + 1) * d], dtype=F64)
    for kh in range(n_kv_heads):
        dk = dk_acc[kh]
        if use_rope:
            dk = rope_transpose(dk, pos, rope_theta)
        if k_norm is not None:
            dk, dg = rmsnorm_bwd(it["uk"][kh], k_norm, eps, dk)
            dkn += dg
        dv = dv_acc[kh]
        dwk[kh * d:(kh + 1) * d] = dk.T @ x
        dwv[kh * d:(kh + 1) * d] = dv.T @ x
        dx += dk @ np.asarray(wk[kh * d:(kh + 1) * d], dtype=F64)
        dx += dv @ np.asarray(wv[kh * d:(kh + 1) * d], dtype=F64)
    return dx, dwq, dwk, dwv, dwo, dqn, dkn


# --------------------------------------------------------------------------
# large-N variants: the same definition restricted to selected rows
# --------------------------------------------------------------------------
def _kv_all(x_rows_fn, n_tokens, wk, wv, kh, d, k_norm, eps, theta, block, use_rope=True):
    """k, v of kv head ``kh`` for every token, computed block by block of x."""
    k = np.empty((n_tokens, d), dtype=F64)
    v = np.empty((n_tokens, d), dtype=F64)
    for r0 in range(0, n_tokens, block):
        r1 = min(n_tokens, r0 + block)
        xb = np.asarray(x_rows_fn(r0, r1), dtype=F64)
        kb, _ = _qk_heads(xb, wk, kh, d, k_norm, eps, theta, np.arange(r0, r1), use_rope)
        k[r0:r1] = kb
        v[r0:r1] = _proj(xb, wv, kh, d)
    return k, v


def layer_fwd_rows(x_rows_fn, x_at_fn, n_tokens, rows, wq, wk, wv, wo, n_q_heads,
                   n_kv_heads, head_dim, rope_theta, q_norm=None, k_norm=None,
                   eps=1e-6, block=65536, row_group=16, progress=None):
    """y and lse at selected query rows only (same definition as ``layer_fwd``).

    ``x_rows_fn(r0, r1)`` returns rows ``[r0, r1)`` of x and ``x_at_fn(idx)``
    returns the rows ``idx``; K and V are needed for all tokens, Q, S, P and O
    only for the selected rows (taken ``row_group`` rows at a time: rows are
    independent, so this bounds memory without reordering any sum).
    ``progress(msg)``, if given, is called after each kv head's K/V and each
    q head (long runs report as they go; it does not touch the arithmetic).
    Returns ``(y_rows [R][D], lse_rows [Hq][R])``.
    """
    rows = np.asarray(rows, dtype=np.int64)
    d = head_dim
    g = n_q_heads // n_kv_heads
    x_sel = np.asarray(x_at_fn(rows), dtype=F64)
    y = np.zeros((rows.size, np.asarray(wo).shape[0]), dtype=F64)
    lse = np.zeros((n_q_heads, rows.size), dtype=F64)
    kpos = np.arange(n_tokens)
    for kh in range(n_kv_heads):
        k, v = _kv_all(x_rows_fn, n_tokens, wk, wv, kh, d, k_norm, eps, rope_theta, block)
        if progress:
            progress(f"oracle: k, v of kv head {kh}")
        for h in range(kh * g, (kh + 1) * g):
            q, _ = _qk_heads(x_sel, wq, h, d, q_norm, eps, rope_theta, rows)
            wo_h = np.asarray(wo[:, h * d:(h + 1) * d], dtype=F64)
            for r0 in range(0, rows.size, row_group):
                r1 = min(rows.size, r0 + row_group)
                o, l_h, _ = causal_attention(q[r0:r1], k, v, q_pos=rows[r0:r1], k_pos=kpos)
                lse[h, r0:r1] = l_h
                y[r0:r1] += o @ wo_h.T
            if progress:
                progress(f"oracle: rows of q head {h}")
    return y, lse


def layer_bwd_tail_dx(x_rows_fn, dy_rows_fn, n_tokens, tail, rows, wq, wk, wv, wo,
                      n_q_heads, n_kv_heads, head_dim, rope_theta, q_norm=None,
                      k_norm=None, eps=1e-6, block=65536, row_group=32, progress=None):
    """dx at selected rows inside the last ``tail`` positions.

    For a row i near the end, dq_i needs only query row i, and dk_i, dv_i need
    only queries q >= i, all of which lie inside the tail window; so the exact
    dx rows follow from K/V of all tokens plus Q, dO, LSE and Delta of the
    window. The window's queries are taken ``row_group`` at a time (each
    query's P row is independent; dk/dv sum their contributions).
    ``progress(msg)`` as in ``layer_fwd_rows``.
    Returns ``dx_rows [R][D]``.
    """
    rows = np.asarray(rows, dtype=np.int64)
    t0 = n_tokens - tail
    assert rows.min() >= t0
    d = head_dim
    g = n_q_heads // n_kv_heads
    sq = math.sqrt(d)
    xw = np.asarray(x_rows_fn(t0, n_tokens), dtype=F64)
    dyw = np.asarray(dy_rows_fn(t0, n_tokens), dtype=F64)
    wpos = np.arange(t0, n_tokens)
    kpos = np.arange(n_tokens)
    sel = rows - t0
    dx = np.zeros((rows.size, xw.shape[1]), dtype=F64)
    for kh in range(n_kv_heads):
        k, v = _kv_all(x_rows_fn, n_tokens, wk, wv, kh, d, k_norm, eps, rope_theta, block)
        if progress:
            progress(f"oracle: k, v of kv head {kh}")
        _, uk = _qk_heads(xw, wk, kh, d, k_norm, eps, rope_theta, wpos)
        dk_w = np.zeros((tail, d))
        dv_w = np.zeros((tail, d))
        for h in range(kh * g, (kh + 1) * g):
            q, uq = _qk_heads(xw, wq, h, d, q_norm, eps, rope_theta, wpos)
            do = dyw @ np.asarray(wo[:, h * d:(h + 1) * d], dtype=F64)
            dq = np.zeros((tail, d))
            for r0 in range(0, tail, row_group):
                r1 = min(tail, r0 + row_group)
                _, _, p = causal_attention(q[r0:r1], k, v, q_pos=wpos[r0:r1], k_pos=kpos)
                dp = do[r0:r1] @ v.T
                delta = np.sum(p * dp, axis=-1, keepdims=True)
                ds = p * (dp - delta)
                dq[r0:r1] = ds @ k / sq
                dk_w += ds[:, t0:].T @ q[r0:r1] / sq
                dv_w += p[:, t0:].T @ do[r0:r1]
            dq = rope_transpose(dq, wpos, rope_theta)
            if q_norm is not None:
                dq, _ = rmsnorm_bwd(uq, q_norm, eps, dq)
            dx += dq[sel] @ np.asarray(wq[h * d:(h + 1) * d], dtype=F64)
            if progress:
                progress(f"oracle: tail of q head {h}")
        dk_w = rope_transpose(dk_w, wpos, rope_theta)
        if k_norm is not None:
            dk_w, _ = rmsnorm_bwd(uk, k_norm, eps, dk_w)
        dx += dk_w[sel] @ np.asarray(wk[kh * d:(kh + 1) * d], dtype=F64)
        dx += dv_w[sel] @ np.asarray(wv[kh * d:(kh + 1) * d], dtype=F64)
    return dx
