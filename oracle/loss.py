"""Plain fp64 CPU oracle of the sequence-tiled cross-entropy loss (LM head).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` (and nothing in the product
path).

What it computes
----------------
The talk's memory stack tiles the element-wise computations, the loss among
them, along the sequence so that no buffer is as long as the whole sequence
along one axis (Arctic sequence length training: "Road to 5 Million Tokens",
talk transcript, the part after CPU offloading; liquidgold.cc notes,
"Progression of Techniques", item 6). For the language-model loss the
sequence-long buffer is the logits tensor [N][V]. The pages do not write the
loss out; the plainest reading is the per-token next-token cross-entropy of
the LM head, computed tile by tile:

    z = h W^T                       (logits, [N][V])
    lse_i = log sum_v exp z[i, v]
    loss_i = lse_i - z[i, t_i]      (t_i the target token of row i)

and its exact backward for an upstream gradient g_i of each token's loss:

    dz = (softmax(z) - onehot(t)) * g[:, None],   dh = dz W,   dW = dz^T h.

Tiling the tokens is a schedule only; the tile loop below exists so that
tests can check that summing per-tile weight gradients is exact.

Parity pins: ``tests/test_oracle_loss.py`` checks these against PyTorch's CPU
cross_entropy and autograd in fp64, brute force in plain Python loops,
central finite differences and closed forms (equal logits give log V).

Layouts: h, dh [N][D]; W, dW [V][D] (nn.Linear [out][in]); targets [N] int;
lse, loss, g [N].
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _tiles(n, tile):
    if tile is None or tile >= n:
        return [(0, n)]
    return [(t0, min(t0 + tile, n)) for t0 in range(0, n, tile)]


def _logsumexp_rows(z):
    m = np.max(z, axis=1)
    return m + np.log(np.sum(np.exp(z - m[:, None]), axis=1))


def ce_fwd(h, w, targets, tile=None):
    """Per-token losses and log-sum-exps: ``(loss [N], lse [N])``."""
    h, w = np.asarray(h, dtype=F64), np.asarray(w, dtype=F64)
    targets = np.asarray(targets, dtype=np.int64)
    n = h.shape[0]
    loss = np.empty(n, dtype=F64)
    lse = np.empty(n, dtype=F64)
    for t0, t1 in _tiles(n, tile):
        z = h[t0:t1] @ w.T
        lse[t0:t1] = _logsumexp_rows(z)
        loss[t0:t1] = lse[t0:t1] - z[np.arange(t1 - t0), targets[t0:t1]]
    return loss, lse


def ce_bwd(h, w, targets, g, tile=None):
    """Exact backward of ``ce_fwd`` for per-token upstream gradients g: ``(dh, dW)``."""
    h, w, g = np.asarray(h, dtype=F64), np.asarray(w, dtype=F64), np.asarray(g, dtype=F64)
    targets = np.asarray(targets, dtype=np.int64)
    n = h.shape[0]
    dh = np.empty_like(h)
    dw = np.zeros_like(w)
    for t0, t1 in _tiles(n, tile):
        z = h[t0:t1] @ w.T
        p = np.exp(z - _logsumexp_rows(z)[:, None])
        p[np.arange(t1 - t0), targets[t0:t1]] -= 1.0
        dz = p * g[t0:t1, None]
        dh[t0:t1] = dz @ w
        dw += dz.T @ h[t0:t1]
    return dh, dw


def ce_rows(h_rows, w, target_rows):
    """loss and lse at a set of rows (row-wise: ``ce_fwd`` of those rows)."""
    return ce_fwd(h_rows, w, target_rows)


def ce_dh_rows(h_rows, w, target_rows, g_rows):
    """dh at a set of rows (row-wise too)."""
    return ce_bwd(h_rows, w, target_rows, g_rows)[0]
