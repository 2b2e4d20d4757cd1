"""Plain fp64 CPU oracle of the sequence-tiled gated-SiLU MLP sublayer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` (and nothing in the product
path).

What it computes
----------------
Besides chunking the attention heads, the talk's memory stack tiles the
element-wise parts of the model, the MLP and the loss, along the sequence, so
that no buffer is as long as the whole sequence along one axis (Arctic
sequence length training: "Road to 5 Million Tokens", talk transcript, the
part after CPU offloading; memeeeeeex.com article, the paragraph after
activation checkpointing; liquidgold.cc notes, "Progression of Techniques",
item 6). Tiling a row-wise computation changes the schedule only, so the
result is the plain MLP of every token. The pages do not write the MLP out;
the models they train (Llama 3, Qwen3) use the gated SiLU ("SwiGLU") MLP
without biases, which is the reading taken here:

    h = x Wg^T,  u = x Wu^T,  a = silu(h) * u,  y = a Wd^T,
    silu(z) = z * s(z),  s(z) = 1 / (1 + e^-z)

and its exact backward for an upstream gradient dy:

    dWd = dy^T a,   da = dy Wd,
    dh = da * u * silu'(h),   du = da * silu(h),   silu'(z) = s(z) (1 + z (1 - s(z))),
    dWg = dh^T x,   dWu = du^T x,   dx = dh Wg + du Wu.

The tile loop (``tile`` tokens at a time) is an outer loop only; it exists so
that tests can check that summing the per-tile weight gradients is exact.

Parity pins: ``tests/test_oracle_mlp.py`` checks every function against
PyTorch's CPU silu and autograd in fp64 (library special cases), brute force
in plain Python loops, central finite differences, closed forms and exact
identities; none is "parity unpinned".

Layouts (nn.Linear, [out][in]): x, y, dy, dx [N][D]; Wg, Wu [F][D]; Wd [D][F].
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def sigmoid(z):
    """Logistic sigmoid in fp64, evaluated without overflow for large |z|."""
    z = np.asarray(z, dtype=F64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def silu(z):
    """silu(z) = z * sigmoid(z)."""
    z = np.asarray(z, dtype=F64)
    return z * sigmoid(z)


def silu_grad(z):
    """d silu / dz = s (1 + z (1 - s)), s = sigmoid(z)."""
    z = np.asarray(z, dtype=F64)
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def _tiles(n, tile):
    if tile is None or tile >= n:
        return [(0, n)]
    return [(t0, min(t0 + tile, n)) for t0 in range(0, n, tile)]


def mlp_fwd(x, wg, wu, wd, tile=None):
    """y [N][D] of the gated-SiLU MLP, tile rows at a time (None: all at once)."""
    x, wg, wu, wd = (np.asarray(t, dtype=F64) for t in (x, wg, wu, wd))
    y = np.empty((x.shape[0], wd.shape[0]), dtype=F64)
    for t0, t1 in _tiles(x.shape[0], tile):
        xt = x[t0:t1]
        a = silu(xt @ wg.T) * (xt @ wu.T)
        y[t0:t1] = a @ wd.T
    return y


def mlp_bwd(x, wg, wu, wd, dy, tile=None):
    """Exact backward of ``mlp_fwd``: ``(dx, dwg, dwu, dwd)``.

    Per tile of rows the forward's h and u are recomputed from x (activation
    checkpointing), then the tile's share of each weight gradient is added.
    """
    x, wg, wu, wd, dy = (np.asarray(t, dtype=F64) for t in (x, wg, wu, wd, dy))
    dx = np.empty_like(x)
    dwg = np.zeros_like(wg)
    dwu = np.zeros_like(wu)
    dwd = np.zeros_like(wd)
    for t0, t1 in _tiles(x.shape[0], tile):
        xt, dyt = x[t0:t1], dy[t0:t1]
        h = xt @ wg.T
        u = xt @ wu.T
        sh = silu(h)
        a = sh * u
        dwd += dyt.T @ a
        da = dyt @ wd
        dh = da * u * silu_grad(h)
        du = da * sh
        dwg += dh.T @ xt
        dwu += du.T @ xt
        dx[t0:t1] = dh @ wg + du @ wu
    return dx, dwg, dwu, dwd


def mlp_rows(x_rows, wg, wu, wd):
    """y at a set of rows: the MLP is row-wise, so this is ``mlp_fwd`` of those rows."""
    return mlp_fwd(x_rows, wg, wu, wd)


def mlp_dx_rows(x_rows, dy_rows, wg, wu, wd):
    """dx at a set of rows (row-wise too): the dx part of ``mlp_bwd`` on those rows."""
    return mlp_bwd(x_rows, wg, wu, wd, dy_rows)[0]
