"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module draws random numbers and nothing else: it holds none of the
attention layer's arithmetic. Both the GPU path and the CPU oracle read the
same arrays from here, so a parity failure can never come from two different
input streams.

Recipe (stated once, used everywhere):
  * every tensor has an integer "tensor id": x 0, Wq 1, Wk 2, Wv 3, Wo 4,
    dY 5, q-norm gamma 6, k-norm gamma 7, MLP gate/up/down weights 8/9/10,
    LM-head weight 11, loss targets 12, per-token loss gradients 13, the
    block's attention-norm and MLP-norm gammas 14/15;
  * a 2-D tensor is drawn in blocks of ``ROW_BLOCK`` rows; block ``b`` of
    tensor ``t`` under run seed ``s`` uses
    ``numpy.random.default_rng(SeedSequence([s, t, b]))`` and draws
    ``standard_normal(float32)``, scaled by the tensor's std;
  * bf16 inputs are the fp32 draws rounded to nearest-even bf16, so the value
    the GPU sees is exactly representable in fp32/fp64 on the host.

Any block can therefore be regenerated on its own, which lets the oracle check
sampled rows of a very long sequence without holding the whole of x.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROW_BLOCK = 8192
GEN_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))

TENSOR_IDS = {"x": 0, "wq": 1, "wk": 2, "wv": 3, "wo": 4, "dy": 5, "q_norm": 6, "k_norm": 7,
              "wg": 8, "wu": 9, "wd": 10, "w_lm": 11, "targets": 12, "g_loss": 13,
              "attn_norm": 14, "mlp_norm": 15}


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns a new float32 array."""
    out = np.array(a, dtype=np.float32, copy=True, order="C")
    _round_bf16_inplace(out)
    return out


def _round_bf16_inplace(a: np.ndarray, rows_per_pass: int = 4096) -> None:
    """In-place round-to-nearest-even of a C-contiguous float32 array to bf16 values."""
    flat = a.reshape(a.shape[0], -1) if a.ndim > 1 else a.reshape(1, -1)
    for r0 in range(0, flat.shape[0], rows_per_pass):
        u = flat[r0:r0 + rows_per_pass].view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        u += np.uint32(0x7FFF)
        u += lsb
        u &= np.uint32(0xFFFF0000)


def _block_rng(seed: int, tensor_id: int, block: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(tensor_id), int(block)]))


def gen_rows(name: str, rows: int, cols: int, std: float, dtype: str, seed: int = 0,
             row_start: int = 0, row_stop: int | None = None,
             row_scale: np.ndarray | None = None) -> np.ndarray:
    """Rows ``[row_start, row_stop)`` of the ``rows x cols`` tensor ``name``.

    ``row_scale`` (length ``rows``), if given, multiplies row p by
    ``row_scale[p]`` after the std and before the bf16 rounding.
    Returns float32 (already bf16-rounded when ``dtype == 'bf16'``).
    """
    if row_stop is None:
        row_stop = rows
    assert 0 <= row_start <= row_stop <= rows
    if dtype not in ("bf16", "fp32"):
        raise ValueError(f"unknown dtype {dtype}")
    tid = TENSOR_IDS[name]
    out = np.empty((row_stop - row_start, cols), dtype=np.float32)
    b0 = row_start // ROW_BLOCK
    b1 = (row_stop + ROW_BLOCK - 1) // ROW_BLOCK

    def fill(b):
        lo = b * ROW_BLOCK
        hi = min(rows, lo + ROW_BLOCK)
        s0 = max(lo, row_start)
        s1 = min(hi, row_stop)
        dst = out[s0 - row_start:s1 - row_start]
        rng = _block_rng(seed, tid, b)
        if s0 == lo and s1 == hi:
            rng.standard_normal((hi - lo, cols), dtype=np.float32, out=dst)
        else:
            dst[...] = rng.standard_normal((hi - lo, cols), dtype=np.float32)[s0 - lo:s1 - lo]
        if std != 1.0:
            dst *= np.float32(std)
        if row_scale is not None:
            dst *= np.asarray(row_scale[s0:s1], dtype=np.float32)[:, None]
        if dtype == "bf16":
            _round_bf16_inplace(dst)

    # blocks are independent streams, so they can be drawn on several threads
    # (numpy's generators release the GIL while filling)
    nblk = b1 - b0
    if nblk > 1 and (row_stop - row_start) * cols >= (1 << 22):
        with ThreadPoolExecutor(max_workers=min(GEN_THREADS, nblk)) as ex:
            list(ex.map(fill, range(b0, b1)))
    else:
        for b in range(b0, b1):
            fill(b)
    return out


def gen_rows_at(name: str, rows: int, cols: int, std: float, dtype: str, seed: int,
                idx: np.ndarray) -> np.ndarray:
    """Selected rows ``idx`` (any order) of tensor ``name``; regenerates only their blocks."""
    idx = np.asarray(idx, dtype=np.int64)
    out = np.empty((idx.size, cols), dtype=np.float32)
    blocks = np.unique(idx // ROW_BLOCK)
    for b in blocks:
        lo = int(b) * ROW_BLOCK
        hi = min(rows, lo + ROW_BLOCK)
        blk = gen_rows(name, rows, cols, std, dtype, seed, lo, hi)
        sel = np.nonzero((idx >= lo) & (idx < hi))[0]
        out[sel] = blk[idx[sel] - lo]
    return out


def gen_gamma(name: str, d: int, mode: str, dtype: str, seed: int = 0) -> np.ndarray:
    """RMSNorm weight of length d: ``mode='ones'`` or ``'random'`` (1 + 0.1*N(0,1))."""
    if mode == "ones":
        return np.ones(d, dtype=np.float32)
    g = 1.0 + 0.1 * gen_rows(name, 1, d, 1.0, "fp32", seed)[0]
    g = g.astype(np.float32)
    return round_to_bf16(g) if dtype == "bf16" else g


def sharp_x_row_scale(n_tokens: int, first: int = 64, first_scale: float = 1.0 / 16,
                      growth: float = 0.25) -> np.ndarray:
    """Row scales of x for the sharp-softmax stress inputs: the first ``first``
    rows are shrunk by ``first_scale`` (the keys of a causal row's first tile
    then score near 0 against every query), and the rest grow linearly from 1
    to ``1 + growth`` along the sequence (later keys score higher)."""
    p = np.arange(n_tokens, dtype=np.float64)
    s = 1.0 + growth * p / max(1, n_tokens)
    s[:first] = first_scale
    return s.astype(np.float32)


class LayerInputs:
    """All inputs of one attention-layer problem, as float32 host arrays.

    Shapes follow the library's layout: x, dy ``[N][D]``; wq ``[Hq*d][D]``;
    wk, wv ``[Hkv*d][D]``; wo ``[D][Hq*d]``; gammas ``[d]`` or None.
    ``qk_std`` (default ``w_std``) is the std of Wq and Wk alone and
    ``x_row_scale`` an optional per-row scale of x: together they make the
    sharp-softmax stress inputs (logit std ``d_model * qk_std**2``).
    """

    def __init__(self, n_tokens: int, d_model: int, n_q_heads: int, n_kv_heads: int,
                 head_dim: int, dtype: str, seed: int = 0, w_std: float = 0.02,
                 qk_norm: str | None = None, with_x: bool = True, with_dy: bool = True,
                 qk_std: float | None = None, x_row_scale: np.ndarray | None = None):
        self.n_tokens, self.d_model = n_tokens, d_model
        self.n_q_heads, self.n_kv_heads, self.head_dim = n_q_heads, n_kv_heads, head_dim
        self.dtype, self.seed, self.w_std = dtype, seed, w_std
        N, D, d = n_tokens, d_model, head_dim
        qk_std = w_std if qk_std is None else qk_std
        self.x = gen_rows("x", N, D, 1.0, dtype, seed, row_scale=x_row_scale) if with_x else None
        self.dy = gen_rows("dy", N, D, 1.0, dtype, seed) if with_dy else None
        self.wq = gen_rows("wq", n_q_heads * d, D, qk_std, dtype, seed)
        self.wk = gen_rows("wk", n_kv_heads * d, D, qk_std, dtype, seed)
        self.wv = gen_rows("wv", n_kv_heads * d, D, w_std, dtype, seed)
        self.wo = gen_rows("wo", D, n_q_heads * d, w_std, dtype, seed)
        if qk_norm is None:
            self.q_norm = self.k_norm = None
        else:
            self.q_norm = gen_gamma("q_norm", d, qk_norm, dtype, seed)
            self.k_norm = gen_gamma("k_norm", d, qk_norm, dtype, seed)


class MlpInputs:
    """All inputs of one gated-SiLU MLP problem, as float32 host arrays.

    x, dy ``[N][D]`` (std 1); wg, wu ``[F][D]``, wd ``[D][F]`` (std ``w_std``).
    """

    def __init__(self, n_tokens: int, d_model: int, d_ff: int, dtype: str, seed: int = 0,
                 w_std: float = 0.02, with_x: bool = True, with_dy: bool = True):
        self.n_tokens, self.d_model, self.d_ff, self.dtype, self.seed = n_tokens, d_model, d_ff, dtype, seed
        N, D, F = n_tokens, d_model, d_ff
        self.x = gen_rows("x", N, D, 1.0, dtype, seed) if with_x else None
        self.dy = gen_rows("dy", N, D, 1.0, dtype, seed) if with_dy else None
        self.wg = gen_rows("wg", F, D, w_std, dtype, seed)
        self.wu = gen_rows("wu", F, D, w_std, dtype, seed)
        self.wd = gen_rows("wd", D, F, w_std, dtype, seed)


class LossInputs:
    """Inputs of one tiled cross-entropy problem, as host arrays.

    h ``[N][D]`` float32 (std 1), w ``[V][D]`` float32 (std ``w_std``),
    targets ``[N]`` int32 uniform in ``[0, V)``, g ``[N]`` float32 per-token
    upstream gradients uniform in ``[0.5, 1.5) / N`` (a mean loss, jittered).
    """

    def __init__(self, n_tokens: int, d_model: int, vocab: int, dtype: str, seed: int = 0, w_std: float = 0.02):
        self.n_tokens, self.d_model, self.vocab, self.dtype, self.seed = n_tokens, d_model, vocab, dtype, seed
        N = n_tokens
        self.h = gen_rows("x", N, d_model, 1.0, dtype, seed)
        self.w = gen_rows("w_lm", vocab, d_model, w_std, dtype, seed)
        rng = _block_rng(seed, TENSOR_IDS["targets"], 0)
        self.targets = rng.integers(0, vocab, N).astype(np.int32)
        rng = _block_rng(seed, TENSOR_IDS["g_loss"], 0)
        self.g = (rng.uniform(0.5, 1.5, N) / N).astype(np.float32)


class BlockInputs:
    """Inputs of one transformer-block problem, as float32 host arrays: the
    attention layer's (``LayerInputs``), the MLP weights (as ``MlpInputs``)
    and the two d_model-long norm weights ``g_attn``, ``g_mlp``
    (``gen_gamma``: ones, or 1 + 0.1 N(0,1))."""

    def __init__(self, n_tokens: int, d_model: int, d_ff: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 dtype: str, seed: int = 0, w_std: float = 0.02, qk_norm: str | None = None,
                 norm: str = "random", with_x: bool = True, with_dy: bool = True):
        lay = LayerInputs(n_tokens, d_model, n_q_heads, n_kv_heads, head_dim, dtype, seed=seed, w_std=w_std,
                          qk_norm=qk_norm, with_x=with_x, with_dy=with_dy)
        self.n_tokens, self.d_model, self.d_ff, self.dtype, self.seed = n_tokens, d_model, d_ff, dtype, seed
        for k in ("x", "dy", "wq", "wk", "wv", "wo", "q_norm", "k_norm"):
            setattr(self, k, getattr(lay, k))
        D, F = d_model, d_ff
        self.g_attn = gen_gamma("attn_norm", D, norm, dtype, seed)
        self.g_mlp = gen_gamma("mlp_norm", D, norm, dtype, seed)
        self.wg = gen_rows("wg", F, D, w_std, dtype, seed)
        self.wu = gen_rows("wu", F, D, w_std, dtype, seed)
        self.wd = gen_rows("wd", D, F, w_std, dtype, seed)
