"""CPU replay of the attention forward kernel's online-softmax base rule.

The training forward (``attn_fwd_kernel``, mode 0) keeps one softmax base per
query and moves it only when it must; the parity tests need inputs that make
it move after the first tile, in both 32-key halves of a tile, so this module
replays the rule on the host, wave by wave, from fp64 scores:

* A wave owns 32 consecutive queries of one head and walks the 64-key tiles
  ``k0 = 0, 64, ...`` up to its last query; keys after a query are masked.
* bf16: each tile is taken as two halves of 32 keys. Lane (query, h) holds 16
  keys of a half (``8*(e//4) + 4*h + e%4``, e = 0..15). The first half sets
  the base to its row max. After that the base moves when some lane's sum of
  ``exp2(S - base)`` exceeds 2^16 (S in log2 units): then every query's base
  becomes the max of its old base and the half's row max.
* fp32: per tile, the base of a query moves to the tile's row max when that
  exceeds the base by more than 8 (log2 units); the first tile sets it.

The kernel decides from bf16 scores and bf16-rounded probabilities, so a
decision is only certain when the fp64 replay clears the threshold by a
margin: a factor 2 on the lane sum (bf16), 0.01 on the score (fp32), far
beyond the rounding of either. ``replay`` counts base moves after the first
whose decision, and every decision of its wave before it, is certain; those
moves happen on the GPU exactly as replayed.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)
P_LIMIT = 65536.0
FP32_STEP = 8.0
ROWS_W = 32
TILE = 64


def scores_log2(q, k):
    """Causal scores of one head in log2 units: ``q k^T / sqrt(d) * log2(e)``, keys after a query at -inf."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    s = (q @ k.T) * (LOG2E / math.sqrt(q.shape[1]))
    n = q.shape[0]
    s[np.triu_indices(n, 1, k.shape[0])] = -np.inf
    return s


def _lane_keys(h):
    return np.array([8 * (e // 4) + 4 * h + e % 4 for e in range(16)])


LANE_KEYS = (_lane_keys(0), _lane_keys(1))


def replay(s, dtype):
    """Replay the base rule over the scores ``s [N][N]`` (log2 units) of one head.

    Returns a dict: ``moves`` (certain base moves after the first, by key half
    for bf16 as ``{0: n, 1: n}``, for fp32 as ``{"tile": n}``), ``waves``
    (waves with at least one certain move), ``uncertain`` (decisions within
    the margin) and ``max_ratio`` (largest lane sum over 2^16, bf16).
    """
    n = s.shape[0]
    moves = {0: 0, 1: 0} if dtype == "bf16" else {"tile": 0}
    waves_moved = 0
    uncertain = 0
    max_ratio = 0.0
    for q0 in range(0, n, ROWS_W):
        q1 = min(n, q0 + ROWS_W)
        rows = s[q0:q1]
        base = np.full(q1 - q0, -np.inf)
        certain = True
        moved = False
        for k0 in range(0, q0 + ROWS_W, TILE):
            if dtype == "bf16":
                for kt in range(2):
                    a = k0 + 32 * kt
                    half = np.full((q1 - q0, 32), -np.inf)
                    b = min(n, a + 32)
                    if b > a:
                        half[:, :b - a] = rows[:, a:b]
                    hmax = half.max(axis=1)
                    if not np.isfinite(base).all():
                        base = np.maximum(base, hmax)  # the first half of the first tile
                        continue
                    with np.errstate(over="ignore"):
                        e = np.exp2(half - base[:, None])
                    ratio = max(float(e[:, LANE_KEYS[h]].sum(axis=1).max()) for h in (0, 1)) / P_LIMIT
                    max_ratio = max(max_ratio, ratio)
                    if 0.5 < ratio < 2.0:
                        uncertain += 1
                        certain = False
                    if ratio > 1.0:
                        if certain:
                            moves[kt] += 1
                            moved = True
                        base = np.maximum(base, hmax)
            else:
                b = min(n, k0 + TILE)
                tmax = rows[:, k0:b].max(axis=1)
                if not np.isfinite(base).all():
                    base = tmax
                    continue
                gap = tmax - base - FP32_STEP
                if np.any(np.abs(gap) < 0.01):
                    uncertain += 1
                    certain = False
                need = gap > 0
                if need.any():
                    if certain:
                        moves["tile"] += 1
                        moved = True
                    base = np.where(need, tmax, base)
        waves_moved += moved
    return {"moves": moves, "waves": waves_moved, "uncertain": uncertain, "max_ratio": max_ratio}


def replay_layer(inter, n_q_heads, n_kv_heads, dtype):
    """``replay`` over every q head, from the oracle's per-head rotated q and k
    (``oracle.layer_fwd(..., keep=True)``'s intermediates); per-head results summed."""
    g = n_q_heads // n_kv_heads
    tot = None
    for h in range(n_q_heads):
        r = replay(scores_log2(inter["q"][h], inter["k"][h // g]), dtype)
        if tot is None:
            tot = r
        else:
            for key in r["moves"]:
                tot["moves"][key] += r["moves"][key]
            tot["waves"] += r["waves"]
            tot["uncertain"] += r["uncertain"]
            tot["max_ratio"] = max(tot["max_ratio"], r["max_ratio"])
    return tot
