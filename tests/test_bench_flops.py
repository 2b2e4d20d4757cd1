"""The flop counts bench.py divides by (CPU only).

``model_flops`` is the algorithmic work of one forward plus backward of the
layer: 14 d flops per visible (query, key) pair and q head (forward S and
P V, backward S, dP, dV, dK, dQ at 2 d each), and the four projections
(forward x Wq^T, x Wk^T, x Wv^T, O Wo^T; the backward twice each, for the
input and the weight gradient). ``hardware_flops`` adds what the backward
recomputes: O from the saved LSE (S and P V) and the Q, K, V projections.
Both are checked against a count made by walking the pairs and products one
by one, and the workload table against the shapes of the configurations the
bench and the tests use.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _gemm(m, n, k):
    return 2 * m * n * k


def _counted(N, D, hq, hkv, d, recompute):
    pairs = sum(1 for i in range(N) for j in range(N) if j <= i)
    per_pair = 2 * d * 2 + 2 * d * 5  # forward S, P V; backward S, dP, dV, dK, dQ
    if recompute:
        per_pair += 2 * d * 2  # the backward's S and P V for O
    attn = per_pair * pairs * hq
    fwd_proj = (_gemm(N, hq * d, D) + _gemm(N, hkv * d, D) + _gemm(N, hkv * d, D)
                + _gemm(N, D, hq * d))
    proj = fwd_proj + 2 * fwd_proj  # backward: input and weight gradient of each
    if recompute:
        proj += _gemm(N, hq * d, D) + 2 * _gemm(N, hkv * d, D)
    return attn + proj


@pytest.mark.parametrize("N,D,hq,hkv,d", [(1, 8, 1, 1, 4), (7, 16, 4, 2, 8), (33, 24, 8, 1, 16)])
def test_model_flops_match_a_direct_count(N, D, hq, hkv, d):
    assert bench.model_flops(N, D, hq, hkv, d) == _counted(N, D, hq, hkv, d, recompute=False)


@pytest.mark.parametrize("N,D,hq,hkv,d", [(1, 8, 1, 1, 4), (7, 16, 4, 2, 8), (33, 24, 8, 1, 16)])
def test_hardware_flops_match_a_direct_count(N, D, hq, hkv, d):
    assert bench.hardware_flops(N, D, hq, hkv, d) == _counted(N, D, hq, hkv, d, recompute=True)


@pytest.mark.parametrize("N,D,hq,hkv,d,total", [
    (2048, 512, 8, 2, 64, 2.31e10),          # tiny fp32 configuration
    (131072, 4096, 4, 1, 128, 6.57e13),      # Llama3-8B share, 131072 tokens
    (1048576, 4096, 4, 1, 128, 3.97e15),     # Llama3-8B share, 1048576 tokens
    (524288, 5120, 8, 1, 128, 2.01e15),      # Qwen3-32B-shaped share
    (5242880, 4096, 4, 1, 128, 9.87e16),     # Llama3-8B share, 5242880 tokens
])
def test_model_flops_of_the_configurations(N, D, hq, hkv, d, total):
    assert bench.model_flops(N, D, hq, hkv, d) == pytest.approx(total, rel=5e-3)


def test_workload_table_shapes():
    llama = dict(d_model=4096, n_q_heads=4, n_kv_heads=1, head_dim=128, rope_theta=5e5)
    for name, n in (("llama3-8b-ulysses-share-131k", 131072), ("llama3-8b-ulysses-share-1m", 1048576),
                    ("llama3-8b-ulysses-share-5m", 5242880)):
        w = bench.WORKLOADS[name]
        assert w["n_tokens"] == n and {k: w[k] for k in llama} == llama and not w.get("qk_norm", False)
    q = bench.WORKLOADS["qwen3-32b-ulysses-share-512k"]
    assert (q["n_tokens"], q["d_model"], q["n_q_heads"], q["n_kv_heads"], q["head_dim"], q["rope_theta"]) == \
        (524288, 5120, 8, 1, 128, 1e6)
    assert q["qk_norm"] and tuple(q["chunks"]) == (1, 2, 4, 8)
    assert bench.WORKLOADS["llama3-8b-ulysses-share-5m"]["chunks"] == (1,)
    assert bench.HEADLINE == "llama3-8b-ulysses-share-1m"


def test_dominant_kernel_flops_per_launch():
    """The dK/dV kernel's algorithmic work per launch (one q head): S, dP, dV
    and dK, 8 d flops per visible pair; the figure the roofline divides."""
    N, d = 1048576, 128
    assert 8 * d * N * (N + 1) // 2 == pytest.approx(5.6295e14, rel=1e-4)
