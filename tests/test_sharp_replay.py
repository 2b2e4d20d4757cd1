"""The sharp-softmax stress inputs make the forward kernel move its softmax
base after the first tile, in both 32-key halves (bf16) and per tile (fp32).

Checked by replaying the kernel's rule on the host (``softmax_replay``) from
the oracle's fp64 scores; only decisions far from the threshold are counted,
so the GPU takes the same ones. The GPU parity of these inputs is in
``test_gpu_sharp.py``."""
import pytest

import oracle
from sharp_cases import CASES, inputs, logit_std
from softmax_replay import replay_layer


@pytest.mark.parametrize("name", list(CASES))
def test_stress_inputs_move_the_base(name):
    dt, N, D, hq, hkv, d, _, _, _ = CASES[name]
    inp = inputs(name)
    _, _, inter = oracle.layer_fwd(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, hq, hkv, d, 5e5, hq, keep=True)
    r = replay_layer(inter, hq, hkv, dt)
    print(name, f"logit std {logit_std(inter, d):.1f}", r)
    assert logit_std(inter, d) > 5.0
    if dt == "bf16":
        # certain moves in the first half (which also corrects the second
        # half's scores) and in the second half
        assert r["moves"][0] >= 100 and r["moves"][1] >= 100, r
        assert r["max_ratio"] > 1e6
    else:
        assert r["moves"]["tile"] >= 1000, r
    assert r["waves"] >= 100


@pytest.mark.parametrize("name", [n for n in CASES if CASES[n][0] == "bf16"])
def test_lse_bound_covers_bf16_stored_scores(name):
    """The per-row LSE bound of the stress test holds for the plainest model of
    the kernel's arithmetic: scores from q (times log2(e)/sqrt(d)) and k
    rounded to bf16, everything else exact. The bound must hold with room,
    and must not be so loose that it says nothing (the rounding reaches at
    least a twentieth of it somewhere)."""
    import math

    import numpy as np

    from headwise_chunked_attention_amd.synth import round_to_bf16
    from sharp_cases import lse_rounding_bound

    dt, N, D, hq, hkv, d, _, _, _ = CASES[name]
    inp = inputs(name)
    _, lse, inter = oracle.layer_fwd(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, hq, hkv, d, 5e5, hq, keep=True)
    bound = lse_rounding_bound(inter, hq, hkv, d, D, dt)
    g = hq // hkv
    worst = 0.0
    for h in range(hq):
        bq = round_to_bf16(inter["q"][h] * (1 / math.log(2) / math.sqrt(d))).astype(np.float64)
        bk = round_to_bf16(inter["k"][h // g]).astype(np.float64)
        s = (bq @ bk.T) * math.log(2)
        s[np.triu_indices(N, 1)] = -np.inf
        m = s.max(axis=1)
        lse_b = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
        worst = max(worst, float(np.max(np.abs(lse_b - lse[h]) / bound[h])))
    print(name, f"max |dLSE| / bound = {worst:.3f}")
    assert 0.05 < worst < 0.5


@pytest.mark.parametrize("name", list(CASES))
def test_ill_conditioned_cases_are_beyond_the_bar_in_plain_arithmetic(name):
    """The cases whose GPU gradients get a derived bar are exactly those where
    the textbook backward in plain fp32 arithmetic with io-dtype storage
    already misses the layer's bar in dx; the others meet it with room."""
    import numpy as np

    from precision_model import plain_grads
    from sharp_cases import ILL_CONDITIONED

    dt, N, D, hq, hkv, d, _, _, _ = CASES[name]
    inp = inputs(name)
    ref = oracle.layer_bwd(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, inp.dy, hq, hkv, d, 5e5, hq)[0]
    dx = plain_grads(inp, hq, hkv, d, 5e5, dt)[0]
    e = float(np.linalg.norm(dx - ref) / np.linalg.norm(ref))
    bar = 2e-2 if dt == "bf16" else 1e-5
    print(name, f"plain {dt} arithmetic: dx rel {e:.3e} (bar {bar:.0e})")
    if name in ILL_CONDITIONED:
        assert e > bar
    else:
        assert e < 0.6 * bar
