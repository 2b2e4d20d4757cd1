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
