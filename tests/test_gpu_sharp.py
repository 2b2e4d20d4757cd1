"""GPU parity on sharp-softmax stress inputs: the forward kernel's online
softmax moves its base after the first tile (bf16: in both 32-key halves;
fp32: per tile), which the config-shaped inputs never make it do.

The inputs (``sharp_cases``) have logit std 6 to 28 and key scores that grow
along the sequence; ``test_sharp_replay.py`` shows on the host that each
case makes hundreds of base moves. Here every output and gradient is
compared element by element with the fp64 oracle at the layer's tolerances
(relative L2 1e-5 fp32, 2e-2 bf16). The LSE's max-abs check uses a per-row
bound derived from the io-dtype rounding of q and k (``lse_rounding_bound``)
instead of a fixed absolute tolerance: with logits of std 6 and more the
rounding of bf16 scores alone moves a row's LSE by up to about 0.08 to 0.2,
as a CPU model that rounds only q and k to bf16 shows.

The gradients of the two cases at logit std 18 and 28 (``ILL_CONDITIONED``) are
beyond the fixed bars for any implementation in their precision: the same
backward done plainly in fp32 with io-dtype storage
(``precision_model.plain_grads``) lands 2.9e-2 (bf16) and 1.6e-5 (fp32) from
the oracle in dx. Their gradients are held to the larger of the bar and 2.5
times that plain-arithmetic distance (the GPU measures 1.0x of it in bf16 and
about 1.8x in fp32, where its exp2 approximation and the online softmax's
rescaling add fp32 rounding of their own). The other cases are held to the
bars."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gpu_util import TOL, Case, check_fwd, host, relerr  # noqa: E402
from precision_model import plain_grads  # noqa: E402
from sharp_cases import CASES, ILL_CONDITIONED, inputs, lse_rounding_bound  # noqa: E402
from softmax_replay import replay_layer  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name", list(CASES))
def test_sharp_softmax_parity(name):
    dt, N, D, hq, hkv, d, _, chunks, _ = CASES[name]
    inp = inputs(name)
    case = Case(N, D, hq, hkv, d, dt, inp=inp)
    y_ref, lse_ref, inter = oracle.layer_fwd(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, hq, hkv, d, case.theta, hq,
                                             keep=True)
    moves = replay_layer(inter, hq, hkv, dt)["moves"]
    print(f"case {name}: N={N} D={D} hq={hq} hkv={hkv} d={d} {dt}; replayed base moves {moves}", flush=True)
    bound = lse_rounding_bound(inter, hq, hkv, d, D, dt)
    g_ref = case.oracle_bwd(hq)
    names = ("dx", "dwq", "dwk", "dwv", "dwo")
    tols = {n: TOL[dt] for n in names}
    if name in ILL_CONDITIONED:
        for n, a, r in zip(names, plain_grads(inp, hq, hkv, d, case.theta, dt), g_ref):
            e_plain = relerr(a, r)
            tols[n] = max(TOL[dt], 2.5 * e_plain)
            print(f"  plain {dt} arithmetic: {n} rel {e_plain:.3e} -> bar {tols[n]:.3e}", flush=True)
    for C in chunks:
        y, lse = case.gpu_fwd(C)
        check_fwd(case, C, y, lse, (y_ref, lse_ref), lse_bound=bound)
        g = case.gpu_bwd(C, lse)
        for n, a, r in zip(names, g, g_ref):
            e = relerr(host(a), r)
            print(f"  bwd C={C}: {n} rel {e:.3e} (bar {tols[n]:.3e})", flush=True)
            assert e <= tols[n], (n, e, tols[n])
