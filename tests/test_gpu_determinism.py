"""Reproducibility and memory discipline of the attention op on the GPU.

* upipe_attn_bwd_deterministic gives bit-identical gradients from run to run
  (and on another stream), and agrees with the oracle at the layer's
  tolerance; the default backward agrees with it to rounding.
* Neither entry point writes outside its workspace or its outputs: every
  buffer is handed over as a view into a larger allocation whose guard bands
  hold a known byte pattern, and the bands are intact after the calls.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import Case, check_bwd  # noqa: E402
from headwise_chunked_attention_amd import api  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bwd(case, C, lse, det, stream=None):
    t = case.t
    g = api.attn_bwd(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], t["dy"], lse, stream=stream, deterministic=det,
                     **case.kw(C))
    torch.cuda.synchronize()
    return g


# (case args, chunk): q/k norm (dgamma sums), a short sequence whose key blocks
# the default backward splits by head, GQA groups spanning chunks, fp32
DET_CASES = {
    "bf16-qwen-norm-c2": (dict(N=1536, D=640, hq=8, hkv=1, d=128, dtype="bf16", theta=1e6, norm="random", seed=41), 2),
    "bf16-llama-c1": (dict(N=2304, D=1024, hq=4, hkv=1, d=128, dtype="bf16", seed=42), 1),
    "bf16-gqa2-c1": (dict(N=900, D=256, hq=4, hkv=2, d=64, dtype="bf16", seed=43), 1),
    "fp32-tiny-c2": (dict(N=2048, D=512, hq=8, hkv=2, d=64, dtype="fp32", seed=44), 2),
}


@pytest.mark.parametrize("name", list(DET_CASES))
def test_deterministic_backward_is_bitwise_repeatable(name):
    args, C = DET_CASES[name]
    print(f"case {name}: {args} C={C}", flush=True)
    case = Case(args.pop("N"), args.pop("D"), args.pop("hq"), args.pop("hkv"), args.pop("d"), args.pop("dtype"),
                **args)
    y, lse = case.gpu_fwd(C)
    g1 = _bwd(case, C, lse, True)
    g2 = _bwd(case, C, lse, True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g3 = _bwd(case, C, lse, True, stream=side)
    for a, b, c in zip(g1, g2, g3):
        if a is None:
            continue
        assert torch.equal(a, b) and torch.equal(a, c)
    # the deterministic gradients are the layer's gradients
    check_bwd(case, C, g1)
    # and the default backward's differ from them by rounding only (within the bars)
    g0 = _bwd(case, C, lse, False)
    for a, b in zip(g0, g1):
        if a is None:
            continue
        e = float((a.double() - b.double()).norm() / b.double().norm())
        assert e <= (1e-5 if case.dtype == "fp32" else 1e-2), e


GUARD = 1 << 20  # bytes on each side (a multiple of 256 keeps the views aligned)
PATTERN = 0xA5


def _guarded(nbytes, dev="cuda"):
    buf = torch.full((GUARD + nbytes + GUARD,), PATTERN, dtype=torch.uint8, device=dev)
    return buf, buf[GUARD:GUARD + nbytes]


def _guarded_tensor(shape, dtype):
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    buf, view = _guarded(n)
    return buf, view.view(dtype).view(*shape)


def _intact(buf):
    g = torch.cat([buf[:GUARD], buf[-GUARD:]])
    return bool((g == PATTERN).all())


@pytest.mark.parametrize("norm", [None, "random"])
def test_nothing_written_outside_workspace_and_outputs(norm):
    N, D, hq, hkv, d, C = 1000, 512, 8, 2, 128, 4
    case = Case(N, D, hq, hkv, d, "bf16", theta=1e6 if norm else 5e5, norm=norm, seed=45)
    t = case.t
    kw = case.kw(C)
    bufs = []
    ws_f = api.workspace_bytes(N, D, hq, hkv, d, C, norm is not None, "bf16", False)
    ws_b = api.workspace_bytes(N, D, hq, hkv, d, C, norm is not None, "bf16", True)
    b, ws = _guarded(ws_f)
    bufs.append(b)
    b, y = _guarded_tensor((N, D), torch.bfloat16)
    bufs.append(b)
    b, lse = _guarded_tensor((hq, N), torch.float32)
    bufs.append(b)
    api.attn_fwd(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], y=y, lse=lse, workspace=ws, **kw)
    torch.cuda.synchronize()
    f32 = torch.float32
    outs = []
    for shape, dt in (((N, D), torch.bfloat16), (t["wq"].shape, f32), (t["wk"].shape, f32), (t["wv"].shape, f32),
                      (t["wo"].shape, f32)):
        b, o = _guarded_tensor(tuple(shape), dt)
        bufs.append(b)
        outs.append(o)
    for _ in range(2 if norm else 0):
        b, o = _guarded_tensor((d,), f32)
        bufs.append(b)
        outs.append(o)
    outs += [None] * (7 - len(outs))
    for det in (False, True):
        b, wsb = _guarded(ws_b)
        bufs.append(b)
        api.attn_bwd(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], t["dy"], lse, out=tuple(outs), workspace=wsb,
                     deterministic=det, **kw)
        torch.cuda.synchronize()
    assert all(_intact(b) for b in bufs)
    # and the results are the layer's
    check_bwd(case, C, tuple(outs))


def test_deterministic_split_partials_at_32k():
    """Llama3-8B layout at N = 32768 with chunks of 4 heads: the deterministic
    backward's weight gradients then run split over the tokens with per-split
    partial tiles (the 256x256 weight-gradient kernel's partial path) and are
    added in split order. Bitwise repeatable, and within the bf16 bar of the
    default backward (whose splits add with atomics)."""
    case = Case(32768, 4096, 4, 1, 128, "bf16", seed=47)
    C = 4
    print(f"case llama-32k: N=32768 D=4096 hq=4 hkv=1 d=128 bf16 C={C}", flush=True)
    y, lse = case.gpu_fwd(C)
    g1 = _bwd(case, C, lse, True)
    g2 = _bwd(case, C, lse, True)
    g0 = _bwd(case, C, lse, False)
    for a, b, c in zip(g1, g2, g0):
        if a is None:
            continue
        assert torch.equal(a, b)
        e = float((c.double() - a.double()).norm() / a.double().norm())
        assert e <= 1e-2, e
