"""upipe_attn_fwd_noalloc, the forward for callers that cannot allocate: it
must give exactly what upipe_attn_fwd gives (same kernels, the chunk buffers
in the library's static scratch instead of a caller workspace), call after
call, and allocate nothing."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import Case, check_fwd  # noqa: E402
from headwise_chunked_attention_amd import api  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pair(case, C):
    """(y, lse) of upipe_attn_fwd and of upipe_attn_fwd_noalloc for one case;
    the no-allocation call must leave both PyTorch's and the device's free
    memory unchanged."""
    t = case.t
    kw = case.kw(C)
    y_ref, lse_ref = api.attn_fwd(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], **kw)
    y = torch.empty_like(y_ref)
    lse = torch.empty_like(lse_ref)
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated()
    free0, _ = torch.cuda.mem_get_info()
    api.attn_fwd_noalloc(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], y, lse, **kw)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == mem0
    assert free1 == free0, (free0, free1)
    return y_ref, lse_ref, y, lse


def _setup():
    """One tiny call: the library looks up the device's scratch address on its
    first call on a device (the runtime backs the static array then)."""
    case = Case(64, 128, 2, 1, 64, "fp32", seed=50)
    t = case.t
    y = torch.empty_like(t["x"])
    lse = torch.empty((2, 64), dtype=torch.float32, device="cuda")
    api.attn_fwd_noalloc(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], y, lse, **case.kw(1))
    torch.cuda.synchronize()


def test_noalloc_forward_matches_workspace_forward_twice():
    _setup()
    # a larger call, then smaller ones: a call must not depend on what the
    # previous one left in the scratch
    for case, C in ((Case(12000, 1024, 4, 1, 128, "bf16", seed=51), 2),
                    (Case(700, 512, 8, 2, 64, "bf16", theta=1e6, norm="random", seed=52), 4),
                    (Case(300, 256, 4, 2, 64, "fp32", seed=53), 2)):
        print(f"case N={case.N} D={case.D} hq={case.hq} hkv={case.hkv} d={case.d} {case.dtype} C={C}", flush=True)
        y_ref, lse_ref, y, lse = _pair(case, C)
        assert torch.equal(y, y_ref) and torch.equal(lse, lse_ref)
        check_fwd(case, C, y, lse)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    N, D, hq, hkv, d, C = 70000, 128, 4, 1, 128, 1
    need = api.workspace_bytes(N, D, hq, hkv, d, C, False, "bf16", False)
    assert need > api.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((N, D), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((hq * d, D), dtype=torch.bfloat16, device="cuda")
    wkv = torch.zeros((hkv * d, D), dtype=torch.bfloat16, device="cuda")
    wo = torch.zeros((D, hq * d), dtype=torch.bfloat16, device="cuda")
    y = torch.full((N, D), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((hq, N), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(api.UpipeError) as e:
        api.attn_fwd_noalloc(x, w, wkv, wkv, wo, y, lse, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, rope_theta=5e5,
                             chunk_heads=C)
    assert e.value.code == -6 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()) and bool((lse == 7.0).all())  # nothing launched
