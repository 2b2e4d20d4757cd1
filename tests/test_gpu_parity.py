"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle,
element by element on the same seeded inputs. Tolerances are the ones the
layer's precision fixes: relative L2 <= 1e-5 for fp32 inputs and <= 2e-2 for
bf16 inputs, per output tensor; LSE also max-abs."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import Case, check_bwd, check_fwd  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(case, C, bwd=True, ref_fwd=None, ref_bwd=None):
    print(f"case N={case.N} D={case.D} hq={case.hq} hkv={case.hkv} d={case.d} {case.dtype} "
          f"norm={case.norm} C={C}", flush=True)
    y, lse = case.gpu_fwd(C)
    check_fwd(case, C, y, lse, ref_fwd)
    if bwd:
        check_bwd(case, C, case.gpu_bwd(C, lse), ref_bwd)


def test_tiny_fp32_config():
    """N=2048, d_model=512, 8 q / 2 kv heads, head_dim 64, theta 5e5, chunk_heads 2, fp32."""
    _run(Case(2048, 512, 8, 2, 64, "fp32"), 2)


@pytest.mark.parametrize("C", [1, 4, 8])
def test_tiny_fp32_other_chunks(C):
    _run(Case(2048, 512, 8, 2, 64, "fp32"), C)


@pytest.mark.parametrize("N", [1, 7, 300, 1000])
@pytest.mark.parametrize("d", [64, 128])
def test_fp32_ragged(N, d):
    _run(Case(N, 256, 4, 1, d, "fp32", seed=N), 2)


@pytest.mark.parametrize("N", [1, 7, 300, 1000])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_ragged(N, d):
    """Sequences shorter than one key block and ragged tails in bf16: with
    head_dim 128 the dK/dV kernel's 256-key block then holds mostly padding
    rows, and its last query step mostly rows past the end."""
    _run(Case(N, 256, 4, 1, d, "bf16", seed=100 + N), 2)


def test_fp32_qk_norm_random_gamma():
    _run(Case(700, 256, 8, 1, 128, "fp32", theta=1e6, norm="random", seed=3), 2)


def test_fp32_qk_norm_c8():
    _run(Case(513, 384, 8, 2, 64, "fp32", theta=1e6, norm="random", seed=4), 8)


def test_bf16_tiny_layout():
    _run(Case(2048, 512, 8, 2, 64, "bf16"), 2)


@pytest.mark.parametrize("C", [1, 2, 4])
def test_bf16_llama_share_reduced_n(C):
    """Llama3-8B share layout (d_model 4096, 4 q / 1 kv, head_dim 128) at N=2304."""
    _run(Case(2304, 4096, 4, 1, 128, "bf16"), C)


@pytest.mark.parametrize("C", [1, 8])
def test_bf16_qwen_share_reduced_n(C):
    """Qwen3-32B-shaped share (d_model 5120, 8 q / 1 kv, q/k RMSNorm, theta 1e6) at N=1536."""
    _run(Case(1536, 5120, 8, 1, 128, "bf16", theta=1e6, norm="random", seed=2), C)


@pytest.mark.parametrize("C", [1, 2])
def test_fp32_mha_group_of_one(C):
    """Multi-head attention (as many kv heads as q heads: kv groups of one head),
    so every chunk projects its own K/V and C kv heads sit side by side."""
    _run(Case(600, 256, 4, 4, 64, "fp32", seed=11), C)


@pytest.mark.parametrize("C", [1, 4])
def test_bf16_group_of_two(C):
    """kv groups of two q heads at head_dim 128: at C=1 a group spans two chunks
    (K/V and their gradients stay resident between them); at C=4 one chunk holds
    two groups. N not a multiple of any tile."""
    _run(Case(900, 256, 4, 2, 128, "bf16", seed=12), C)


def test_side_stream_with_internal_workspace():
    """fwd+bwd enqueued on a second stream, letting the binding allocate the
    workspace and outputs, while the default stream allocates and writes
    memory right after each call: the results must equal those of the same
    calls on the default stream (the forward bit for bit; the binding allocates on the
    stream it launches on, so its freed workspace cannot be reused under the
    side stream's kernels)."""
    case = Case(1500, 512, 4, 1, 128, "bf16", seed=31)
    t = case.t
    kw = case.kw(1)
    y0, lse0 = api_fwd(t, kw)
    g0 = api_bwd(t, kw, lse0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    y1, lse1 = api_fwd(t, kw, stream=side)
    junk = [torch.full((1 << 24,), float(i), device="cuda") for i in range(8)]  # default stream, may reuse freed blocks
    g1 = api_bwd(t, kw, lse1, stream=side)
    junk += [torch.full((1 << 24,), -float(i), device="cuda") for i in range(8)]
    torch.cuda.synchronize()
    del junk
    assert torch.equal(y0, y1) and torch.equal(lse0, lse1)
    for a, b in zip(g0[:5], g1[:5]):
        # gradients: split sums are added atomically, in no fixed order, so
        # only the forward is compared bit for bit
        e = float((a.double() - b.double()).norm() / a.double().norm())
        assert e <= 1e-3, e


def api_fwd(t, kw, stream=None):
    from headwise_chunked_attention_amd import api
    return api.attn_fwd(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], stream=stream, **kw)


def api_bwd(t, kw, lse, stream=None):
    from headwise_chunked_attention_amd import api
    return api.attn_bwd(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], t["dy"], lse, stream=stream, **kw)
