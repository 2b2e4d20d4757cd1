"""GPU parity of the sequence-tiled gated-SiLU MLP (through the C ABI) against
the fp64 CPU oracle on the same seeded inputs: relative L2 <= 1e-5 for fp32
inputs and <= 2e-2 for bf16 inputs, per output tensor.

Small shapes cover several tiles, a ragged last tile, a tile larger than the
sequence, N = 1 and both dtypes. At the Llama3-8B MLP shape (d_model 4096,
d_ff 14336) the MLP is row-wise, so y and dx are checked exactly at sampled
rows, and the weight gradients through the identities
<dWd, Wd> = <dWu, Wu> = <dy, y>, which hold at any size.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gpu_util import TOL, dev, host, relerr  # noqa: E402
from headwise_chunked_attention_amd import api  # noqa: E402
from headwise_chunked_attention_amd.synth import MlpInputs  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _upload(inp, dt):
    return {k: dev(getattr(inp, k), dt) for k in ("x", "dy", "wg", "wu", "wd")}


def _run(N, D, F, T, dt, seed=0):
    print(f"mlp case N={N} D={D} F={F} tile={T} {dt}", flush=True)
    inp = MlpInputs(N, D, F, dt, seed=seed)
    t = _upload(inp, dt)
    y = api.mlp_fwd(t["x"], t["wg"], t["wu"], t["wd"], tile_tokens=T)
    # gradients are overwritten, whatever the buffers held
    f32 = torch.float32
    out = (torch.full((N, D), 7.0, dtype=t["x"].dtype, device="cuda"),
           torch.full((F, D), 3.0, dtype=f32, device="cuda"), torch.full((F, D), 3.0, dtype=f32, device="cuda"),
           torch.full((D, F), 3.0, dtype=f32, device="cuda"))
    g = api.mlp_bwd(t["x"], t["wg"], t["wu"], t["wd"], t["dy"], tile_tokens=T, out=out)
    torch.cuda.synchronize()
    y_ref = oracle.mlp_fwd(inp.x, inp.wg, inp.wu, inp.wd)
    g_ref = oracle.mlp_bwd(inp.x, inp.wg, inp.wu, inp.wd, inp.dy)
    errs = {"y": relerr(host(y), y_ref)}
    for name, a, b in zip(("dx", "dw_gate", "dw_up", "dw_down"), g, g_ref):
        errs[name] = relerr(host(a), b)
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[dt]}
    assert not bad, bad


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_mlp_ragged_tiles(dt):
    """N = 300 in tiles of 128 (128, 128, 44 rows), d_model 256, d_ff 384."""
    _run(300, 256, 384, 128, dt)


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_mlp_one_tile_larger_than_n(dt):
    _run(200, 384, 256, 4096, dt, seed=1)


@pytest.mark.parametrize("N", [1, 129])
def test_mlp_edge_lengths(N):
    _run(N, 128, 128, 128, "fp32", seed=N)


def test_mlp_bf16_wide_multi_tile():
    """d_model 1024, d_ff 2816 (Llama-like ratio), 5 tiles of 256 rows with a ragged last one."""
    _run(1100, 1024, 2816, 256, "bf16", seed=2)


@pytest.mark.parametrize("N,T", [(16384, 4096), (4480, 8192)])
def test_mlp_llama8b_shape_sampled_rows_and_identities(N, T):
    """Llama3-8B MLP (d_model 4096, d_ff 14336), bf16: N = 16384 in tiles of 4096, and
    N = 4480 in one tile, whose last 256-row GEMM tile holds 128 rows and whose weight
    gradients sum over 70 (not a multiple of 4) k tiles of 64 tokens."""
    D, F = 4096, 14336
    print(f"mlp large N={N} D={D} F={F} tile={T} bf16", flush=True)
    inp = MlpInputs(N, D, F, "bf16", seed=3)
    t = _upload(inp, "bf16")
    y = api.mlp_fwd(t["x"], t["wg"], t["wu"], t["wd"], tile_tokens=T)
    dx, dwg, dwu, dwd = api.mlp_bwd(t["x"], t["wg"], t["wu"], t["wd"], t["dy"], tile_tokens=T)
    torch.cuda.synchronize()

    def dot(a, b):
        return float((a.double() * b.double()).sum().item())

    ref = dot(t["dy"], y)
    a_d, a_u = dot(dwd, t["wd"]), dot(dwu, t["wu"])
    print(f"  <dy,y>={ref:.6e} <dWd,Wd>={a_d:.6e} <dWu,Wu>={a_u:.6e}", flush=True)
    assert abs(a_d - ref) <= TOL["bf16"] * abs(ref)
    assert abs(a_u - ref) <= TOL["bf16"] * abs(ref)

    rng = np.random.default_rng(11)
    edge = [0, 1, N - 129, N - 128, N - 1] + ([T - 1, T] if T < N else [])
    rows = np.unique(np.concatenate([edge, rng.integers(0, N, 27)]))
    idx = torch.from_numpy(rows).to("cuda")
    y_rows = host(y.index_select(0, idx))
    dx_rows = host(dx.index_select(0, idx))
    y_ref = oracle.mlp_rows(inp.x[rows], inp.wg, inp.wu, inp.wd)
    dx_ref = oracle.mlp_dx_rows(inp.x[rows], inp.dy[rows], inp.wg, inp.wu, inp.wd)
    ey, edx = relerr(y_rows, y_ref), relerr(dx_rows, dx_ref)
    print(f"  sampled rows: y {ey:.2e} dx {edx:.2e}", flush=True)
    assert ey <= TOL["bf16"] and edx <= TOL["bf16"]
