"""GPU parity of the checkpointed pre-norm transformer block (through the C
ABI) against the fp64 CPU oracle on the same seeded inputs.

Tolerances: relative L2 <= 1e-5 (fp32 inputs) and <= 2e-2 (bf16 inputs) per
output tensor (y, h, dx and every weight and norm gradient); lse max-abs
<= 1e-4 and 2e-2. Small shapes cover several sequence tiles with a ragged
last one, a tile larger than N, N = 1, GQA, chunk sizes 1-4, q/k norm and
both backward modes (recompute from the block input; h and lse kept by the
forward). At the Llama3-8B shape (d_model 4096, d_ff 14336, 4 q / 1 kv heads
of 128, N = 32768, bf16) y and h are checked at sampled rows, dx at rows of
the last 256 positions for an upstream gradient that is zero before them,
and the weight and norm gradients through homogeneity identities that hold
at any size.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gpu_util import TOL, dev, host, relerr  # noqa: E402
from headwise_chunked_attention_amd import api  # noqa: E402
from headwise_chunked_attention_amd.synth import BlockInputs  # noqa: E402

THETA, EPS, QK_EPS = 5e5, 1e-5, 1e-6
ATOL = {"fp32": 1e-4, "bf16": 2e-2}
# library weight name -> BlockInputs attribute / oracle gradient key
ATTR = {"attn_norm": "g_attn", "wq": "wq", "wk": "wk", "wv": "wv", "wo": "wo", "q_norm": "q_norm",
        "k_norm": "k_norm", "mlp_norm": "g_mlp", "w_gate": "wg", "w_up": "wu", "w_down": "wd"}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _weights(inp, dt):
    return {n: dev(getattr(inp, a), dt) for n, a in ATTR.items() if getattr(inp, a) is not None}


def _oracle_args(inp):
    return (inp.g_attn, inp.wq, inp.wk, inp.wv, inp.wo, inp.g_mlp, inp.wg, inp.wu, inp.wd)


def _run(N, D, F, T, hq, hkv, d, C, dt, keep, qk=None, seed=0):
    print(f"block case N={N} D={D} F={F} tile={T} hq={hq} hkv={hkv} d={d} C={C} {dt} keep={keep} qk={qk}",
          flush=True)
    inp = BlockInputs(N, D, F, hq, hkv, d, dt, seed=seed, qk_norm=qk)
    w = _weights(inp, dt)
    x, dy = dev(inp.x, dt), dev(inp.dy, dt)
    shape = api.block_shape(N, D, F, T, hq, hkv, d, C, THETA, EPS, QK_EPS)
    f32 = torch.float32
    # outputs start as garbage: everything must be overwritten
    h_mid = torch.full((N, D), 9.0, dtype=x.dtype, device="cuda") if keep else None
    lse = torch.full((hq, N), 9.0, dtype=f32, device="cuda") if keep else None
    y, h_mid, lse = api.block_fwd(x, w, shape, y=torch.full_like(x, 7.0), h_mid=h_mid, lse=lse)
    grads = {n: torch.full(t.shape, 3.0, dtype=f32, device="cuda") for n, t in w.items()}
    dx, grads = api.block_bwd(x, w, shape, dy, h_mid=h_mid, lse=lse, dx=torch.full_like(x, 5.0), grads=grads)
    torch.cuda.synchronize()
    y_ref, h_ref, lse_ref = oracle.block_fwd(inp.x, *_oracle_args(inp), hq, hkv, d, THETA, C, inp.q_norm,
                                             inp.k_norm, QK_EPS, EPS)
    g_ref = oracle.block_bwd(inp.x, *_oracle_args(inp), inp.dy, hq, hkv, d, THETA, C, inp.q_norm, inp.k_norm,
                             QK_EPS, EPS)
    errs = {"y": relerr(host(y), y_ref), "dx": relerr(host(dx), g_ref["dx"])}
    if keep:
        errs["h"] = relerr(host(h_mid), h_ref)
        errs["lse_maxabs"] = float(np.max(np.abs(host(lse) - lse_ref)))
    for n, a in ATTR.items():
        if n in grads:
            got, ref = host(grads[n]), g_ref[a]
            # N = 1: one visible key, dS = 0, so dWq and dWk are exactly zero: max-abs
            errs["d" + n] = relerr(got, ref) if np.any(ref) else float(np.max(np.abs(got)))
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= (ATOL[dt] if k == "lse_maxabs" else TOL[dt])}
    assert not bad, bad


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("keep", [False, True])
def test_block_ragged_tiles(dt, keep):
    """N = 300 in MLP tiles of 128 (128, 128, 44 rows), GQA 4/2, chunk 2."""
    _run(300, 256, 384, 128, 4, 2, 64, 2, dt, keep)


def test_block_qk_norm_whole_group_chunk():
    _run(257, 256, 256, 128, 4, 1, 128, 4, "fp32", False, qk="random", seed=1)


def test_block_bf16_tile_larger_than_n_single_head_chunks():
    _run(200, 384, 512, 4096, 4, 4, 64, 1, "bf16", True, seed=2)


@pytest.mark.parametrize("N", [1, 129])
def test_block_edge_lengths(N):
    _run(N, 128, 128, 128, 2, 1, 64, 1, "fp32", N == 1, seed=N)


# ---------------------------------------------------------------------------
# Llama3-8B shape
# ---------------------------------------------------------------------------
BIG = dict(N=32768, D=4096, F=14336, T=4096, hq=4, hkv=1, d=128, C=1)
TAIL = 256


def _dot(a, b):
    return float((a.double() * b.double()).sum().item())


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = BIG
    N, D = c["N"], c["D"]
    print(f"block large N={N} D={D} F={c['F']} tile={c['T']} bf16: inputs", flush=True)
    inp = BlockInputs(N, D, c["F"], c["hq"], c["hkv"], c["d"], "bf16", seed=5)
    w = _weights(inp, "bf16")
    x, dy = dev(inp.x, "bf16"), dev(inp.dy, "bf16")
    shape = api.block_shape(N, D, c["F"], c["T"], c["hq"], c["hkv"], c["d"], c["C"], THETA, EPS, QK_EPS)
    h_mid = torch.empty_like(x)
    lse = torch.empty((c["hq"], N), dtype=torch.float32, device="cuda")
    y, _, _ = api.block_fwd(x, w, shape, h_mid=h_mid, lse=lse)
    print("  forward done; backward from the block input", flush=True)
    dx, g = api.block_bwd(x, w, shape, dy)
    dy_tail = dy.clone()
    dy_tail[: N - TAIL] = 0
    print("  backward with h and lse kept, upstream gradient in the tail only", flush=True)
    dx_tail, _ = api.block_bwd(x, w, shape, dy_tail, h_mid=h_mid, lse=lse)
    torch.cuda.synchronize()
    return dict(inp=inp, w=w, x=x, dy=dy, y=y, h=h_mid, lse=lse, dx=dx, g=g, dx_tail=dx_tail)


def _a_rows(inp):
    return (lambda a, b: oracle.rmsnorm(inp.x[a:b], inp.g_attn, EPS),
            lambda i: oracle.rmsnorm(inp.x[np.asarray(i)], inp.g_attn, EPS))


def test_block_large_sampled_rows_forward(big):
    c, inp = BIG, big["inp"]
    N, T = c["N"], c["T"]
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, T - 1, T, N // 2, N - 1], rng.integers(0, N, 26)]))
    print(f"oracle: {rows.size} sampled rows", flush=True)
    att, lse_ref = oracle.layer_fwd_rows(*_a_rows(inp), N, rows, inp.wq, inp.wk, inp.wv, inp.wo, c["hq"], c["hkv"],
                                         c["d"], THETA)
    h_ref = inp.x[rows] + att
    y_ref = h_ref + oracle.mlp_rows(oracle.rmsnorm(h_ref, inp.g_mlp, EPS), inp.wg, inp.wu, inp.wd)
    idx = torch.from_numpy(rows).to("cuda")
    eh = relerr(host(big["h"].index_select(0, idx)), h_ref)
    ey = relerr(host(big["y"].index_select(0, idx)), y_ref)
    el = float(np.max(np.abs(host(big["lse"].index_select(1, idx)) - lse_ref)))
    print(f"  h {eh:.2e} y {ey:.2e} lse max-abs {el:.2e}", flush=True)
    assert eh <= TOL["bf16"] and ey <= TOL["bf16"] and el <= ATOL["bf16"]


def test_block_large_tail_rows_dx(big):
    c, inp = BIG, big["inp"]
    N = c["N"]
    t0 = N - TAIL
    rng = np.random.default_rng(4)
    rows = np.sort(rng.choice(np.arange(t0, N), size=48, replace=False))
    rows[-1] = N - 1
    win = np.arange(t0, N)
    print(f"oracle: h and dh over the last {TAIL} rows, dx at {rows.size} of them", flush=True)
    att, _ = oracle.layer_fwd_rows(*_a_rows(inp), N, win, inp.wq, inp.wk, inp.wv, inp.wo, c["hq"], c["hkv"], c["d"],
                                   THETA)
    h_w = inp.x[t0:] + att
    dy_w = np.asarray(inp.dy[t0:], dtype=np.float64)
    db_w = oracle.mlp_dx_rows(oracle.rmsnorm(h_w, inp.g_mlp, EPS), dy_w, inp.wg, inp.wu, inp.wd)
    dh_w = dy_w + oracle.rmsnorm_bwd(h_w, inp.g_mlp, EPS, db_w)[0]

    def dh_rows(a, b):
        assert (a, b) == (t0, N)
        return dh_w

    da = oracle.layer_bwd_tail_dx(_a_rows(inp)[0], dh_rows, N, TAIL, rows, inp.wq, inp.wk, inp.wv, inp.wo, c["hq"],
                                  c["hkv"], c["d"], THETA)
    ref = dh_w[rows - t0] + oracle.rmsnorm_bwd(inp.x[rows], inp.g_attn, EPS, da)[0]
    got = host(big["dx_tail"].index_select(0, torch.from_numpy(rows).to("cuda")))
    e = relerr(got, ref)
    print(f"  tail dx rel {e:.3e}", flush=True)
    assert e <= TOL["bf16"]
    # no upstream gradient before the tail: dx there comes only through the
    # attention's keys and values, so it is not zero, but dx is finite everywhere
    assert bool(torch.isfinite(big["dx_tail"].float()).all())


def test_block_large_gradient_identities(big):
    w, g = big["w"], big["g"]
    m = _dot(big["dy"], big["y"].double() - big["h"].double())
    a_d, a_u, a_g = _dot(g["w_down"], w["w_down"]), _dot(g["w_up"], w["w_up"]), _dot(g["w_gate"], w["w_gate"])
    n2 = _dot(g["mlp_norm"], w["mlp_norm"])
    n1 = _dot(g["attn_norm"], w["attn_norm"])
    qkv = _dot(g["wq"], w["wq"]) + _dot(g["wk"], w["wk"]) + _dot(g["wv"], w["wv"])
    print(f"  <dy,y-h>={m:.6e} <dWd,Wd>={a_d:.6e} <dWu,Wu>={a_u:.6e} <dg2,g2>={n2:.6e} "
          f"<dWg,Wg>+<dWu,Wu>={a_g + a_u:.6e} <dg1,g1>={n1:.6e} <dWqkv,Wqkv>={qkv:.6e}", flush=True)
    tol = TOL["bf16"]
    assert abs(a_d - m) <= tol * abs(m)
    assert abs(a_u - m) <= tol * abs(m)
    assert abs(n2 - (a_g + a_u)) <= tol * abs(a_g + a_u)
    assert abs(n1 - qkv) <= tol * max(abs(qkv), 1e-30)
