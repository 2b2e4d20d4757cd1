"""GPU parity at full size, through the same C ABI and launch configuration
the bench uses, for the one-GPU Ulysses shares of the workloads:
  * Llama3-8B share, N = 131072 (the bench workload) and N = 1048576:
    d_model 4096, 4 q / 1 kv heads, head_dim 128, bf16, RoPE theta 5e5;
  * Qwen3-32B-shaped share, N = 524288: d_model 5120, 8 q / 1 kv heads,
    head_dim 128, q/k RMSNorm, RoPE theta 1e6, bf16.

The oracle cannot afford the whole layer at these N, so it checks what it can
compute exactly one row at a time:
  * y and LSE at 256 sampled query rows (corners, tile boundaries, seeded
    uniform draws);
  * dx at 64 rows of the last 512 positions (their dk/dv only involve queries
    inside that window).
The weight gradients need every row; they are checked with identities that
hold exactly at any size:
  * y is linear in Wo and in Wv, so <dWo, Wo> = <dWv, Wv> = <dY, y>;
  * without q/k norm, scaling Wq by a and Wk by 1/a leaves every score
    unchanged (RoPE is linear), so <dWq, Wq> = <dWk, Wk>;
  * with q/k RMSNorm, y does not depend on the scale of Wq (or Wk), so
    <dWq, Wq> = 0 up to the norm's epsilon, and scaling gamma_q by a and
    gamma_k by 1/a leaves the scores unchanged, so <dgq, gq> = <dgk, gk>;
and with chunk invariance (every chunk size gives the same outputs up to bf16
rounding) and causality (rows before a change in x keep y bit for bit).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from headwise_chunked_attention_amd import api  # noqa: E402
from headwise_chunked_attention_amd.synth import LayerInputs  # noqa: E402

TOL = 2e-2

CONFIGS = {
    "llama3-8b-share-131k": dict(N=131072, D=4096, hq=4, hkv=1, d=128, theta=5e5, norm=None, chunks=(1, 2, 4)),
    "llama3-8b-share-1m": dict(N=1048576, D=4096, hq=4, hkv=1, d=128, theta=5e5, norm=None, chunks=(1, 2, 4)),
    "qwen3-32b-share-512k": dict(N=524288, D=5120, hq=8, hkv=1, d=128, theta=1e6, norm="random",
                                 chunks=(1, 2, 4, 8)),
}


def _sample_rows(n, count=256, seed=0):
    fixed = {0, 1, n - 1, 63, 64, 127, 128, 255, 256, n // 2 - 1, n // 2}
    rng = np.random.default_rng(seed)
    rows = set(fixed)
    while len(rows) < count:
        rows.add(int(rng.integers(0, n)))
    return np.array(sorted(rows), dtype=np.int64)


def _relerr(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _dot(a, b):
    return float((a.double() * b.double()).sum().item())


@pytest.fixture(scope="module", params=list(CONFIGS))
def share(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = dict(CONFIGS[request.param])
    c["name"] = request.param
    print(f"[{request.param}] generating inputs", flush=True)
    inp = LayerInputs(c["N"], c["D"], c["hq"], c["hkv"], c["d"], "bf16", seed=0, qk_norm=c["norm"])
    t = {k: torch.from_numpy(getattr(inp, k)).to("cuda").to(torch.bfloat16)
         for k in ("x", "dy", "wq", "wk", "wv", "wo")}
    for k in ("q_norm", "k_norm"):
        t[k] = None if getattr(inp, k) is None else torch.from_numpy(getattr(inp, k)).to("cuda").to(torch.bfloat16)
    torch.cuda.synchronize()
    yield c, inp, t
    del t
    torch.cuda.empty_cache()


def _kw(c, C):
    return dict(n_q_heads=c["hq"], n_kv_heads=c["hkv"], head_dim=c["d"], rope_theta=c["theta"], chunk_heads=C)


@pytest.fixture(scope="module")
def runs(share):
    c, _, t = share
    out = {}
    for C in c["chunks"]:
        print(f"[{c['name']}] N={c['N']} C={C}: fwd+bwd", flush=True)
        y, lse = api.attn_fwd(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], q_norm=t["q_norm"], k_norm=t["k_norm"],
                              **_kw(c, C))
        g = api.attn_bwd(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], t["dy"], lse, q_norm=t["q_norm"],
                         k_norm=t["k_norm"], **_kw(c, C))
        torch.cuda.synchronize()
        out[C] = (y, lse, g)
    yield out
    del out
    torch.cuda.empty_cache()


def test_sampled_rows_forward(share, runs):
    c, inp, _ = share
    rows = _sample_rows(c["N"])
    print(f"[{c['name']}] oracle: y, lse at {rows.size} rows", flush=True)
    y_ref, lse_ref = oracle.layer_fwd_rows(lambda a, b: inp.x[a:b], lambda i: inp.x[i], c["N"], rows, inp.wq,
                                           inp.wk, inp.wv, inp.wo, c["hq"], c["hkv"], c["d"], c["theta"],
                                           inp.q_norm, inp.k_norm)
    idx = torch.from_numpy(rows).to("cuda")
    for C, (y, lse, _) in runs.items():
        yg = y.index_select(0, idx).float().cpu().numpy()
        lg = lse.index_select(1, idx).float().cpu().numpy()
        ey, el = _relerr(yg, y_ref), _relerr(lg, lse_ref)
        ml = float(np.max(np.abs(lg - lse_ref)))
        print(f"  C={C}: y rel {ey:.3e}  lse rel {el:.3e} max {ml:.3e}", flush=True)
        assert ey <= TOL and el <= TOL and ml <= TOL, (C, ey, el, ml)


def test_tail_rows_dx(share, runs):
    c, inp, _ = share
    N, tail = c["N"], 512
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(np.arange(N - tail, N), size=64, replace=False))
    rows[-1] = N - 1
    print(f"[{c['name']}] oracle: dx at {rows.size} tail rows", flush=True)
    ref = oracle.layer_bwd_tail_dx(lambda a, b: inp.x[a:b], lambda a, b: inp.dy[a:b], N, tail, rows, inp.wq,
                                   inp.wk, inp.wv, inp.wo, c["hq"], c["hkv"], c["d"], c["theta"], inp.q_norm,
                                   inp.k_norm)
    for C, (_, _, g) in runs.items():
        got = g[0].index_select(0, torch.from_numpy(rows).to("cuda")).float().cpu().numpy()
        e = _relerr(got, ref)
        print(f"  C={C}: tail dx rel {e:.3e}", flush=True)
        assert e <= TOL, (C, e)


def test_weight_gradient_identities(share, runs):
    c, _, t = share
    for C, (y, _, g) in runs.items():
        dx, dwq, dwk, dwv, dwo, dgq, dgk = g
        ref = _dot(t["dy"], y)
        a_o, a_v = _dot(dwo, t["wo"]), _dot(dwv, t["wv"])
        a_q, a_k = _dot(dwq, t["wq"]), _dot(dwk, t["wk"])
        print(f"  C={C}: <dY,y>={ref:.6e} <dWo,Wo>={a_o:.6e} <dWv,Wv>={a_v:.6e} <dWq,Wq>={a_q:.6e} "
              f"<dWk,Wk>={a_k:.6e}", flush=True)
        assert abs(a_o - ref) <= TOL * abs(ref)
        assert abs(a_v - ref) <= TOL * abs(ref)
        if c["norm"] is None:
            assert abs(a_q - a_k) <= TOL * max(abs(a_q), abs(a_k))
        else:
            g_q, g_k = _dot(dgq, t["q_norm"]), _dot(dgk, t["k_norm"])
            print(f"         <dgq,gq>={g_q:.6e} <dgk,gk>={g_k:.6e}", flush=True)
            assert abs(g_q - g_k) <= TOL * max(abs(g_q), abs(g_k))
            assert abs(a_q) <= TOL * abs(g_q) and abs(a_k) <= TOL * abs(g_k)


def test_chunk_invariance(share, runs):
    chunks = sorted(runs)
    y1, l1, g1 = runs[chunks[0]]
    for C in chunks[1:]:
        y, lse, g = runs[C]
        assert _relerr(y.float().cpu().numpy(), y1.float().cpu().numpy()) <= TOL
        assert float((lse - l1).abs().max()) <= 1e-3
        for a, b in zip(g, g1):
            if a is None:
                continue
            e = _relerr(a.float().cpu().numpy(), b.float().cpu().numpy())
            assert e <= TOL, (C, e)


def test_causality_bitwise(share, runs):
    c, _, t = share
    r = c["N"] // 2
    x2 = t["x"].clone()
    x2[r + 1:] = -x2[r + 1:]
    C = sorted(runs)[0]
    y2, lse2 = api.attn_fwd(x2, t["wq"], t["wk"], t["wv"], t["wo"], q_norm=t["q_norm"], k_norm=t["k_norm"],
                            **_kw(c, C))
    torch.cuda.synchronize()
    y1, l1, _ = runs[C]
    assert torch.equal(y2[:r + 1], y1[:r + 1])
    assert torch.equal(lse2[:, :r + 1], l1[:, :r + 1])
    assert not torch.equal(y2[r + 1:], y1[r + 1:])
    del x2, y2, lse2


def test_workspace_scaling_reported(share):
    """Workspace bytes per chunk size: the per-q-head part scales as chunk_heads."""
    c, _, _ = share
    ws = {C: api.workspace_bytes(c["N"], c["D"], c["hq"], c["hkv"], c["d"], C, c["norm"] is not None, "bf16",
                                 False) for C in c["chunks"]}
    kv = 2 * ((c["N"] + 255) // 256 * 256) * c["d"] * 2
    per_q = {C: ws[C] - kv for C in ws}
    print(f"[{c['name']}] fwd workspace GB per chunk: " + ", ".join(f"C={C}: {v / 1e9:.3f}" for C, v in ws.items()),
          flush=True)
    lo = min(per_q)
    for C in per_q:
        assert per_q[C] * lo == per_q[lo] * C
