"""Helpers for the GPU parity tests: upload synthetic inputs, run the HIP
path through the C ABI binding, run the oracle on the same inputs."""
import numpy as np
import torch

import oracle
from headwise_chunked_attention_amd import api
from headwise_chunked_attention_amd.synth import LayerInputs

TORCH_DT = {"fp32": torch.float32, "bf16": torch.bfloat16}
TOL = {"fp32": 1e-5, "bf16": 2e-2}


def relerr(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def dev(a, dt):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(TORCH_DT[dt])


def host(t):
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64)


class Case:
    def __init__(self, N, D, hq, hkv, d, dtype, theta=5e5, norm=None, seed=0, eps=1e-6, inp=None):
        self.N, self.D, self.hq, self.hkv, self.d = N, D, hq, hkv, d
        self.dtype, self.theta, self.eps = dtype, theta, eps
        self.inp = inp if inp is not None else LayerInputs(N, D, hq, hkv, d, dtype, seed=seed, qk_norm=norm)
        self.norm = norm is not None
        i = self.inp
        self.t = {k: dev(getattr(i, k), dtype) for k in ("x", "dy", "wq", "wk", "wv", "wo", "q_norm", "k_norm")}

    def kw(self, C):
        return dict(n_q_heads=self.hq, n_kv_heads=self.hkv, head_dim=self.d, rope_theta=self.theta,
                    chunk_heads=C, q_norm=self.t["q_norm"], k_norm=self.t["k_norm"], eps=self.eps)

    def gpu_fwd(self, C):
        t = self.t
        y, lse = api.attn_fwd(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], **self.kw(C))
        torch.cuda.synchronize()
        return y, lse

    def gpu_bwd(self, C, lse):
        t = self.t
        g = api.attn_bwd(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], t["dy"], lse, **self.kw(C))
        torch.cuda.synchronize()
        return g

    def oracle_fwd(self, C):
        i = self.inp
        return oracle.layer_fwd(i.x, i.wq, i.wk, i.wv, i.wo, self.hq, self.hkv, self.d, self.theta, C,
                                i.q_norm, i.k_norm, self.eps)

    def oracle_bwd(self, C):
        i = self.inp
        return oracle.layer_bwd(i.x, i.wq, i.wk, i.wv, i.wo, i.dy, self.hq, self.hkv, self.d, self.theta, C,
                                i.q_norm, i.k_norm, self.eps)


GRAD_NAMES = ("dx", "dwq", "dwk", "dwv", "dwo", "dq_norm", "dk_norm")


def check_fwd(case, C, y, lse, ref=None, tol=None, lse_bound=None):
    """y and LSE against the oracle: relative L2 <= tol, and LSE max-abs <= tol,
    or, with ``lse_bound`` ([Hq][N]), |LSE - ref| <= lse_bound element by element."""
    tol = tol or TOL[case.dtype]
    y_ref, lse_ref = ref if ref is not None else case.oracle_fwd(C)
    ey = relerr(host(y), y_ref)
    el = relerr(host(lse), lse_ref)
    dl = np.abs(host(lse) - lse_ref)
    ml = float(np.max(dl))
    msg = f"  fwd C={C}: y rel {ey:.3e}  lse rel {el:.3e} max {ml:.3e}"
    if lse_bound is not None:
        msg += f" (max of |dLSE| / its rounding bound {float(np.max(dl / lse_bound)):.3f})"
    print(msg, flush=True)
    assert ey <= tol, ("y", ey)
    assert el <= tol, ("lse", el)
    if lse_bound is None:
        assert ml <= tol, ("lse max abs", ml)
    else:
        assert bool(np.all(dl <= lse_bound)), ("lse beyond its rounding bound", float(np.max(dl / lse_bound)))


def check_bwd(case, C, grads, ref=None, tol=None):
    tol = tol or TOL[case.dtype]
    ref = ref if ref is not None else case.oracle_bwd(C)
    for name, g, r in zip(GRAD_NAMES, grads, ref):
        if r is None:
            assert g is None
            continue
        if np.linalg.norm(r) == 0.0:
            # exactly zero (e.g. N=1: one visible key, so dS = P (dP - Delta) = 0)
            e = float(np.max(np.abs(host(g))))
            print(f"  bwd C={C}: {name} exact 0, max abs {e:.3e}", flush=True)
        else:
            e = relerr(host(g), r)
            print(f"  bwd C={C}: {name} rel {e:.3e}", flush=True)
        assert e <= tol, (name, e)
