"""Pins of the fp64 cross-entropy oracle against facts that do not come from it.

PyTorch's CPU cross_entropy and autograd in fp64 (library special cases),
brute force in plain Python loops, central finite differences, closed forms
(equal logits give log V; a dominant target logit gives a loss near 0) and
the exactness of tiling. A plausible slip (the target logit's sign, a missing
max shift that overflows, the onehot at the wrong column, a transposed W)
fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")

RNG = np.random.default_rng(99)


def _relerr(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _problem(N=9, D=6, V=11, scale=1.0):
    return (RNG.standard_normal((N, D)), RNG.standard_normal((V, D)) * scale, RNG.integers(0, V, N),
            RNG.standard_normal(N))


def test_matches_torch_cross_entropy_and_autograd():
    h, w, t, g = _problem()
    th, tw = (torch.from_numpy(a).requires_grad_(True) for a in (h, w))
    z = th @ tw.T
    ref = torch.nn.functional.cross_entropy(z, torch.from_numpy(t), reduction="none")
    loss, lse = oracle.ce_fwd(h, w, t)
    assert np.max(np.abs(loss - ref.detach().numpy())) < 1e-12
    assert np.max(np.abs(lse - torch.logsumexp(z, dim=1).detach().numpy())) < 1e-12
    dh_ref, dw_ref = torch.autograd.grad(ref, (th, tw), grad_outputs=torch.from_numpy(g))
    dh, dw = oracle.ce_bwd(h, w, t, g)
    assert _relerr(dh, dh_ref.numpy()) < 1e-13
    assert _relerr(dw, dw_ref.numpy()) < 1e-13


def test_bruteforce_loops():
    h, w, t, _ = _problem(N=3, D=4, V=5)
    loss, lse = oracle.ce_fwd(h, w, t)
    for i in range(3):
        z = [sum(h[i][c] * w[v][c] for c in range(4)) for v in range(5)]
        s = math.log(sum(math.exp(x) for x in z))
        assert abs(lse[i] - s) < 1e-12
        assert abs(loss[i] - (s - z[t[i]])) < 1e-12


def test_closed_forms():
    h, w, t, _ = _problem(N=5, D=4, V=7)
    # all logits equal (W = 0): lse = log V, loss = log V
    loss, lse = oracle.ce_fwd(h, np.zeros_like(w), t)
    assert np.max(np.abs(loss - math.log(7))) < 1e-15 and np.max(np.abs(lse - math.log(7))) < 1e-15
    # huge logits stay finite (max shift), and a dominant target gives ~0 loss
    w2 = np.zeros((7, 4))
    w2[3] = 1e3
    hp = np.abs(h) + 1.0
    loss, _ = oracle.ce_fwd(hp, w2, np.full(5, 3))
    assert np.all(np.isfinite(loss)) and np.max(loss) < 1e-12


def test_finite_differences():
    h, w, t, g = _problem(N=3, D=3, V=4)
    dh, dw = oracle.ce_bwd(h, w, t, g)

    def f(h_, w_):
        return float(np.sum(oracle.ce_fwd(h_, w_, t)[0] * g))

    eps = 1e-6
    for which, grad in ((0, dh), (1, dw)):
        for idx in np.ndindex(grad.shape):
            args_p = [h.copy(), w.copy()]
            args_m = [h.copy(), w.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            fd = (f(*args_p) - f(*args_m)) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-7 * (1 + abs(fd)), (which, idx)


@pytest.mark.parametrize("tile", [1, 3, 8])
def test_tiling_exact_and_rows_local(tile):
    h, w, t, g = _problem(N=13, D=5, V=9)
    loss, lse = oracle.ce_fwd(h, w, t)
    lt, st = oracle.ce_fwd(h, w, t, tile=tile)
    assert np.max(np.abs(lt - loss)) < 1e-13 and np.max(np.abs(st - lse)) < 1e-13
    dh, dw = oracle.ce_bwd(h, w, t, g)
    dht, dwt = oracle.ce_bwd(h, w, t, g, tile=tile)
    assert _relerr(dht, dh) < 1e-13 and _relerr(dwt, dw) < 1e-13
    rows = np.array([0, 4, 12])
    lr, sr = oracle.ce_rows(h[rows], w, t[rows])
    assert np.max(np.abs(lr - loss[rows])) < 1e-13
    assert _relerr(oracle.ce_dh_rows(h[rows], w, t[rows], g[rows]), dh[rows]) < 1e-13
