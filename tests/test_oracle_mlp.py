"""Pins of the fp64 MLP oracle against facts that do not come from it.

The pages print no worked example of the MLP, so the pins are: PyTorch's CPU
silu and autograd in fp64 (library special cases), brute force in plain
Python loops, central finite differences, closed forms (silu at chosen
points, a zero gate, the large-gate limit), the exact identities
<dWd, Wd> = <dWu, Wu> = <dy, y>, row locality and the exactness of tiling.
A plausible slip in the oracle (a sign in silu', gate and up swapped, a
transposed weight, a missing term in dx) fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")

RNG = np.random.default_rng(77)


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def _relerr(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _problem(N=7, D=6, F=5, scale=0.5):
    return _rand(N, D), _rand(F, D, scale=scale), _rand(F, D, scale=scale), _rand(D, F, scale=scale), _rand(N, D)


def test_silu_closed_forms_and_torch():
    # closed forms: silu(0) = 0, silu(1) = 1/(1 + 1/e), silu(-1) = -1/(1 + e)
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(oracle.silu(-1.0) + 1.0 / (1.0 + math.e)) < 1e-15
    # far tails: silu(z) -> z and -> 0 without overflow
    assert oracle.silu(800.0) == 800.0
    assert oracle.silu(-800.0) == 0.0
    z = np.concatenate([np.linspace(-40, 40, 2001), _rand(500, scale=8.0)])
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    assert np.max(np.abs(oracle.silu(z) - ref) / (1.0 + np.abs(ref))) < 1e-15


def test_silu_grad_torch_autograd_and_finite_differences():
    z = np.concatenate([np.linspace(-30, 30, 601), _rand(200, scale=5.0)])
    t = torch.from_numpy(z).requires_grad_(True)
    (g,) = torch.autograd.grad(torch.nn.functional.silu(t).sum(), t)
    assert np.max(np.abs(oracle.silu_grad(z) - g.numpy())) < 1e-14
    eps = 1e-6
    fd = (oracle.silu(z + eps) - oracle.silu(z - eps)) / (2 * eps)
    assert np.max(np.abs(oracle.silu_grad(z) - fd)) < 1e-8
    # closed form at 0: silu'(0) = 1/2
    assert oracle.silu_grad(0.0) == 0.5


def test_forward_bruteforce_loops():
    x, wg, wu, wd, _ = _problem(N=4, D=5, F=3)
    y = oracle.mlp_fwd(x, wg, wu, wd)
    for i in range(4):
        a = []
        for f in range(3):
            h = sum(x[i][c] * wg[f][c] for c in range(5))
            u = sum(x[i][c] * wu[f][c] for c in range(5))
            a.append(h / (1.0 + math.exp(-h)) * u)
        for d in range(5):
            want = sum(a[f] * wd[d][f] for f in range(3))
            assert abs(y[i][d] - want) < 1e-12


def test_forward_and_backward_match_torch_autograd():
    x, wg, wu, wd, dy = _problem(N=9, D=8, F=11)
    tx, tg, tu, td = (torch.from_numpy(a).requires_grad_(True) for a in (x, wg, wu, wd))
    F = torch.nn.functional
    ty = F.linear(F.silu(F.linear(tx, tg)) * F.linear(tx, tu), td)
    assert _relerr(oracle.mlp_fwd(x, wg, wu, wd), ty.detach().numpy()) < 1e-14
    grads = torch.autograd.grad(ty, (tx, tg, tu, td), grad_outputs=torch.from_numpy(dy))
    mine = oracle.mlp_bwd(x, wg, wu, wd, dy)
    for a, b in zip(mine, grads):
        assert _relerr(a, b.numpy()) < 1e-13


def test_backward_finite_differences():
    x, wg, wu, wd, dy = _problem(N=3, D=4, F=5)
    dx, dwg, dwu, dwd = oracle.mlp_bwd(x, wg, wu, wd, dy)

    def loss(x_, wg_, wu_, wd_):
        return float(np.sum(oracle.mlp_fwd(x_, wg_, wu_, wd_) * dy))

    eps = 1e-6
    for which, grad in ((0, dx), (1, dwg), (2, dwu), (3, dwd)):
        args = [x, wg, wu, wd]
        for idx in np.ndindex(grad.shape):
            p = [a.copy() for a in args]
            m = [a.copy() for a in args]
            p[which][idx] += eps
            m[which][idx] -= eps
            fd = (loss(*p) - loss(*m)) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-7 * (1.0 + abs(fd)), (which, idx)


def test_zero_gate_and_large_gate_limits():
    x, wg, wu, wd, dy = _problem(N=6, D=5, F=4)
    # silu(0) = 0: a zero gate weight gives exactly zero output and zero dx
    z = np.zeros_like(wg)
    assert np.all(oracle.mlp_fwd(x, z, wu, wd) == 0.0)
    # a large positive gate (h >> 0): silu(h) = h (to e^-h), so y is the bilinear form
    xp = np.abs(x) + 1.0
    big = np.abs(wg) * 40.0 + 40.0
    want = ((xp @ big.T) * (xp @ wu.T)) @ wd.T
    assert _relerr(oracle.mlp_fwd(xp, big, wu, wd), want) < 1e-12


def test_weight_gradient_identities():
    x, wg, wu, wd, dy = _problem(N=12, D=7, F=9)
    y = oracle.mlp_fwd(x, wg, wu, wd)
    dx, dwg, dwu, dwd = oracle.mlp_bwd(x, wg, wu, wd, dy)
    ref = float(np.sum(dy * y))
    assert abs(float(np.sum(dwd * wd)) - ref) < 1e-11 * (1 + abs(ref))
    assert abs(float(np.sum(dwu * wu)) - ref) < 1e-11 * (1 + abs(ref))
    # the gate identity: <dWg, Wg> = sum dh * h
    h = x @ wg.T
    da = dy @ wd
    dh = da * (x @ wu.T) * oracle.silu_grad(h)
    assert abs(float(np.sum(dwg * wg)) - float(np.sum(dh * h))) < 1e-11 * (1 + abs(ref))


@pytest.mark.parametrize("tile", [1, 4, 5, 64])
def test_tiling_is_exact_and_rows_are_local(tile):
    x, wg, wu, wd, dy = _problem(N=13, D=6, F=7)
    y = oracle.mlp_fwd(x, wg, wu, wd)
    assert np.max(np.abs(oracle.mlp_fwd(x, wg, wu, wd, tile=tile) - y)) < 1e-13
    g = oracle.mlp_bwd(x, wg, wu, wd, dy)
    gt = oracle.mlp_bwd(x, wg, wu, wd, dy, tile=tile)
    for a, b in zip(g, gt):
        assert _relerr(b, a) < 1e-13
    rows = np.array([0, 5, 12])
    assert np.max(np.abs(oracle.mlp_rows(x[rows], wg, wu, wd) - y[rows])) < 1e-13
    assert np.max(np.abs(oracle.mlp_dx_rows(x[rows], dy[rows], wg, wu, wd) - g[0][rows])) < 1e-13
