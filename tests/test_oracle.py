"""Pins of the CPU fp64 oracle against facts that do not come from the oracle.

The pages print no worked example, so the pins are: brute force written
independently in plain Python loops (complex-number RoPE, explicit sums),
closed forms at row 0, a library special case (PyTorch CPU SDPA in fp64),
GQA as MHA with repeated kv heads, RoPE/RMSNorm identities, central finite
differences for every gradient, exactness of the chunk sum, causality and
linearity. Each is chosen so that a plausible slip in the oracle (a dropped
term, a wrong sign, index or scale, a transposed operand) fails at least one.
"""
import cmath
import math

import numpy as np
import pytest

import oracle
from headwise_chunked_attention_amd import synth

RNG = np.random.default_rng(1234)


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def _relerr(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------------------
# brute force: pure Python, written without any oracle helper
# ---------------------------------------------------------------------------
def _bf_matvec_rows(x, w, r0, r1):
    """rows r0..r1 of W applied to each row of x: out[p][r-r0] = sum_c x[p][c] W[r][c]."""
    return [[sum(x[p][c] * w[r][c] for c in range(len(x[p]))) for r in range(r0, r1)]
            for p in range(len(x))]


def _bf_norm(t, gamma, eps):
    out = []
    for row in t:
        ms = sum(a * a for a in row) / len(row)
        out.append([gamma[i] * row[i] / math.sqrt(ms + eps) for i in range(len(row))])
    return out


def _bf_rope(t, theta):
    """Complex form: the pair (t[i], t[i+d/2]) is the number t[i] + 1j*t[i+d/2],
    multiplied by exp(1j * p * theta**(-2i/d))."""
    out = []
    for p, row in enumerate(t):
        d = len(row)
        h = d // 2
        new = [0.0] * d
        for i in range(h):
            z = complex(row[i], row[i + h]) * cmath.exp(1j * p * theta ** (-2.0 * i / d))
            new[i], new[i + h] = z.real, z.imag
        out.append(new)
    return out


def _bf_layer(x, wq, wk, wv, wo, hq, hkv, d, theta, gq=None, gk=None, eps=1e-6):
    x = x.tolist()
    wq, wk, wv, wo = wq.tolist(), wk.tolist(), wv.tolist(), wo.tolist()
    n = len(x)
    dm = len(wo)
    grp = hq // hkv
    y = [[0.0] * dm for _ in range(n)]
    lse = [[0.0] * n for _ in range(hq)]
    for h in range(hq):
        g = h // grp
        q = _bf_matvec_rows(x, wq, h * d, (h + 1) * d)
        k = _bf_matvec_rows(x, wk, g * d, (g + 1) * d)
        v = _bf_matvec_rows(x, wv, g * d, (g + 1) * d)
        if gq is not None:
            q = _bf_norm(q, gq.tolist(), eps)
            k = _bf_norm(k, gk.tolist(), eps)
        q = _bf_rope(q, theta)
        k = _bf_rope(k, theta)
        for i in range(n):
            scores = [sum(q[i][c] * k[j][c] for c in range(d)) / math.sqrt(d) for j in range(i + 1)]
            m = max(scores)
            z = sum(math.exp(s - m) for s in scores)
            lse[h][i] = m + math.log(z)
            o = [sum(math.exp(scores[j] - m) / z * v[j][c] for j in range(i + 1)) for c in range(d)]
            for r in range(dm):
                y[i][r] += sum(o[c] * wo[r][h * d + c] for c in range(d))
    return np.array(y), np.array(lse)


@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("hq,hkv", [(4, 2), (4, 1), (2, 2)])
def test_bruteforce_forward(norm, hq, hkv):
    n, dm, d, theta = 7, 12, 4, 50.0
    x = _rand(n, dm)
    wq, wk, wv = _rand(hq * d, dm, scale=0.5), _rand(hkv * d, dm, scale=0.5), _rand(hkv * d, dm, scale=0.5)
    wo = _rand(dm, hq * d, scale=0.5)
    gq = 1 + 0.1 * _rand(d) if norm else None
    gk = 1 + 0.1 * _rand(d) if norm else None
    y_bf, lse_bf = _bf_layer(x, wq, wk, wv, wo, hq, hkv, d, theta, gq, gk)
    for c in [1, hq]:
        y, lse = oracle.layer_fwd(x, wq, wk, wv, wo, hq, hkv, d, theta, c, gq, gk)
        assert np.max(np.abs(y - y_bf)) < 1e-12 * (1 + np.max(np.abs(y_bf)))
        assert np.max(np.abs(lse - lse_bf)) < 1e-12


# ---------------------------------------------------------------------------
# softmax / closed forms / library special cases
# ---------------------------------------------------------------------------
def _layer_inputs(n=24, dm=32, hq=4, hkv=2, d=8, wscale=0.3, seed=0):
    r = np.random.default_rng(seed)
    x = r.standard_normal((n, dm))
    wq = r.standard_normal((hq * d, dm)) * wscale
    wk = r.standard_normal((hkv * d, dm)) * wscale
    wv = r.standard_normal((hkv * d, dm)) * wscale
    wo = r.standard_normal((dm, hq * d)) * wscale
    return x, wq, wk, wv, wo


def test_softmax_rows_and_causal_zeros():
    x, wq, wk, wv, wo = _layer_inputs()
    _, _, it = oracle.layer_fwd(x, wq, wk, wv, wo, 4, 2, 8, 1e4, 2, keep=True)
    for h, p in it["p"].items():
        assert np.allclose(p.sum(axis=1), 1.0, atol=1e-13, rtol=0)
        assert np.all(p[np.triu_indices(p.shape[0], 1)] == 0.0)
        assert np.all(p >= 0)


def test_row0_closed_form():
    x, wq, wk, wv, wo = _layer_inputs()
    _, lse, it = oracle.layer_fwd(x, wq, wk, wv, wo, 4, 2, 8, 1e4, 4, keep=True)
    for h in range(4):
        g = h // 2
        q0, k0 = it["q"][h][0], it["k"][g][0]
        assert abs(lse[h, 0] - q0 @ k0 / math.sqrt(8)) < 1e-13
        assert np.allclose(it["o"][h][0], it["v"][g][0], atol=1e-14, rtol=0)


def test_attention_core_matches_torch_sdpa():
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(5)
    q, k, v = r.standard_normal((3, 40, 16))
    o, lse, _ = oracle.causal_attention(q, k, v)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], is_causal=True)[0, 0].numpy()
    assert _relerr(o, ref) < 1e-13
    # LSE against torch.logsumexp of the masked scores
    s = torch.from_numpy(q @ k.T / 4.0)
    s = s.masked_fill(torch.triu(torch.ones(40, 40, dtype=torch.bool), 1), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) < 1e-13


def test_layer_without_rope_matches_torch_sdpa():
    torch = pytest.importorskip("torch")
    x, wq, wk, wv, wo = _layer_inputs(hq=3, hkv=3)
    y, _ = oracle.layer_fwd(x, wq, wk, wv, wo, 3, 3, 8, 1e4, 1, use_rope=False)
    xt = torch.from_numpy(x)
    q = (xt @ torch.from_numpy(wq).T).reshape(-1, 3, 8).transpose(0, 1)
    k = (xt @ torch.from_numpy(wk).T).reshape(-1, 3, 8).transpose(0, 1)
    v = (xt @ torch.from_numpy(wv).T).reshape(-1, 3, 8).transpose(0, 1)
    o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True)[0]
    ref = o.transpose(0, 1).reshape(-1, 24) @ torch.from_numpy(wo).T
    assert _relerr(y, ref.numpy()) < 1e-13


def test_gqa_equals_mha_with_repeated_kv():
    x, wq, wk, wv, wo = _layer_inputs(hq=8, hkv=2)
    y, lse = oracle.layer_fwd(x, wq, wk, wv, wo, 8, 2, 8, 1e4, 2)
    # torch.repeat_interleave semantics: kv head g serves q heads g*G .. g*G+G-1
    wk8 = np.repeat(wk.reshape(2, 8, -1), 4, axis=0).reshape(64, -1)
    wv8 = np.repeat(wv.reshape(2, 8, -1), 4, axis=0).reshape(64, -1)
    y8, lse8 = oracle.layer_fwd(x, wq, wk8, wv8, wo, 8, 8, 8, 1e4, 8)
    assert _relerr(y, y8) < 1e-14
    assert np.max(np.abs(lse - lse8)) < 1e-13


# ---------------------------------------------------------------------------
# RoPE and RMSNorm identities
# ---------------------------------------------------------------------------
def test_rope_identities():
    t = _rand(50, 16)
    pos = np.arange(50)
    r = oracle.apply_rope(t, pos, 500000.0)
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(t, axis=1), rtol=1e-14)
    assert np.array_equal(r[0], t[0])  # angle 0 at position 0
    # relative position: <rope(q, m), rope(k, n)> depends on m - n only
    q, k = _rand(1, 16), _rand(1, 16)
    for m, n in [(5, 2), (37, 11)]:
        a = oracle.apply_rope(q, [m], 1e4) @ oracle.apply_rope(k, [n], 1e4).T
        b = oracle.apply_rope(q, [m + 1000], 1e4) @ oracle.apply_rope(k, [n + 1000], 1e4).T
        assert abs(a - b) < 1e-11
    # complex-multiplication form, pair (i, i + d/2)
    p = 123
    z = (t[3, :8] + 1j * t[3, 8:]) * np.exp(1j * p * 1e4 ** (-2.0 * np.arange(8) / 16))
    r3 = oracle.apply_rope(t[3:4], [p], 1e4)[0]
    assert np.allclose(r3, np.concatenate([z.real, z.imag]), atol=1e-13, rtol=0)
    # transpose: adjoint and inverse of the rotation
    b = _rand(50, 16)
    lhs = np.sum(oracle.apply_rope(t, pos, 1e4) * b)
    rhs = np.sum(t * oracle.rope_transpose(b, pos, 1e4))
    assert abs(lhs - rhs) < 1e-11
    assert np.allclose(oracle.rope_transpose(oracle.apply_rope(t, pos, 1e4), pos, 1e4), t, atol=1e-13)


def test_rope_large_position_angle_in_fp64():
    # at position 5,242,879 the fp64 angle must not be degraded by float32 rounding
    p = 5242879
    c, s = oracle.rope_cos_sin([p], 128, 500000.0)
    assert abs(c[0, 0] - math.cos(p)) < 1e-9 and abs(s[0, 0] - math.sin(p)) < 1e-9
    w = 500000.0 ** (-2.0 * 5 / 128)
    assert abs(c[0, 5] - math.cos(p * w)) < 1e-9


def test_rmsnorm_identities():
    u = _rand(20, 16) * 3
    y = oracle.rmsnorm(u, np.ones(16), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)
    assert np.allclose(oracle.rmsnorm(7.5 * u, np.ones(16), 0.0), y, rtol=1e-13)
    g = 1 + 0.1 * _rand(16)
    assert np.allclose(oracle.rmsnorm(u, g, 0.0), g * y, rtol=1e-14)


# ---------------------------------------------------------------------------
# gradients: central finite differences of the forward
# ---------------------------------------------------------------------------
FD_SHAPE = dict(n=8, dm=16, hq=4, hkv=2, d=8)


def _fd_check(norm, chunk, theta=1e4, n_coords=24):
    r = np.random.default_rng(7 + chunk + 10 * norm)
    n, dm, hq, hkv, d = (FD_SHAPE[k] for k in ("n", "dm", "hq", "hkv", "d"))
    x, wq, wk, wv, wo = _layer_inputs(n, dm, hq, hkv, d, wscale=0.5, seed=3 + chunk)
    gq = 1 + 0.2 * r.standard_normal(d) if norm else None
    gk = 1 + 0.2 * r.standard_normal(d) if norm else None
    dy = r.standard_normal((n, dm))
    eps = 1e-6
    grads = oracle.layer_bwd(x, wq, wk, wv, wo, dy, hq, hkv, d, theta, chunk, gq, gk, eps)
    names = ["x", "wq", "wk", "wv", "wo", "gq", "gk"]
    params = {"x": x, "wq": wq, "wk": wk, "wv": wv, "wo": wo, "gq": gq, "gk": gk}

    def loss(p):
        y, _ = oracle.layer_fwd(p["x"], p["wq"], p["wk"], p["wv"], p["wo"], hq, hkv, d, theta,
                                chunk, p["gq"], p["gk"], eps)
        return float(np.sum(y * dy))

    h = 1e-6
    for name, g in zip(names, grads):
        if params[name] is None:
            assert g is None
            continue
        base = params[name]
        flat = base.reshape(-1)
        idx = r.choice(flat.size, size=min(n_coords, flat.size), replace=False)
        num = np.empty(idx.size)
        for t, i in enumerate(idx):
            pp = dict(params)
            a = flat.copy(); a[i] += h; pp[name] = a.reshape(base.shape); lp = loss(pp)
            a = flat.copy(); a[i] -= h; pp[name] = a.reshape(base.shape); lm = loss(pp)
            num[t] = (lp - lm) / (2 * h)
        ana = np.asarray(g).reshape(-1)[idx]
        err = np.linalg.norm(ana - num) / max(np.linalg.norm(num), 1e-12)
        assert err < 1e-6, (name, err)
        # directional derivative over the whole tensor
        dirn = r.standard_normal(base.shape)
        pp = dict(params); pp[name] = base + h * dirn; lp = loss(pp)
        pp[name] = base - h * dirn; lm = loss(pp)
        num_dir = (lp - lm) / (2 * h)
        ana_dir = float(np.sum(np.asarray(g) * dirn))
        assert abs(ana_dir - num_dir) < 1e-6 * max(1.0, abs(num_dir)), (name, ana_dir, num_dir)


@pytest.mark.parametrize("chunk", [1, 2, 4])
def test_finite_differences_plain(chunk):
    _fd_check(norm=False, chunk=chunk)


@pytest.mark.parametrize("chunk", [1, 4])
def test_finite_differences_qk_norm(chunk):
    _fd_check(norm=True, chunk=chunk)


def test_rmsnorm_bwd_finite_differences():
    u = _rand(5, 8)
    g = 1 + 0.1 * _rand(8)
    dout = _rand(5, 8)
    du, dg = oracle.rmsnorm_bwd(u, g, 1e-6, dout)
    h = 1e-6
    for i in range(u.size):
        a = u.copy().reshape(-1); a[i] += h
        b = u.copy().reshape(-1); b[i] -= h
        num = (np.sum(oracle.rmsnorm(a.reshape(u.shape), g, 1e-6) * dout)
               - np.sum(oracle.rmsnorm(b.reshape(u.shape), g, 1e-6) * dout)) / (2 * h)
        assert abs(num - du.reshape(-1)[i]) < 1e-7
    for i in range(8):
        a = g.copy(); a[i] += h
        b = g.copy(); b[i] -= h
        num = (np.sum(oracle.rmsnorm(u, a, 1e-6) * dout) - np.sum(oracle.rmsnorm(u, b, 1e-6) * dout)) / (2 * h)
        assert abs(num - dg[i]) < 1e-7


# ---------------------------------------------------------------------------
# the method's own invariants: chunking is exact, the layer is causal
# ---------------------------------------------------------------------------
def test_chunk_invariance_forward_and_backward():
    x, wq, wk, wv, wo = _layer_inputs(n=20, dm=24, hq=8, hkv=2, d=8)
    dy = np.random.default_rng(9).standard_normal((20, 24))
    gq = 1 + 0.1 * np.random.default_rng(10).standard_normal(8)
    gk = 1 + 0.1 * np.random.default_rng(11).standard_normal(8)
    ref_y, ref_l = oracle.layer_fwd(x, wq, wk, wv, wo, 8, 2, 8, 1e4, 8, gq, gk)
    ref_g = oracle.layer_bwd(x, wq, wk, wv, wo, dy, 8, 2, 8, 1e4, 8, gq, gk)
    for c in [1, 2, 4]:
        y, l_ = oracle.layer_fwd(x, wq, wk, wv, wo, 8, 2, 8, 1e4, c, gq, gk)
        assert _relerr(y, ref_y) < 1e-13 and np.max(np.abs(l_ - ref_l)) < 1e-13
        for a, b in zip(oracle.layer_bwd(x, wq, wk, wv, wo, dy, 8, 2, 8, 1e4, c, gq, gk), ref_g):
            assert _relerr(a, b) < 1e-13


def test_chunk_plan():
    assert [(list(q), list(k)) for q, k in oracle.chunk_plan(8, 2, 2)] == [
        ([0, 1], [0]), ([2, 3], [0]), ([4, 5], [1]), ([6, 7], [1])]
    assert [(list(q), list(k)) for q, k in oracle.chunk_plan(8, 2, 8)] == [(list(range(8)), [0, 1])]
    with pytest.raises(ValueError):
        oracle.chunk_plan(8, 2, 3)
    with pytest.raises(ValueError):
        oracle.chunk_plan(12, 2, 4)  # G = 6 vs C = 4


def test_causality():
    x, wq, wk, wv, wo = _layer_inputs(n=30)
    y, lse = oracle.layer_fwd(x, wq, wk, wv, wo, 4, 2, 8, 1e4, 2)
    x2 = x.copy()
    x2[17:] += np.random.default_rng(3).standard_normal(x2[17:].shape)
    y2, lse2 = oracle.layer_fwd(x2, wq, wk, wv, wo, 4, 2, 8, 1e4, 2)
    assert np.array_equal(y[:17], y2[:17]) and np.array_equal(lse[:, :17], lse2[:, :17])
    assert not np.allclose(y[17:], y2[17:])


def test_linearity_in_wo():
    x, wq, wk, wv, wo = _layer_inputs()
    dy = np.random.default_rng(4).standard_normal((24, 32))
    y, _, it = oracle.layer_fwd(x, wq, wk, wv, wo, 4, 2, 8, 1e4, 2, keep=True)
    y3, _ = oracle.layer_fwd(x, wq, wk, wv, 3.0 * wo, 4, 2, 8, 1e4, 2)
    assert _relerr(y3, 3.0 * y) < 1e-15
    dwo = oracle.layer_bwd(x, wq, wk, wv, wo, dy, 4, 2, 8, 1e4, 2)[4]
    for h in range(4):
        assert np.allclose(dwo[:, h * 8:(h + 1) * 8], dy.T @ it["o"][h], atol=1e-13, rtol=0)


# ---------------------------------------------------------------------------
# large-N variants equal the full oracle on a small problem
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("norm", [False, True])
def test_sampled_rows_and_tail_match_full(norm):
    n, dm, hq, hkv, d = 300, 32, 4, 1, 16
    x, wq, wk, wv, wo = _layer_inputs(n, dm, hq, hkv, d, wscale=0.2, seed=21)
    dy = np.random.default_rng(22).standard_normal((n, dm))
    gq = 1 + 0.1 * np.random.default_rng(23).standard_normal(d) if norm else None
    gk = 1 + 0.1 * np.random.default_rng(24).standard_normal(d) if norm else None
    y, lse = oracle.layer_fwd(x, wq, wk, wv, wo, hq, hkv, d, 1e4, 1, gq, gk)
    dx = oracle.layer_bwd(x, wq, wk, wv, wo, dy, hq, hkv, d, 1e4, 2, gq, gk)[0]
    rows = np.array([0, 1, 63, 64, 150, 299])
    yr, lr = oracle.layer_fwd_rows(lambda a, b: x[a:b], lambda i: x[i], n, rows, wq, wk, wv, wo,
                                   hq, hkv, d, 1e4, gq, gk, block=64, row_group=4)
    assert _relerr(yr, y[rows]) < 1e-13
    assert np.max(np.abs(lr - lse[:, rows])) < 1e-13
    tail_rows = np.array([250, 251, 280, 299])
    dxr = oracle.layer_bwd_tail_dx(lambda a, b: x[a:b], lambda a, b: dy[a:b], n, 64, tail_rows,
                                   wq, wk, wv, wo, hq, hkv, d, 1e4, gq, gk, block=64, row_group=16)
    assert _relerr(dxr, dx[tail_rows]) < 1e-12


# ---------------------------------------------------------------------------
# the shared input generator
# ---------------------------------------------------------------------------
def test_bf16_rounding_pins():
    v = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -7, -2.5, 3.0e-3], dtype=np.float32)
    r = synth.round_to_bf16(v)
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even mantissa (1.0);
    # 1+3*2^-8 is a tie between 1+2^-7 and 1+2^-6 -> even (1+2^-6)
    assert r.tolist()[:5] == [1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, -2.5]
    assert abs(r[5] - 3.0e-3) <= 2 ** -8 * 3.0e-3  # half an ulp of an 8-bit significand
    torch = pytest.importorskip("torch")
    w = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 5
    ref = torch.from_numpy(w).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(synth.round_to_bf16(w), ref)


def test_generator_blocks_regenerate():
    n = 3 * synth.ROW_BLOCK + 100
    b = synth.ROW_BLOCK
    full = synth.gen_rows("x", n, 8, 1.0, "bf16", seed=0)
    part = synth.gen_rows("x", n, 8, 1.0, "bf16", seed=0, row_start=b - 6, row_stop=b + 4)
    assert np.array_equal(full[b - 6:b + 4], part)
    idx = np.array([n - 1, 3, b, b - 1, 2 * b + 5])
    assert np.array_equal(synth.gen_rows_at("x", n, 8, 1.0, "bf16", 0, idx), full[idx])
    # threaded generation of a large tensor equals block-by-block generation
    big = synth.gen_rows("dy", 4 * b, 1024, 1.0, "bf16", seed=3)
    for k in range(4):
        blk = synth.gen_rows("dy", 4 * b, 1024, 1.0, "bf16", seed=3, row_start=k * b + 1, row_stop=(k + 1) * b)
        assert np.array_equal(big[k * b + 1:(k + 1) * b], blk)
    other = synth.gen_rows("wq", n, 8, 1.0, "bf16", seed=0)
    assert not np.array_equal(full, other)
