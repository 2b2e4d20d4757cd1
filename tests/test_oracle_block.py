"""Pins of the fp64 transformer-block oracle against facts that do not come from it.

The pages print no worked example of the block, so the pins are:
- a second forward built from PyTorch library routines in fp64 (rms_norm,
  scaled_dot_product_attention, silu) and its autograd gradients;
- special cases that reduce the block to the separately pinned sublayer
  oracles: zero output weights give y = h = x, a zero MLP down weight leaves
  y = h, a zero attention output weight leaves h = x;
- exact homogeneity identities of the weight gradients (each holds at any
  size because the block is linear in that weight or in that norm weight);
- central finite differences of every gradient along random directions;
- for the stack of blocks: one block is the block, each block's kept input is
  the previous block's output, and finite differences through two blocks.
A plausible slip in the oracle (a norm on the wrong tensor, a lost residual
term in dx or dh, the two norm weights swapped, the MLP reading h instead of
its norm) fails at least one of them.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
F = torch.nn.functional

SHAPE = dict(N=11, D=16, Hq=4, Hkv=2, d=8, Ff=24)
THETA = 1e4


def _problem(seed=0, qk_norm=False, wscale=0.4):
    r = np.random.default_rng(seed)
    N, D, Hq, Hkv, d, Ff = (SHAPE[k] for k in ("N", "D", "Hq", "Hkv", "d", "Ff"))
    p = {
        "x": r.standard_normal((N, D)),
        "g_attn": 1 + 0.2 * r.standard_normal(D),
        "wq": wscale * r.standard_normal((Hq * d, D)),
        "wk": wscale * r.standard_normal((Hkv * d, D)),
        "wv": wscale * r.standard_normal((Hkv * d, D)),
        "wo": wscale * r.standard_normal((D, Hq * d)),
        "g_mlp": 1 + 0.2 * r.standard_normal(D),
        "wg": wscale * r.standard_normal((Ff, D)),
        "wu": wscale * r.standard_normal((Ff, D)),
        "wd": wscale * r.standard_normal((D, Ff)),
    }
    p["q_norm"] = 1 + 0.2 * r.standard_normal(d) if qk_norm else None
    p["k_norm"] = 1 + 0.2 * r.standard_normal(d) if qk_norm else None
    dy = r.standard_normal((N, D))
    return p, dy


WEIGHTS = ("g_attn", "wq", "wk", "wv", "wo", "g_mlp", "wg", "wu", "wd")


def _fwd(p, chunk=1, tile=None, eps=1e-5):
    return oracle.block_fwd(p["x"], p["g_attn"], p["wq"], p["wk"], p["wv"], p["wo"], p["g_mlp"],
                            p["wg"], p["wu"], p["wd"], SHAPE["Hq"], SHAPE["Hkv"], SHAPE["d"], THETA,
                            chunk, p["q_norm"], p["k_norm"], 1e-6, eps, tile)


def _bwd(p, dy, chunk=1, tile=None, eps=1e-5):
    return oracle.block_bwd(p["x"], p["g_attn"], p["wq"], p["wk"], p["wv"], p["wo"], p["g_mlp"],
                            p["wg"], p["wu"], p["wd"], dy, SHAPE["Hq"], SHAPE["Hkv"], SHAPE["d"], THETA,
                            chunk, p["q_norm"], p["k_norm"], 1e-6, eps, tile)


def _torch_block(t, eps=1e-5, qk_eps=1e-6):
    """The same block from PyTorch library routines (fp64, CPU)."""
    N, D, Hq, Hkv, d = (SHAPE[k] for k in ("N", "D", "Hq", "Hkv", "d"))
    x = t["x"]
    a = F.rms_norm(x, (D,), t["g_attn"], eps)
    pos = torch.arange(N, dtype=torch.float64)
    inv = THETA ** (-2.0 * torch.arange(d // 2, dtype=torch.float64) / d)
    ang = pos[:, None] * inv[None, :]
    cos, sin = torch.cos(ang), torch.sin(ang)

    def rope(z):  # [H][N][d], rotate-half pairs (i, i + d/2)
        z1, z2 = z[..., : d // 2], z[..., d // 2:]
        return torch.cat([z1 * cos - z2 * sin, z2 * cos + z1 * sin], dim=-1)

    q = (a @ t["wq"].T).reshape(N, Hq, d).transpose(0, 1)
    k = (a @ t["wk"].T).reshape(N, Hkv, d).transpose(0, 1)
    v = (a @ t["wv"].T).reshape(N, Hkv, d).transpose(0, 1)
    if t.get("q_norm") is not None:
        q = F.rms_norm(q, (d,), t["q_norm"], qk_eps)
        k = F.rms_norm(k, (d,), t["k_norm"], qk_eps)
    q, k = rope(q), rope(k)
    g = Hq // Hkv
    k = k.repeat_interleave(g, dim=0)
    v = v.repeat_interleave(g, dim=0)
    o = F.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True)[0]
    h = x + o.transpose(0, 1).reshape(N, Hq * d) @ t["wo"].T
    b = F.rms_norm(h, (D,), t["g_mlp"], eps)
    y = h + (F.silu(b @ t["wg"].T) * (b @ t["wu"].T)) @ t["wd"].T
    return y, h


@pytest.mark.parametrize("qk_norm", [False, True])
def test_forward_and_gradients_match_torch_library_block(qk_norm):
    p, dy = _problem(seed=1 + qk_norm, qk_norm=qk_norm)
    y, h, _ = _fwd(p)
    t = {k: (torch.from_numpy(v).requires_grad_(True) if v is not None else None) for k, v in p.items()}
    yt, ht = _torch_block(t)
    assert np.max(np.abs(y - yt.detach().numpy())) < 1e-12
    assert np.max(np.abs(h - ht.detach().numpy())) < 1e-12
    (yt * torch.from_numpy(dy)).sum().backward()
    g = _bwd(p, dy)
    for name in ("x",) + WEIGHTS + (("q_norm", "k_norm") if qk_norm else ()):
        ref = t[name].grad.numpy()
        got = g["dx" if name == "x" else name]
        assert np.max(np.abs(got - ref)) < 1e-10 * (1 + np.max(np.abs(ref))), name


def test_zero_output_weights_give_identity():
    p, _ = _problem(seed=3)
    p["wo"][:] = 0.0
    p["wd"][:] = 0.0
    y, h, lse = _fwd(p)
    assert np.array_equal(y, p["x"]) and np.array_equal(h, p["x"])
    # the attention still runs on the normed input: its lse is the sublayer's
    a = oracle.rmsnorm(p["x"], p["g_attn"], 1e-5)
    _, lse_ref = oracle.layer_fwd(a, p["wq"], p["wk"], p["wv"], p["wo"], SHAPE["Hq"], SHAPE["Hkv"],
                                  SHAPE["d"], THETA, 1)
    assert np.array_equal(lse, lse_ref)


def test_each_branch_alone_reduces_to_its_sublayer():
    p, _ = _problem(seed=4)
    # no attention output: h = x, y = x + mlp(rmsnorm(x; g_mlp))
    q = {k: (v.copy() if v is not None else None) for k, v in p.items()}
    q["wo"][:] = 0.0
    y, h, _ = _fwd(q)
    m = oracle.mlp_fwd(oracle.rmsnorm(p["x"], p["g_mlp"], 1e-5), p["wg"], p["wu"], p["wd"])
    assert np.array_equal(h, p["x"])
    assert np.allclose(y, p["x"] + m, rtol=0, atol=1e-13)
    # no MLP output: y = h = x + attn(rmsnorm(x; g_attn))
    q = {k: (v.copy() if v is not None else None) for k, v in p.items()}
    q["wd"][:] = 0.0
    y, h, _ = _fwd(q)
    att, _ = oracle.layer_fwd(oracle.rmsnorm(p["x"], p["g_attn"], 1e-5), p["wq"], p["wk"], p["wv"],
                              p["wo"], SHAPE["Hq"], SHAPE["Hkv"], SHAPE["d"], THETA, 1)
    assert np.array_equal(y, h)
    assert np.allclose(h, p["x"] + att, rtol=0, atol=1e-13)


@pytest.mark.parametrize("qk_norm", [False, True])
def test_homogeneity_identities(qk_norm):
    """y is linear in Wd and in Wu; h in Wo. b enters the MLP only through
    b Wg^T and b Wu^T, and b is linear in g_mlp, so <dg_mlp, g_mlp> =
    <dWg, Wg> + <dWu, Wu>; likewise <dg_attn, g_attn> = <dWq, Wq> +
    <dWk, Wk> + <dWv, Wv>."""
    p, dy = _problem(seed=5 + qk_norm, qk_norm=qk_norm)
    y, h, _ = _fwd(p)
    g = _bwd(p, dy)

    def dot(a, b):
        return float(np.sum(a * b))

    m = dot(dy, y - h)
    assert abs(dot(g["wd"], p["wd"]) - m) < 1e-10 * (1 + abs(m))
    assert abs(dot(g["wu"], p["wu"]) - m) < 1e-10 * (1 + abs(m))
    s2 = dot(g["wg"], p["wg"]) + dot(g["wu"], p["wu"])
    assert abs(dot(g["g_mlp"], p["g_mlp"]) - s2) < 1e-10 * (1 + abs(s2))
    s1 = dot(g["wq"], p["wq"]) + dot(g["wk"], p["wk"]) + dot(g["wv"], p["wv"])
    assert abs(dot(g["g_attn"], p["g_attn"]) - s1) < 1e-10 * (1 + abs(s1))


@pytest.mark.parametrize("qk_norm", [False, True])
def test_gradients_central_finite_differences(qk_norm):
    p, dy = _problem(seed=9 + qk_norm, qk_norm=qk_norm)
    g = _bwd(p, dy, chunk=2)
    r = np.random.default_rng(21)
    names = ("x",) + WEIGHTS + (("q_norm", "k_norm") if qk_norm else ())
    for name in names:
        v = r.standard_normal(p[name].shape)
        e = 1e-5

        def loss(sign):
            q = dict(p)
            q[name] = p[name] + sign * e * v
            return float(np.sum(_fwd(q, chunk=2)[0] * dy))

        num = (loss(1) - loss(-1)) / (2 * e)
        ana = float(np.sum(g["dx" if name == "x" else name] * v))
        assert abs(num - ana) < 1e-6 * (1 + abs(ana)), (name, num, ana)


def test_chunk_and_tile_invariance():
    p, dy = _problem(seed=12)
    y1, h1, l1 = _fwd(p, chunk=1)
    y4, h4, l4 = _fwd(p, chunk=4, tile=3)
    assert np.allclose(y1, y4, rtol=0, atol=1e-13) and np.allclose(l1, l4, rtol=0, atol=1e-13)
    g1, g4 = _bwd(p, dy, chunk=1), _bwd(p, dy, chunk=2, tile=5)
    for k in ("dx",) + WEIGHTS:
        assert np.allclose(g1[k], g4[k], rtol=0, atol=1e-11), k


def _layers(n, seed):
    out = []
    for i in range(n):
        p, _ = _problem(seed=seed + i)
        p.pop("x")
        out.append(p)
    return out


def test_stack_of_one_is_the_block_and_inputs_chain():
    p, dy = _problem(seed=30)
    lay = [{k: v for k, v in p.items() if k != "x"}]
    y, inputs = oracle.stack_fwd(p["x"], lay, SHAPE["Hq"], SHAPE["Hkv"], SHAPE["d"], THETA)
    assert np.array_equal(y, _fwd(p)[0]) and np.array_equal(inputs[0], p["x"])
    dx, grads = oracle.stack_bwd(p["x"], lay, dy, SHAPE["Hq"], SHAPE["Hkv"], SHAPE["d"], THETA)
    ref = _bwd(p, dy)
    assert np.array_equal(dx, ref["dx"])
    for k in WEIGHTS:
        assert np.array_equal(grads[0][k], ref[k]), k
    # two blocks: block 1's input is block 0's output
    lay2 = _layers(2, 40)
    y2, inp2 = oracle.stack_fwd(p["x"], lay2, SHAPE["Hq"], SHAPE["Hkv"], SHAPE["d"], THETA)
    q = dict(lay2[0], x=p["x"])
    assert np.array_equal(inp2[1], _fwd(q)[0])


def test_stack_gradients_central_finite_differences():
    """Chain rule across blocks: the input gradient and a weight gradient of
    the first of two blocks, against finite differences of <dy, y>."""
    r = np.random.default_rng(50)
    x = r.standard_normal((SHAPE["N"], SHAPE["D"]))
    dy = r.standard_normal((SHAPE["N"], SHAPE["D"]))
    lay = _layers(2, 60)
    dx, grads = oracle.stack_bwd(x, lay, dy, SHAPE["Hq"], SHAPE["Hkv"], SHAPE["d"], THETA)
    e = 1e-5

    def loss(xx, ll):
        return float(np.sum(oracle.stack_fwd(xx, ll, SHAPE["Hq"], SHAPE["Hkv"], SHAPE["d"], THETA)[0] * dy))

    v = r.standard_normal(x.shape)
    num = (loss(x + e * v, lay) - loss(x - e * v, lay)) / (2 * e)
    assert abs(num - float(np.sum(dx * v))) < 1e-6 * (1 + abs(num))
    for name in ("wq", "wd", "g_attn"):
        v = r.standard_normal(lay[0][name].shape)
        lp = [dict(lay[0], **{name: lay[0][name] + e * v}), lay[1]]
        lm = [dict(lay[0], **{name: lay[0][name] - e * v}), lay[1]]
        num = (loss(x, lp) - loss(x, lm)) / (2 * e)
        ana = float(np.sum(grads[0][name] * v))
        assert abs(num - ana) < 1e-6 * (1 + abs(ana)), name
