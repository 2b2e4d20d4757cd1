"""Host-side checks of the C ABI: the library loads, exports what the header
declares, sizes the workspace as documented and rejects bad arguments before
touching the GPU (no valid compute call is made here)."""
import ctypes

import pytest

from headwise_chunked_attention_amd import api

OK, INVALID, UNSUPPORTED, WORKSPACE, ALIGN = 0, -1, -2, -3, -4


@pytest.fixture(scope="module")
def lib():
    return api.load()


def test_exports_every_header_symbol(lib):
    names = api.header_symbols()
    assert set(names) == {"upipe_attn_workspace_bytes", "upipe_choose_chunk_heads", "upipe_attn_fwd",
                          "upipe_attn_bwd", "upipe_strerror", "upipe_version", "upipe_profile_start",
                          "upipe_profile_stop", "upipe_mlp_workspace_bytes", "upipe_mlp_fwd", "upipe_mlp_bwd",
                          "upipe_loss_workspace_bytes", "upipe_loss_fwd", "upipe_loss_bwd",
                          "upipe_block_workspace_bytes", "upipe_block_fwd", "upipe_block_bwd",
                          "upipe_stack_workspace_bytes", "upipe_stack_fwd", "upipe_stack_bwd", "upipe_device_peak",
                          "upipe_attn_bwd_deterministic", "upipe_attn_fwd_noalloc"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.upipe_version() == 100
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, ALIGN, -5, -6):
        assert len(api.strerror(code)) > 5
    assert "unknown" in api.strerror(-99)


def _expected_ws(N, D, hq, hkv, d, C, norm, es, bwd):
    """The documented layout: per-chunk buffers of Np = ceil(N/256)*256 rows."""
    Np = (N + 255) // 256 * 256
    G = hq // hkv
    kvc = C // G if C > G else 1
    head = Np * d
    if not bwd:
        return head * es * (2 * C + 2 * kvc)
    t = head * es * (3 * C + 2 * kvc + (C + kvc if norm else 0))
    t += Np * C * 4 + head * 4 * (C + 2 * kvc)
    t += d * D * es * (2 * C + 2 * kvc)
    return t


@pytest.mark.parametrize("N,D,hq,hkv,d", [(2048, 512, 8, 2, 64), (131072, 4096, 4, 1, 128),
                                          (1000, 128, 4, 1, 128), (524288, 5120, 8, 1, 128)])
def test_workspace_formula(N, D, hq, hkv, d):
    G = hq // hkv
    for C in [c for c in (1, 2, 4, 8) if hq % c == 0 and (c % G == 0 or G % c == 0)]:
        for dt, es in (("fp32", 4), ("bf16", 2)):
            for norm in (False, True):
                for bwd in (False, True):
                    got = api.workspace_bytes(N, D, hq, hkv, d, C, norm, dt, bwd)
                    assert got == _expected_ws(N, D, hq, hkv, d, C, norm, es, bwd), (C, dt, norm, bwd)


def test_workspace_scales_with_chunk_not_heads():
    # forward per-q-head part = 2 * Np * d * es * C; at C=1 of 8 heads it is 1/8 of C=8
    f = {C: api.workspace_bytes(524288, 5120, 8, 1, 128, C, True, "bf16", False) for C in (1, 2, 4, 8)}
    kv_part = 2 * 524288 * 128 * 2
    per_q = {C: f[C] - kv_part for C in f}
    assert per_q[8] == 8 * per_q[1] and per_q[4] == 4 * per_q[1]
    assert 1 - per_q[1] / per_q[8] == pytest.approx(0.875)


def test_workspace_rejects_bad_shapes():
    assert api.workspace_bytes(100, 512, 8, 2, 96, 2, False, "bf16", False) == 0
    assert api.workspace_bytes(100, 500, 8, 2, 64, 2, False, "bf16", False) == 0
    assert api.workspace_bytes(100, 512, 8, 3, 64, 2, False, "bf16", False) == 0
    assert api.workspace_bytes(100, 512, 12, 2, 64, 4, False, "bf16", False) == 0
    assert api.workspace_bytes(0, 512, 8, 2, 64, 2, False, "bf16", False) == 0


# Fake, never-dereferenced device addresses: every call below must fail validation.
P = 1 << 20


def _fwd(lib, **kw):
    a = dict(dtype=1, N=256, D=512, hq=8, hkv=2, d=64, theta=5e5, C=2, x=P, wq=P, wk=P, wv=P, wo=P,
             qn=None, kn=None, eps=1e-6, y=P, lse=P, ws=P, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.upipe_attn_fwd(a["dtype"], a["N"], a["D"], a["hq"], a["hkv"], a["d"], a["theta"], a["C"],
                              a["x"], a["wq"], a["wk"], a["wv"], a["wo"], a["qn"], a["kn"], a["eps"],
                              a["y"], a["lse"], a["ws"], a["wsb"], a["stream"])


def _valid_chunks(hq, hkv):
    G = hq // hkv
    return [c for c in range(1, hq + 1) if hq % c == 0 and (c % G == 0 or G % c == 0)]


@pytest.mark.parametrize("N,D,hq,hkv,d,norm", [(2048, 512, 8, 2, 64, False), (131072, 4096, 4, 1, 128, False),
                                               (524288, 5120, 8, 1, 128, True), (1000, 128, 12, 3, 128, False),
                                               (4096, 256, 6, 6, 64, True)])
def test_chunk_chooser_picks_largest_fitting_chunk(N, D, hq, hkv, d, norm):
    # brute force over every accepted chunk size, each priced by the documented layout
    for dt, es in (("fp32", 4), ("bf16", 2)):
        for bwd in (False, True):
            sizes = {c: _expected_ws(N, D, hq, hkv, d, c, norm, es, bwd) for c in _valid_chunks(hq, hkv)}
            budgets = {0, min(sizes.values()) - 1, max(sizes.values()) * 10}
            for v in sizes.values():
                budgets |= {v - 1, v, v + 1}
            for b in sorted(x for x in budgets if x >= 0):
                fits = [c for c, v in sizes.items() if v <= b]
                if not fits:
                    with pytest.raises(api.UpipeError) as e:
                        api.choose_chunk_heads(N, D, hq, hkv, d, norm, dt, bwd, b)
                    assert e.value.code == WORKSPACE
                    continue
                c, ws = api.choose_chunk_heads(N, D, hq, hkv, d, norm, dt, bwd, b)
                assert (c, ws) == (max(fits), sizes[max(fits)]), (dt, bwd, b)


def test_chunk_chooser_at_the_llama_and_qwen_shares():
    gb = 10 ** 9
    # Llama3-8B share at 131072 tokens, backward 0.37 / 0.54 / 0.88 GB for C = 1 / 2 / 4
    assert api.choose_chunk_heads(131072, 4096, 4, 1, 128, False, "bf16", True, 0.5 * gb)[0] == 1
    assert api.choose_chunk_heads(131072, 4096, 4, 1, 128, False, "bf16", True, 0.6 * gb)[0] == 2
    assert api.choose_chunk_heads(131072, 4096, 4, 1, 128, False, "bf16", True, 288 * gb)[0] == 4
    # 5242880 tokens: the forward at C = 1 takes 5.37 GB, so a 5 GB budget fits nothing
    with pytest.raises(api.UpipeError):
        api.choose_chunk_heads(5242880, 4096, 4, 1, 128, False, "bf16", False, 5 * gb)
    # Qwen3-32B share at 524288 tokens with q/k norm: forward 0.54 / 0.81 / 1.34 / 2.42 GB
    assert api.choose_chunk_heads(524288, 5120, 8, 1, 128, True, "bf16", False, 2 * gb)[0] == 4


def test_chunk_chooser_reports_shape_errors(lib):
    ws = ctypes.c_size_t(12345)
    big = 1 << 62
    # (dtype, N, D, hq, hkv, d) -> the entry points' code
    for args, code in [((1, 0, 512, 8, 2, 64), INVALID), ((1, 2048, 512, 8, 3, 64), INVALID),
                       ((1, 2048, 512, 8, 2, 96), UNSUPPORTED), ((1, 2048, 500, 8, 2, 64), UNSUPPORTED),
                       ((7, 2048, 512, 8, 2, 64), INVALID)]:
        dt, N, D, hq, hkv, d = args
        rc = lib.upipe_choose_chunk_heads(N, D, hq, hkv, d, 0, dt, 1, big, ctypes.byref(ws))
        assert rc == code, args
        assert ws.value == 12345  # untouched on error
    # a NULL ws_bytes is allowed
    assert lib.upipe_choose_chunk_heads(2048, 512, 8, 2, 64, 0, 1, 1, big, None) == 8


def test_fwd_validation_errors(lib):
    assert _fwd(lib, d=96) == UNSUPPORTED
    assert _fwd(lib, D=500) == UNSUPPORTED
    assert _fwd(lib, C=3) == UNSUPPORTED
    assert _fwd(lib, hkv=3) == INVALID
    assert _fwd(lib, N=0) == INVALID
    assert _fwd(lib, dtype=7) == INVALID
    assert _fwd(lib, theta=0.0) == INVALID
    assert _fwd(lib, theta=float("nan")) == INVALID
    assert _fwd(lib, x=None) == INVALID
    assert _fwd(lib, lse=None) == INVALID
    assert _fwd(lib, qn=P) == INVALID            # q norm without k norm
    assert _fwd(lib, wq=P + 8) == ALIGN
    assert _fwd(lib, ws=None) == WORKSPACE
    assert _fwd(lib, ws=P + 128) == ALIGN
    need = api.workspace_bytes(256, 512, 8, 2, 64, 2, False, "bf16", False)
    assert _fwd(lib, wsb=need - 1) == WORKSPACE


def test_bwd_validation_errors(lib):
    def bwd(**kw):
        a = dict(dtype=0, N=256, D=512, hq=8, hkv=2, d=64, theta=5e5, C=2, qn=None, kn=None, dqn=None,
                 dkn=None, ws=P, wsb=1 << 40, dx=P)
        a.update(kw)
        return lib.upipe_attn_bwd(a["dtype"], a["N"], a["D"], a["hq"], a["hkv"], a["d"], a["theta"], a["C"],
                                  P, P, P, P, P, a["qn"], a["kn"], 1e-6, P, P, a["dx"], P, P, P, P,
                                  a["dqn"], a["dkn"], a["ws"], a["wsb"], None)
    assert bwd(d=32) == UNSUPPORTED
    assert bwd(dx=None) == INVALID
    assert bwd(qn=P, kn=P) == INVALID             # norm weights without their gradients
    assert bwd(dqn=P) == INVALID                  # gradients without norm weights
    need = api.workspace_bytes(256, 512, 8, 2, 64, 2, False, "fp32", True)
    assert bwd(wsb=need - 256) == WORKSPACE
    assert bwd(ws=P + 16) == ALIGN


def test_noalloc_fwd_validation_errors(lib):
    """The allocation-free forward checks like upipe_attn_fwd, and rejects a
    problem whose forward workspace exceeds its built-in scratch before any
    HIP call (so this runs without a GPU)."""
    def fwd(N=256, D=512, hq=8, hkv=2, d=64, C=2, x=P):
        return lib.upipe_attn_fwd_noalloc(1, N, D, hq, hkv, d, 5e5, C, x, P, P, P, P, None, None, 1e-6, P, P, None)
    assert fwd(d=96) == UNSUPPORTED
    assert fwd(x=None) == INVALID
    assert fwd(x=P + 8) == ALIGN
    scratch = 64 << 20
    for N, D, hq, hkv, d, C in ((70000, 128, 4, 1, 128, 1), (4096, 512, 64, 8, 128, 64), (1 << 20, 4096, 4, 1, 128, 1)):
        assert api.workspace_bytes(N, D, hq, hkv, d, C, False, "bf16", False) > scratch
        assert fwd(N, D, hq, hkv, d, C) == -6
    assert "scratch" in api.strerror(-6)


def test_profile_stop_without_launches_is_empty(lib):
    api.profile_start()
    res = api.profile_stop()
    assert set(res) == set(api.KERNEL_KINDS)
    assert all(v["launches"] == 0 and v["ms"] == 0.0 for v in res.values())


# ---------------------------------------------------------------------------
# sequence-tiled MLP
# ---------------------------------------------------------------------------
def _expected_mlp_ws(N, D, F, T, es, bwd):
    """The documented layout: tile buffers of min(T, N rounded up to 128) rows."""
    rows = min(T, (N + 127) // 128 * 128)
    tile = rows * F * es

    def r(b):
        return (b + 255) // 256 * 256
    total = r(tile)  # a
    if bwd:
        total += r(2 * tile) + r(tile) + r(tile)  # h|u, dh, du
        total += r(F * D * es) + r(2 * F * D * es)  # Wd^T, [Wg^T | Wu^T]
    return total


@pytest.mark.parametrize("N,D,F,T", [(300, 256, 384, 128), (1, 128, 128, 128), (16384, 4096, 14336, 4096),
                                     (100, 512, 1024, 4096), (5242880 // 8, 5120, 25600, 8192)])
def test_mlp_workspace_formula(N, D, F, T):
    for dt, es in (("fp32", 4), ("bf16", 2)):
        for bwd in (False, True):
            assert api.mlp_workspace_bytes(N, D, F, T, dt, bwd) == _expected_mlp_ws(N, D, F, T, es, bwd)


def test_mlp_workspace_scales_with_tile_not_tokens():
    # the tile buffers grow with tile_tokens; past one tile, N does not change them
    a = api.mlp_workspace_bytes(1 << 20, 4096, 14336, 4096, "bf16", True)
    b = api.mlp_workspace_bytes(1 << 22, 4096, 14336, 4096, "bf16", True)
    c = api.mlp_workspace_bytes(1 << 20, 4096, 14336, 8192, "bf16", True)
    assert a == b
    assert c - a == 5 * 4096 * 14336 * 2


def test_mlp_workspace_rejects_bad_shapes():
    assert api.mlp_workspace_bytes(0, 256, 384, 128, "bf16", False) == 0
    assert api.mlp_workspace_bytes(300, 250, 384, 128, "bf16", False) == 0
    assert api.mlp_workspace_bytes(300, 256, 320, 128, "bf16", False) == 0
    assert api.mlp_workspace_bytes(300, 256, 384, 100, "bf16", False) == 0
    assert api.mlp_workspace_bytes(300, 256, 384, 0, "bf16", False) == 0


def _mlp_fwd(lib, **kw):
    a = dict(dtype=1, N=300, D=256, F=384, T=128, x=P, wg=P, wu=P, wd=P, y=P, ws=P, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.upipe_mlp_fwd(a["dtype"], a["N"], a["D"], a["F"], a["T"], a["x"], a["wg"], a["wu"], a["wd"],
                             a["y"], a["ws"], a["wsb"], a["stream"])


def _mlp_bwd(lib, **kw):
    a = dict(dtype=0, N=300, D=256, F=384, T=128, x=P, wg=P, wu=P, wd=P, dy=P, dx=P, dwg=P, dwu=P, dwd=P, ws=P,
             wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.upipe_mlp_bwd(a["dtype"], a["N"], a["D"], a["F"], a["T"], a["x"], a["wg"], a["wu"], a["wd"],
                             a["dy"], a["dx"], a["dwg"], a["dwu"], a["dwd"], a["ws"], a["wsb"], a["stream"])


def test_mlp_fwd_validation_errors(lib):
    assert _mlp_fwd(lib, dtype=5) == INVALID
    assert _mlp_fwd(lib, N=0) == INVALID
    assert _mlp_fwd(lib, D=200) == UNSUPPORTED
    assert _mlp_fwd(lib, F=200) == UNSUPPORTED
    assert _mlp_fwd(lib, T=64) == UNSUPPORTED
    assert _mlp_fwd(lib, wu=None) == INVALID
    assert _mlp_fwd(lib, y=P + 2) == ALIGN
    need = api.mlp_workspace_bytes(300, 256, 384, 128, "bf16", False)
    assert _mlp_fwd(lib, wsb=need - 1) == WORKSPACE
    assert _mlp_fwd(lib, ws=None) == WORKSPACE
    assert _mlp_fwd(lib, ws=P + 16) == ALIGN


def test_mlp_bwd_validation_errors(lib):
    assert _mlp_bwd(lib, dwd=None) == INVALID
    assert _mlp_bwd(lib, dy=P + 4) == ALIGN
    assert _mlp_bwd(lib, F=0) == INVALID
    need = api.mlp_workspace_bytes(300, 256, 384, 128, "fp32", True)
    assert _mlp_bwd(lib, wsb=need - 256) == WORKSPACE


# ---------------------------------------------------------------------------
# sequence-tiled cross-entropy loss
# ---------------------------------------------------------------------------
def _expected_loss_ws(N, D, V, T, es, bwd):
    rows = min(T, (N + 127) // 128 * 128)

    def r(b):
        return (b + 255) // 256 * 256
    if not bwd:
        return r(rows * (V // 128) * 2 * 4) + r(rows * 4)
    return r(rows * V * es) + r(V * D * es)


@pytest.mark.parametrize("N,D,V,T", [(300, 256, 1024, 128), (1, 128, 128, 128), (16384, 4096, 128256, 1024),
                                     (100, 512, 151936, 4096)])
def test_loss_workspace_formula(N, D, V, T):
    for dt, es in (("fp32", 4), ("bf16", 2)):
        for bwd in (False, True):
            assert api.loss_workspace_bytes(N, D, V, T, dt, bwd) == _expected_loss_ws(N, D, V, T, es, bwd)
    # past one tile, N does not change the workspace
    assert api.loss_workspace_bytes(1 << 22, D, V, T, "bf16", True) == api.loss_workspace_bytes(1 << 20, D, V, T,
                                                                                                "bf16", True)


def test_loss_validation_errors(lib):
    def fwd(**kw):
        a = dict(dtype=1, N=300, D=256, V=1024, T=128, h=P, w=P, t=P, loss=P, lse=P, ws=P, wsb=1 << 40)
        a.update(kw)
        return lib.upipe_loss_fwd(a["dtype"], a["N"], a["D"], a["V"], a["T"], a["h"], a["w"], a["t"], a["loss"],
                                  a["lse"], a["ws"], a["wsb"], None)

    def bwd(**kw):
        a = dict(dtype=0, N=300, D=256, V=1024, T=128, h=P, w=P, t=P, lse=P, g=P, dh=P, dw=P, ws=P, wsb=1 << 40)
        a.update(kw)
        return lib.upipe_loss_bwd(a["dtype"], a["N"], a["D"], a["V"], a["T"], a["h"], a["w"], a["t"], a["lse"],
                                  a["g"], a["dh"], a["dw"], a["ws"], a["wsb"], None)

    assert fwd(dtype=3) == INVALID
    assert fwd(N=0) == INVALID
    assert fwd(V=1000) == UNSUPPORTED
    assert fwd(D=100) == UNSUPPORTED
    assert fwd(T=200) == UNSUPPORTED
    assert fwd(t=None) == INVALID
    assert fwd(lse=P + 4) == ALIGN
    assert fwd(wsb=api.loss_workspace_bytes(300, 256, 1024, 128, "bf16", False) - 1) == WORKSPACE
    assert bwd(g=None) == INVALID
    assert bwd(dw=P + 8) == ALIGN
    assert bwd(wsb=api.loss_workspace_bytes(300, 256, 1024, 128, "fp32", True) - 256) == WORKSPACE


# ---------------------------------------------------------------------------
# checkpointed transformer block
# ---------------------------------------------------------------------------
def _r256(b):
    return (b + 255) // 256 * 256


def _expected_block_ws(N, D, F, T, hq, hkv, d, C, norm, dt, es, bwd):
    rows = min(T, (N + 127) // 128 * 128)
    nd, td = _r256(N * D * es), _r256(rows * D * es)
    t = nd + td + _r256(hq * N * 4)
    if bwd:  # da, the db tile, and every head's O kept by the rerun forward
        t += nd + td + _r256(hq * ((N + 255) // 256 * 256) * d * es)
    stage = max(_expected_ws(N, D, hq, hkv, d, C, norm, es, False), _expected_mlp_ws(N, D, F, T, es, bwd))
    if bwd:
        stage = max(stage, _expected_ws(N, D, hq, hkv, d, C, norm, es, True))
    return t + _r256(stage)


@pytest.mark.parametrize("N,D,F,T,hq,hkv,d,C,norm", [(300, 256, 384, 128, 4, 2, 64, 2, False),
                                                    (131072, 4096, 14336, 4096, 4, 1, 128, 1, False),
                                                    (1000, 1024, 2816, 256, 8, 2, 128, 4, True)])
def test_block_workspace_formula(N, D, F, T, hq, hkv, d, C, norm):
    s = api.block_shape(N, D, F, T, hq, hkv, d, C, 5e5)
    for dt, es in (("fp32", 4), ("bf16", 2)):
        for bwd in (False, True):
            want = _expected_block_ws(N, D, F, T, hq, hkv, d, C, norm, dt, es, bwd)
            assert api.block_workspace_bytes(s, norm, dt, bwd) == want


def test_block_workspace_rejects_bad_shapes():
    good = dict(n_tokens=300, d_model=256, d_ff=384, tile_tokens=128, n_q_heads=4, n_kv_heads=2, head_dim=64,
                chunk_heads=2, rope_theta=1e4)
    assert api.block_workspace_bytes(api.block_shape(**good), False, "bf16", True) > 0
    for k, v in (("n_tokens", 0), ("d_model", 200), ("d_ff", 200), ("tile_tokens", 64), ("head_dim", 96),
                 ("chunk_heads", 3), ("n_kv_heads", 3), ("rope_theta", 0.0), ("d_model", 8192 + 128)):
        bad = dict(good, **{k: v})
        assert api.block_workspace_bytes(api.block_shape(**bad), False, "bf16", True) == 0, k
    assert api.block_workspace_bytes(api.block_shape(**good, norm_eps=-1.0), False, "bf16", False) == 0
    # d_model 8192 (the largest the row norm takes) is accepted
    assert api.block_workspace_bytes(api.block_shape(**dict(good, d_model=8192)), False, "fp32", True) > 0


def _block_call(lib, bwd=False, shape=None, weights=None, grads=None, **kw):
    s = shape or api.block_shape(300, 256, 384, 128, 4, 2, 64, 2, 1e4)
    w = weights or api.BlockWeights(**{n: P for n in api._BLOCK_TENSORS if n not in ("q_norm", "k_norm")})
    a = dict(dtype=1, x=P, y=P, h=None, lse=None, dy=P, dx=P, ws=P, wsb=1 << 40)
    a.update(kw)
    if not bwd:
        return lib.upipe_block_fwd(a["dtype"], ctypes.byref(s), a["x"], ctypes.byref(w), a["y"], a["h"], a["lse"],
                                   a["ws"], a["wsb"], None)
    g = grads or api.BlockGrads(**{n: P for n in api._BLOCK_TENSORS if n not in ("q_norm", "k_norm")})
    return lib.upipe_block_bwd(a["dtype"], ctypes.byref(s), a["x"], ctypes.byref(w), a["h"], a["lse"], a["dy"],
                               a["dx"], ctypes.byref(g), a["ws"], a["wsb"], None)


def test_block_validation_errors(lib):
    full = {n: P for n in api._BLOCK_TENSORS if n not in ("q_norm", "k_norm")}
    assert _block_call(lib, dtype=7) == INVALID
    assert _block_call(lib, x=None) == INVALID
    assert _block_call(lib, y=P + 2) == ALIGN
    assert _block_call(lib, h=P + 8) == ALIGN
    assert _block_call(lib, shape=api.block_shape(300, 256, 384, 100, 4, 2, 64, 2, 1e4)) == UNSUPPORTED
    assert _block_call(lib, shape=api.block_shape(300, 256, 384, 128, 4, 2, 64, 3, 1e4)) == UNSUPPORTED
    assert _block_call(lib, shape=api.block_shape(0, 256, 384, 128, 4, 2, 64, 2, 1e4)) == INVALID
    assert _block_call(lib, weights=api.BlockWeights(**dict(full, w_up=None))) == INVALID
    assert _block_call(lib, weights=api.BlockWeights(**dict(full, q_norm=P))) == INVALID  # k_norm missing
    assert _block_call(lib, weights=api.BlockWeights(**dict(full, mlp_norm=P + 4))) == ALIGN
    need = api.block_workspace_bytes(api.block_shape(300, 256, 384, 128, 4, 2, 64, 2, 1e4), False, "bf16", False)
    assert _block_call(lib, wsb=need - 1) == WORKSPACE
    assert _block_call(lib, ws=None) == WORKSPACE
    assert _block_call(lib, ws=P + 16) == ALIGN
    # backward: h_mid and lse together, gradients complete, q/k norm grads only with q/k norm
    assert _block_call(lib, bwd=True, h=P) == INVALID
    assert _block_call(lib, bwd=True, lse=P) == INVALID
    assert _block_call(lib, bwd=True, dy=None) == INVALID
    assert _block_call(lib, bwd=True, grads=api.BlockGrads(**dict(full, wo=None))) == INVALID
    assert _block_call(lib, bwd=True, grads=api.BlockGrads(**dict(full, q_norm=P, k_norm=P))) == INVALID
    assert _block_call(lib, bwd=True, grads=api.BlockGrads(**dict(full, w_down=P + 4))) == ALIGN
    need = api.block_workspace_bytes(api.block_shape(300, 256, 384, 128, 4, 2, 64, 2, 1e4), False, "bf16", True)
    assert _block_call(lib, bwd=True, wsb=need - 256) == WORKSPACE


# ---------------------------------------------------------------------------
# stack of blocks with offloaded inputs
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,D,F,T,hq,hkv,d,C", [(300, 256, 384, 128, 4, 2, 64, 2),
                                               (32768, 4096, 14336, 4096, 32, 8, 128, 4)])
def test_stack_workspace_formula(N, D, F, T, hq, hkv, d, C):
    s = api.block_shape(N, D, F, T, hq, hkv, d, C, 5e5)
    for dt, es in (("fp32", 4), ("bf16", 2)):
        blk = max(api.block_workspace_bytes(s, False, dt, False), api.block_workspace_bytes(s, False, dt, True))
        assert api.stack_workspace_bytes(s, False, dt) == 4 * _r256(N * D * es) + blk
    assert api.stack_workspace_bytes(api.block_shape(N, 200, F, T, hq, hkv, d, C, 5e5), False, "bf16") == 0


def test_stack_validation_errors(lib):
    s = api.block_shape(300, 256, 384, 128, 4, 2, 64, 2, 1e4)
    full = {n: P for n in api._BLOCK_TENSORS if n not in ("q_norm", "k_norm")}
    need = api.stack_workspace_bytes(s, False, "bf16")

    def fwd(L=3, layers=None, x=P, y=P, host=P, ws=P, wsb=need, dtype=1):
        w = (api.BlockWeights * max(L, 1))(*(layers or [api.BlockWeights(**full)] * max(L, 1)))
        return lib.upipe_stack_fwd(dtype, ctypes.byref(s), L, w, x, y, host, ws, wsb, None, None)

    def bwd(L=3, grads=None, host=P, dy=P, dx=P, wsb=need):
        w = (api.BlockWeights * L)(*[api.BlockWeights(**full)] * L)
        g = (api.BlockGrads * L)(*(grads or [api.BlockGrads(**full)] * L))
        return lib.upipe_stack_bwd(1, ctypes.byref(s), L, w, host, dy, dx, g, P, wsb, None, None)

    assert fwd(L=0) == INVALID
    assert fwd(dtype=9) == INVALID
    # a bad weight in the last layer is found before anything is enqueued
    bad = [api.BlockWeights(**full), api.BlockWeights(**full), api.BlockWeights(**dict(full, w_down=None))]
    assert fwd(layers=bad) == INVALID
    mixed = [api.BlockWeights(**full), api.BlockWeights(**dict(full, q_norm=P, k_norm=P)), api.BlockWeights(**full)]
    assert fwd(layers=mixed) == INVALID
    assert fwd(host=None) == INVALID
    assert fwd(host=P + 8) == ALIGN
    assert fwd(y=None) == INVALID
    assert fwd(wsb=need - 256) == WORKSPACE
    assert fwd(ws=None) == WORKSPACE
    assert bwd(grads=[api.BlockGrads(**full), api.BlockGrads(**dict(full, wq=None)), api.BlockGrads(**full)]) \
        == INVALID
    assert bwd(host=None) == INVALID
    assert bwd(dx=P + 2) == ALIGN
    assert bwd(wsb=need - 1) == WORKSPACE
