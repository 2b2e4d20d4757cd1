"""GPU parity of the stack of checkpointed blocks whose inputs are offloaded
to pinned host memory (through the C ABI).

- Against the fp64 oracle (``oracle.stack_fwd`` / ``stack_bwd``): y, dx and
  every layer's weight and norm gradients, relative L2 <= 1e-5 (fp32) and
  <= 2e-2 (bf16); the host copies of the block inputs against the oracle's
  block inputs.
- Against the same blocks run one by one with device-resident inputs
  (``upipe_block_fwd`` / ``upipe_block_bwd``): the offload moves data only,
  so y and the host copies are bitwise equal; the gradients agree to fp32
  rounding (the weight gradients add split partial sums atomically, in no
  fixed order).
- With and without a separate copy stream, and a stack of one block.
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
ATTR = {"attn_norm": "g_attn", "wq": "wq", "wk": "wk", "wv": "wv", "wo": "wo", "q_norm": "q_norm",
        "k_norm": "k_norm", "mlp_norm": "g_mlp", "w_gate": "wg", "w_up": "wu", "w_down": "wd"}
ORACLE_KEYS = ("g_attn", "wq", "wk", "wv", "wo", "q_norm", "k_norm", "g_mlp", "wg", "wu", "wd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _problem(L, N, D, F, hq, hkv, d, dt, seed):
    # layer i takes the weights of seed + i; x and dy come from layer 0's draw
    inps = [BlockInputs(N, D, F, hq, hkv, d, dt, seed=seed + i, with_x=(i == 0), with_dy=(i == 0))
            for i in range(L)]
    layers_dev = [{n: dev(getattr(p, a), dt) for n, a in ATTR.items() if getattr(p, a) is not None} for p in inps]
    layers_ref = [{k: getattr(p, k) for k in ORACLE_KEYS} for p in inps]
    return inps[0].x, inps[0].dy, layers_dev, layers_ref


def _run_stack(x, dy, layers, shape, copy_stream):
    L = len(layers)
    hin = torch.empty((L,) + tuple(x.shape), dtype=x.dtype, pin_memory=True)
    y = api.stack_fwd(x, layers, shape, hin, copy_stream=copy_stream)
    dx, grads = api.stack_bwd(layers, shape, hin, dy, copy_stream=copy_stream)
    torch.cuda.synchronize()
    return y, hin, dx, grads


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_stack_matches_oracle_and_unoffloaded_blocks(dt):
    L, N, D, F, T, hq, hkv, d, C = 3, 300, 256, 384, 128, 4, 2, 64, 2
    print(f"stack case L={L} N={N} D={D} F={F} tile={T} {dt}", flush=True)
    x_h, dy_h, layers, layers_ref = _problem(L, N, D, F, hq, hkv, d, dt, seed=3)
    x, dy = dev(x_h, dt), dev(dy_h, dt)
    shape = api.block_shape(N, D, F, T, hq, hkv, d, C, THETA, EPS, QK_EPS)
    side = torch.cuda.Stream()
    y, hin, dx, grads = _run_stack(x, dy, layers, shape, side)

    # the same blocks one by one, inputs kept on the device
    acts = [x]
    for w in layers:
        acts.append(api.block_fwd(acts[-1], w, shape)[0])
    g = dy
    ref_grads = [None] * L
    for i in range(L - 1, -1, -1):
        g, ref_grads[i] = api.block_bwd(acts[i], layers[i], shape, g)
    torch.cuda.synchronize()
    assert torch.equal(y, acts[-1])
    for i in range(L):
        assert torch.equal(hin[i].to("cuda"), acts[i]), i
    e = relerr(host(dx), host(g))
    assert e <= 1e-6, e
    for i in range(L):
        for n in grads[i]:
            assert relerr(host(grads[i][n]), host(ref_grads[i][n])) <= 1e-6, (i, n)

    # the oracle
    y_ref, inputs_ref = oracle.stack_fwd(x_h, layers_ref, hq, hkv, d, THETA, C, QK_EPS, EPS)
    dx_ref, g_ref = oracle.stack_bwd(x_h, layers_ref, dy_h, hq, hkv, d, THETA, C, QK_EPS, EPS)
    errs = {"y": relerr(host(y), y_ref), "dx": relerr(host(dx), dx_ref)}
    for i in range(L):
        errs[f"in{i}"] = relerr(hin[i].double().numpy(), inputs_ref[i])
        for n, a in ATTR.items():
            if n in grads[i]:
                errs[f"{i}.d{n}"] = relerr(host(grads[i][n]), g_ref[i][a])
    print("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[dt]}
    assert not bad, bad


def test_stack_single_stream_and_one_layer():
    N, D, F, T, hq, hkv, d, C = 129, 128, 256, 128, 2, 1, 64, 1
    for L in (1, 2):
        print(f"stack case L={L} N={N} fp32, copy stream and single stream", flush=True)
        x_h, dy_h, layers, layers_ref = _problem(L, N, D, F, hq, hkv, d, "fp32", seed=11)
        x, dy = dev(x_h, "fp32"), dev(dy_h, "fp32")
        shape = api.block_shape(N, D, F, T, hq, hkv, d, C, THETA, EPS, QK_EPS)
        y1, h1, dx1, g1 = _run_stack(x, dy, layers, shape, torch.cuda.Stream())
        y2, h2, dx2, g2 = _run_stack(x, dy, layers, shape, None)
        assert torch.equal(y1, y2) and torch.equal(h1, h2)
        assert relerr(host(dx1), host(dx2)) <= 1e-6
        dx_ref, _ = oracle.stack_bwd(x_h, layers_ref, dy_h, hq, hkv, d, THETA, C, QK_EPS, EPS)
        y_ref, _ = oracle.stack_fwd(x_h, layers_ref, hq, hkv, d, THETA, C, QK_EPS, EPS)
        assert relerr(host(y1), y_ref) <= TOL["fp32"] and relerr(host(dx1), dx_ref) <= TOL["fp32"]
