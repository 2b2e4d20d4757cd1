"""Benchmark: fwd+bwd of the headwise-chunked attention layer on one MI355X.

One "step" is one forward plus one backward of the whole hot path (every
chunk: projections, RoPE, causal GQA attention, output projection, and the
backward with its recompute) over the Llama3-8B one-GPU Ulysses share at
N = 1048576 tokens: d_model 4096, 4 q heads / 1 kv head, head_dim 128, bf16,
RoPE theta 5e5, causal; inputs x ~ N(0,1), W ~ N(0, 0.02), dY ~ N(0,1),
seeded, generated on the host and resident in HBM before timing starts.

Printed (one JSON line): model TFLOP/s of the step at the headline chunk size
(chunk_heads=1 unless --chunk is given) and its fraction of the bf16 dense
MFMA peak; median and minimum step, forward and backward times; the
attention-core and hardware (recompute included) rates; the workspace bytes
per chunk size; a chunk-size sweep over {1, 2, 4} with the peak workspace of
each; per-kernel event timings (from a second, profiled run of two steps);
the roofline entry of the dominant kernel; the CPU fp64 oracle timed on
bounded samples; the same measurements at N = 131072 (``secondary``); and the
sequence-tiled MLP and LM-head loss next to the op (``mlp``, ``loss``), one
checkpointed transformer block built from them (``block``), and four such
blocks with their inputs offloaded to host memory (``stack``).

  python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--chunk 1] [--no-sweep] [--no-cpu]
                  [--workload llama3-8b-ulysses-share-5m | qwen3-32b-ulysses-share-512k | ...]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
METRIC = "causal attn fwd+bwd TFLOP/s (frac of bf16 MFMA peak) + peak workspace GB vs chunk"

LLAMA = dict(d_model=4096, n_q_heads=4, n_kv_heads=1, head_dim=128, rope_theta=5e5, dtype="bf16", chunks=(1, 2, 4))
WORKLOADS = {
    "llama3-8b-ulysses-share-1m": dict(LLAMA, n_tokens=1048576),
    "llama3-8b-ulysses-share-131k": dict(LLAMA, n_tokens=131072),
    # the other two large configurations, on request (--workload): the 5M-token
    # share (one step takes minutes) and the Qwen3-32B-shaped share with q/k
    # RMSNorm
    "llama3-8b-ulysses-share-5m": dict(LLAMA, n_tokens=5242880, chunks=(1,)),
    "qwen3-32b-ulysses-share-512k": dict(d_model=5120, n_q_heads=8, n_kv_heads=1, head_dim=128, rope_theta=1e6,
                                         dtype="bf16", chunks=(1, 2, 4, 8), n_tokens=524288, qk_norm=True),
}
HEADLINE = "llama3-8b-ulysses-share-1m"
SECONDARY = "llama3-8b-ulysses-share-131k"
QWEN_SHAPE = dict(d_model=5120, n_q_heads=8, n_kv_heads=1, head_dim=128, rope_theta=1e6, n_tokens=524288)

KERNEL_NAMES = {"attn_fwd": "attn_fwd_kernel<bf16,128,0>", "attn_recompute": "attn_fwd_kernel<bf16,128,1>",
                "attn_bwd_dkdv": "attn_bwd_dkdv_kernel<bf16,128>", "attn_bwd_dq": "attn_bwd_dq_kernel<bf16,128>"}

# HBM bytes per launch (FETCH_SIZE + WRITE_SIZE from rocprofv3, each scaled by
# the same counter's reading for a plain copy of known size), per workload and
# kernel kind, as measured on the kernel as it now stands. A kernel change
# removes its entries until they are measured again; a workload without an
# entry reports null.
TRAFFIC_BYTES = {
    # profiles/attn_llama1m_hbm_traffic.md: fetch 666.965 GB + write 1.074 GB
    ("llama3-8b-ulysses-share-1m", "attn_bwd_dkdv"): 668.04e9,
    # profiles/attn_llama131k_hbm_traffic.md: fetch 5.314 GB + write 0.135 GB
    ("llama3-8b-ulysses-share-131k", "attn_bwd_dkdv"): 5.449e9,
}


def model_flops(N, D, hq, hkv, d):
    """Algorithmic fwd+bwd flops: attention core 14*d per visible pair per q head
    (fwd QK^T + PV = 4d, bwd S, dP, dV, dK, dQ = 10d) plus the four projections
    (fwd 2*N*D*d per head for q, k, v, o; bwd twice that)."""
    pairs = N * (N + 1) / 2
    return 14.0 * d * hq * pairs + 12.0 * N * D * d * (hq + hkv)


def attn_core_flops(N, hq, d):
    """The attention-core part of model_flops: 14*d per visible (query, key) pair per q head."""
    return 14.0 * d * hq * N * (N + 1) / 2


def hardware_flops(N, D, hq, hkv, d):
    """Flops the step actually executes: model flops plus the backward's recompute
    of O from the saved LSE (4*d per pair per q head) and of the projections
    (2*N*D*d per q head and per k/v head)."""
    pairs = N * (N + 1) / 2
    return model_flops(N, D, hq, hkv, d) + 4.0 * d * hq * pairs + 2.0 * N * D * d * (hq + 2 * hkv)


def cpu_baseline(w, sample_n=8192):
    """The oracle, as it stands, timed on this host's cores (all of them in this
    process's affinity mask; the BLAS thread pool is set to that count).

    ``value``: model TFLOP/s of the oracle's full fp64 fwd+bwd at sample_n
    tokens with the workload's d_model, heads and head_dim. ``rows`` adds:
    the tiny fp32 configuration in full; the same sample at the Qwen3-32B
    share's shape; each projected to its configuration's N by model flops
    (labelled "projected"); and the oracle work that the parity tests run at
    the workload's N (y and LSE at 256 sampled rows, dx at 64 tail rows)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from headwise_chunked_attention_amd.synth import LayerInputs, gen_rows, gen_rows_at

    cores = len(os.sched_getaffinity(0))
    rows = []
    with threadpool_limits(limits=cores):
        def full(N, D, hq, hkv, d, theta, dt, C, label, proj_n=None):
            inp = LayerInputs(N, D, hq, hkv, d, dt, seed=0)
            t0 = time.perf_counter()
            oracle.layer_fwd(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, hq, hkv, d, theta, C)
            oracle.layer_bwd(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, inp.dy, hq, hkv, d, theta, C)
            dt_s = time.perf_counter() - t0
            fl = model_flops(N, D, hq, hkv, d)
            r = {"sample": label, "seconds": dt_s, "model_tflops": fl / dt_s / 1e12}
            if proj_n:
                r["projected_seconds_at_n"] = {"n_tokens": proj_n, "seconds": dt_s * model_flops(proj_n, D, hq, hkv, d) / fl,
                                               "label": "projected"}
            rows.append(r)
            return r

        main = full(sample_n, w["d_model"], w["n_q_heads"], w["n_kv_heads"], w["head_dim"], w["rope_theta"], "bf16",
                    1, f"full fp64 fwd+bwd at N={sample_n}, the workload's layer shape", w["n_tokens"])
        full(2048, 512, 8, 2, 64, 5e5, "fp32", 2, "tiny fp32 configuration, full fp64 fwd+bwd (N=2048)")
        q = QWEN_SHAPE
        full(sample_n, q["d_model"], q["n_q_heads"], q["n_kv_heads"], q["head_dim"], q["rope_theta"], "bf16", 1,
             f"full fp64 fwd+bwd at N={sample_n}, Qwen3-32B share shape (q/k norm off)", q["n_tokens"])
        # the parity tests' own oracle work at the workload's N
        N, D = w["n_tokens"], w["d_model"]
        hq, hkv, d, th = w["n_q_heads"], w["n_kv_heads"], w["head_dim"], w["rope_theta"]
        wts = LayerInputs(8, D, hq, hkv, d, "bf16", seed=0, with_x=False, with_dy=False)
        xr = lambda a, b: gen_rows("x", N, D, 1.0, "bf16", 0, a, b)  # noqa: E731
        sel = np.unique(np.concatenate([[0, 1, N - 1], np.random.default_rng(0).integers(0, N, 253)]))
        t0 = time.perf_counter()
        oracle.layer_fwd_rows(xr, lambda i: gen_rows_at("x", N, D, 1.0, "bf16", 0, np.asarray(i)), N, sel, wts.wq,
                              wts.wk, wts.wv, wts.wo, hq, hkv, d, th)
        rows.append({"sample": f"sampled-row forward at N={N}: y and LSE at {sel.size} rows (K/V of all N "
                               f"tokens, x regenerated on the host)", "seconds": time.perf_counter() - t0})
    return {"value": main["model_tflops"], "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"full fp64 fwd+bwd (layer_fwd + layer_bwd, which recomputes the fwd) at N={sample_n} "
                      f"with the workload's d_model/heads/head_dim, chunk_heads=1; {main['seconds']:.1f} s; "
                      f"rate = model flops of that sample / time; BLAS threads = cores",
            "rows": rows}


def tiny_gpu_seconds(dev, reps=10, warmup=3):
    """Median fwd+bwd seconds of the tiny fp32 configuration (N 2048, d_model
    512, 8 q / 2 kv heads, head_dim 64, chunk_heads 2) on the GPU, inputs
    resident: the GPU side of the oracle's tiny-configuration row."""
    import numpy as np
    import torch

    from headwise_chunked_attention_amd import api
    from headwise_chunked_attention_amd.synth import LayerInputs

    inp = LayerInputs(2048, 512, 8, 2, 64, "fp32", seed=0)
    t = {k: torch.from_numpy(getattr(inp, k)).to(dev) for k in ("x", "wq", "wk", "wv", "wo", "dy")}
    kw = dict(n_q_heads=8, n_kv_heads=2, head_dim=64, rope_theta=5e5, chunk_heads=2)
    ws = api.alloc_workspace(max(api.workspace_bytes(2048, 512, 8, 2, 64, 2, False, "fp32", b) for b in (False, True)),
                             dev)
    times = []
    for i in range(warmup + reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        y, lse = api.attn_fwd(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], workspace=ws, **kw)
        api.attn_bwd(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], t["dy"], lse, workspace=ws, **kw)
        e1.record()
        e1.synchronize()
        if i >= warmup:
            times.append(e0.elapsed_time(e1) * 1e-3)
    return float(np.median(times))


MLP_WORKLOAD = dict(name="llama3-8b-mlp-seq-shard-16k", n_tokens=16384, d_model=4096, d_ff=14336,
                    tile_tokens=4096, dtype="bf16")


def mlp_bench(dev, steps, warmup):
    """The sequence-tiled gated-SiLU MLP on one GPU's sequence shard of the same
    131072-token Llama3-8B run (131072 / 8 tokens, d_model 4096, d_ff 14336),
    tile_tokens 4096, bf16: forward and backward times, model TFLOP/s
    (18 N D F: three GEMMs forward, six backward), the per-kind kernel table
    and the tiled vs untiled workspace."""
    import numpy as np
    import torch

    from headwise_chunked_attention_amd import api
    from headwise_chunked_attention_amd.synth import MlpInputs

    w = MLP_WORKLOAD
    N, D, F, T = w["n_tokens"], w["d_model"], w["d_ff"], w["tile_tokens"]
    inp = MlpInputs(N, D, F, "bf16", seed=0)
    t = {k: torch.from_numpy(getattr(inp, k)).to(dev).to(torch.bfloat16) for k in ("x", "dy", "wg", "wu", "wd")}
    del inp
    ws = api.alloc_workspace(api.mlp_workspace_bytes(N, D, F, T, "bf16", True), dev)
    y = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
    f32 = torch.float32
    out = (torch.empty((N, D), dtype=torch.bfloat16, device=dev), torch.empty((F, D), dtype=f32, device=dev),
           torch.empty((F, D), dtype=f32, device=dev), torch.empty((D, F), dtype=f32, device=dev))
    stream = torch.cuda.current_stream(dev)

    def fwd():
        api.mlp_fwd(t["x"], t["wg"], t["wu"], t["wd"], tile_tokens=T, y=y, workspace=ws)

    def bwd():
        api.mlp_bwd(t["x"], t["wg"], t["wu"], t["wd"], t["dy"], tile_tokens=T, out=out, workspace=ws)

    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        e[0].record(stream)
        fwd()
        e[1].record(stream)
        bwd()
        e[2].record(stream)
    torch.cuda.synchronize()
    t_f = [e[0].elapsed_time(e[1]) for e in evs]
    t_b = [e[1].elapsed_time(e[2]) for e in evs]
    api.profile_start()
    fwd()
    bwd()
    prof = api.profile_stop()
    model = 18.0 * N * D * F
    step_ms = float(np.median([a + b for a, b in zip(t_f, t_b)]))
    kinds = {k: {"ms": v["ms"], "launches": v["launches"],
                 "tflops": (v["flops"] / (v["ms"] * 1e-3) / 1e12) if v["flops"] else None}
             for k, v in prof.items() if v["launches"]}
    g = prof["mlp_gemm"]
    achieved = g["flops"] / (g["ms"] * 1e-3) / 1e12
    es = 2
    return {"workload": w["name"], "n_tokens": N, "d_model": D, "d_ff": F, "tile_tokens": T, "dtype": "bf16",
            "fwd_ms": float(np.median(t_f)), "bwd_ms": float(np.median(t_b)), "step_ms": step_ms,
            "model_tflops": model / (step_ms * 1e-3) / 1e12, "model_flops": model,
            "kernels": kinds,
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                         "kernel": "gemm_nt_kernel (gated-SiLU, store epilogues)"},
            "workspace_gb": {"tiled_bwd": api.mlp_workspace_bytes(N, D, F, T, "bf16", True) / 1e9,
                             "untiled_intermediates": 5 * N * F * es / 1e9}}


BLOCK_WORKLOAD = dict(name="llama3-8b-block-one-gpu-32k", n_tokens=32768, d_model=4096, d_ff=14336,
                      n_q_heads=32, n_kv_heads=8, head_dim=128, chunk_heads=4, tile_tokens=4096, rope_theta=5e5,
                      dtype="bf16")


def block_bench(dev, steps, warmup):
    """One checkpointed pre-norm Llama3-8B block with every head on one GPU
    (no context parallelism) at 32768 tokens: 32 q / 8 kv heads of 128 in
    chunks of 4 q heads (one kv group per chunk), MLP tile 4096, bf16. A
    step is upipe_block_fwd (nothing kept) plus upipe_block_bwd from the
    block input alone (norm and attention forward recomputed). Also timed:
    the backward when the forward kept h and lse. Model flops: the attention
    layer's (as in the headline step) plus 18 N D F for the MLP."""
    import numpy as np
    import torch

    from headwise_chunked_attention_amd import api
    from headwise_chunked_attention_amd.synth import BlockInputs

    w = BLOCK_WORKLOAD
    N, D, F, T = w["n_tokens"], w["d_model"], w["d_ff"], w["tile_tokens"]
    hq, hkv, d, C = w["n_q_heads"], w["n_kv_heads"], w["head_dim"], w["chunk_heads"]
    inp = BlockInputs(N, D, F, hq, hkv, d, "bf16", seed=0)
    names = {"attn_norm": "g_attn", "wq": "wq", "wk": "wk", "wv": "wv", "wo": "wo", "mlp_norm": "g_mlp",
             "w_gate": "wg", "w_up": "wu", "w_down": "wd"}
    wt = {n: torch.from_numpy(getattr(inp, a)).to(dev).to(torch.bfloat16) for n, a in names.items()}
    x = torch.from_numpy(inp.x).to(dev).to(torch.bfloat16)
    dy = torch.from_numpy(inp.dy).to(dev).to(torch.bfloat16)
    del inp
    shape = api.block_shape(N, D, F, T, hq, hkv, d, C, w["rope_theta"])
    ws_f = api.block_workspace_bytes(shape, False, "bf16", False)
    ws_b = api.block_workspace_bytes(shape, False, "bf16", True)
    ws = api.alloc_workspace(max(ws_f, ws_b), dev)
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    grads = {n: torch.empty(t.shape, dtype=torch.float32, device=dev) for n, t in wt.items()}
    h_mid = torch.empty_like(x)
    lse = torch.empty((hq, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def fwd():
        api.block_fwd(x, wt, shape, y=y, workspace=ws)

    def bwd():
        api.block_bwd(x, wt, shape, dy, dx=dx, grads=grads, workspace=ws)

    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        e[0].record(stream)
        fwd()
        e[1].record(stream)
        bwd()
        e[2].record(stream)
    # backward from the kept residual and lse
    api.block_fwd(x, wt, shape, y=y, h_mid=h_mid, lse=lse, workspace=ws)
    ek = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ek[0].record(stream)
    api.block_bwd(x, wt, shape, dy, h_mid=h_mid, lse=lse, dx=dx, grads=grads, workspace=ws)
    ek[1].record(stream)
    torch.cuda.synchronize()
    t_f = [e[0].elapsed_time(e[1]) for e in evs]
    t_b = [e[1].elapsed_time(e[2]) for e in evs]
    api.profile_start()
    fwd()
    bwd()
    prof = api.profile_stop()
    attn_fwd_model = 2.0 * d * hq * N * (N + 1) + 4.0 * N * D * d * (hq + hkv)
    model = model_flops(N, D, hq, hkv, d) + 18.0 * N * D * F
    # recomputed in the backward: the attention forward (which keeps O for
    # the attention backward) and the MLP's h|u
    hw = model + attn_fwd_model + 4.0 * N * D * F
    step_ms = float(np.median([a + b for a, b in zip(t_f, t_b)]))
    kinds = {k: {"ms": v["ms"], "launches": v["launches"],
                 "tflops": (v["flops"] / (v["ms"] * 1e-3) / 1e12) if v["flops"] else None}
             for k, v in prof.items() if v["launches"]}
    return {"workload": w["name"], "n_tokens": N, "d_model": D, "d_ff": F, "n_q_heads": hq, "n_kv_heads": hkv,
            "head_dim": d, "chunk_heads": C, "tile_tokens": T, "dtype": "bf16",
            "fwd_ms": float(np.median(t_f)), "bwd_ms": float(np.median(t_b)), "step_ms": step_ms,
            "bwd_kept_ms": ek[0].elapsed_time(ek[1]),
            "model_tflops": model / (step_ms * 1e-3) / 1e12, "model_flops": model,
            "hardware_tflops": hw / (step_ms * 1e-3) / 1e12,
            "kernels": kinds,
            "memory_gb": {"saved_per_block": N * D * 2 / 1e9, "saved_with_h_and_lse": (2 * N * D * 2 + hq * N * 4) / 1e9,
                          "workspace_fwd": ws_f / 1e9, "workspace_bwd": ws_b / 1e9}}


STACK_LAYERS = 4


def stack_bench(dev, steps):
    """Four of the blocks above, stacked, with each block's input offloaded to
    pinned host memory between the passes (upipe_stack_fwd/bwd, copies on a
    second stream), against the same four blocks run one by one with their
    inputs kept in HBM. The layers share one set of weights (the time does not
    depend on the values). Reports both step times, the offload's overhead,
    the HBM the offload frees and the host link rate of one input copy."""
    import numpy as np
    import torch

    from headwise_chunked_attention_amd import api
    from headwise_chunked_attention_amd.synth import BlockInputs

    w = BLOCK_WORKLOAD
    L = STACK_LAYERS
    N, D, F, T = w["n_tokens"], w["d_model"], w["d_ff"], w["tile_tokens"]
    hq, hkv, d, C = w["n_q_heads"], w["n_kv_heads"], w["head_dim"], w["chunk_heads"]
    inp = BlockInputs(N, D, F, hq, hkv, d, "bf16", seed=1)
    names = {"attn_norm": "g_attn", "wq": "wq", "wk": "wk", "wv": "wv", "wo": "wo", "mlp_norm": "g_mlp",
             "w_gate": "wg", "w_up": "wu", "w_down": "wd"}
    wt = {n: torch.from_numpy(getattr(inp, a)).to(dev).to(torch.bfloat16) for n, a in names.items()}
    x = torch.from_numpy(inp.x).to(dev).to(torch.bfloat16)
    dy = torch.from_numpy(inp.dy).to(dev).to(torch.bfloat16)
    del inp
    layers = [wt] * L
    grads = [{n: torch.empty(t.shape, dtype=torch.float32, device=dev) for n, t in wt.items()} for _ in range(L)]
    shape = api.block_shape(N, D, F, T, hq, hkv, d, C, w["rope_theta"])
    ws = api.alloc_workspace(api.stack_workspace_bytes(shape, False, "bf16"), dev)
    hin = torch.empty((L, N, D), dtype=torch.bfloat16, pin_memory=True)
    side = torch.cuda.Stream(device=dev)
    stream = torch.cuda.current_stream(dev)
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    acts = [torch.empty_like(x) for _ in range(L)]  # the unoffloaded run's kept inputs

    def offloaded():
        api.stack_fwd(x, layers, shape, hin, y=y, workspace=ws, copy_stream=side)
        api.stack_bwd(layers, shape, hin, dy, dx=dx, grads=grads, workspace=ws, copy_stream=side)

    def resident():
        a = x
        for i in range(L):
            out = acts[i] if i < L - 1 else y
            api.block_fwd(a, layers[i], shape, y=out, workspace=ws)
            a = out
        g = dy
        for i in range(L - 1, -1, -1):
            src = x if i == 0 else acts[i - 1]
            g, _ = api.block_bwd(src, layers[i], shape, g, dx=dx if i == 0 else None, grads=grads[i], workspace=ws)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    t_off = timed(offloaded)
    t_res = timed(resident)
    # one input's copy to host and back, alone (the link rate the overlap hides)
    a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    with torch.cuda.stream(side):
        a.record(side)
        hin[0].copy_(x, non_blocking=True)
        b.record(side)
        acts[0].copy_(hin[0], non_blocking=True)
        c.record(side)
    torch.cuda.synchronize()
    nbytes = N * D * 2
    return {"workload": f"{L} x {w['name']}", "n_layers": L, "step_ms_offloaded": t_off, "step_ms_resident": t_res,
            "offload_overhead": t_off / t_res - 1.0,
            "hbm_gb_block_inputs": {"resident": L * nbytes / 1e9, "offloaded": 2 * nbytes / 1e9},
            "host_gb": L * nbytes / 1e9,
            "copy_gbs": {"to_host": nbytes / (a.elapsed_time(b) * 1e-3) / 1e9,
                         "to_device": nbytes / (b.elapsed_time(c) * 1e-3) / 1e9}}


LOSS_WORKLOAD = dict(name="llama3-lm-head-loss-seq-shard-16k", n_tokens=16384, d_model=4096, vocab=128256,
                     tile_tokens=4096, lean_tile_tokens=1024, dtype="bf16")


def loss_bench(dev, steps, warmup):
    """The sequence-tiled cross-entropy of the Llama3 LM head (vocab 128256) on
    the same 16384-token sequence shard, tile_tokens 4096 (as the MLP), bf16:
    forward and backward times, model TFLOP/s (2 N D V forward, 4 N D V
    backward: dh and dW), kernel table and the tiled vs untiled logits buffer;
    plus the step time and workspace at tile_tokens 1024 (``lean_tile``), the
    smaller-memory point of the same trade."""
    import numpy as np
    import torch

    from headwise_chunked_attention_amd import api
    from headwise_chunked_attention_amd.synth import LossInputs

    w = LOSS_WORKLOAD
    N, D, V, T = w["n_tokens"], w["d_model"], w["vocab"], w["tile_tokens"]
    inp = LossInputs(N, D, V, "bf16", seed=0)
    h = torch.from_numpy(inp.h).to(dev).to(torch.bfloat16)
    wt = torch.from_numpy(inp.w).to(dev).to(torch.bfloat16)
    tg = torch.from_numpy(inp.targets).to(dev)
    g = torch.from_numpy(inp.g).to(dev)
    del inp
    ws = api.alloc_workspace(max(api.loss_workspace_bytes(N, D, V, T, "bf16", True),
                                 api.loss_workspace_bytes(N, D, V, T, "bf16", False)), dev)
    loss = torch.empty((N,), dtype=torch.float32, device=dev)
    lse = torch.empty((N,), dtype=torch.float32, device=dev)
    dh = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((V, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def fwd():
        api.loss_fwd(h, wt, tg, tile_tokens=T, loss=loss, lse=lse, workspace=ws)

    def bwd():
        api.loss_bwd(h, wt, tg, lse, g, tile_tokens=T, dh=dh, dw=dw, workspace=ws)

    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        e[0].record(stream)
        fwd()
        e[1].record(stream)
        bwd()
        e[2].record(stream)
    torch.cuda.synchronize()
    t_f = [e[0].elapsed_time(e[1]) for e in evs]
    t_b = [e[1].elapsed_time(e[2]) for e in evs]
    api.profile_start()
    fwd()
    bwd()
    prof = api.profile_stop()
    model = 6.0 * N * D * V
    step_ms = float(np.median([a + b for a, b in zip(t_f, t_b)]))
    kinds = {k: {"ms": v["ms"], "launches": v["launches"],
                 "tflops": (v["flops"] / (v["ms"] * 1e-3) / 1e12) if v["flops"] else None}
             for k, v in prof.items() if v["launches"]}
    lg = prof["loss_gemm"]
    achieved = lg["flops"] / (lg["ms"] * 1e-3) / 1e12
    return {"workload": w["name"], "n_tokens": N, "d_model": D, "vocab": V, "tile_tokens": T, "dtype": "bf16",
            "fwd_ms": float(np.median(t_f)), "bwd_ms": float(np.median(t_b)), "step_ms": step_ms,
            "model_tflops": model / (step_ms * 1e-3) / 1e12, "model_flops": model, "kernels": kinds,
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                         "kernel": "gemm_nt_kernel (loss and store epilogues) + row reduction"},
            "workspace_gb": {"tiled_bwd": api.loss_workspace_bytes(N, D, V, T, "bf16", True) / 1e9,
                             "untiled_logits": N * V * 2 / 1e9},
            "lean_tile": _loss_lean_tile(dev, h, wt, tg, g, loss, lse, dh, dw, w["lean_tile_tokens"], model)}


def _loss_lean_tile(dev, h, wt, tg, g, loss, lse, dh, dw, T, model, steps=3):
    """The loss fwd+bwd at a smaller tile: median step time and its workspace."""
    import numpy as np
    import torch

    from headwise_chunked_attention_amd import api

    N, D = h.shape
    V = wt.shape[0]
    ws = api.alloc_workspace(max(api.loss_workspace_bytes(N, D, V, T, "bf16", True),
                                 api.loss_workspace_bytes(N, D, V, T, "bf16", False)), dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        api.loss_fwd(h, wt, tg, tile_tokens=T, loss=loss, lse=lse, workspace=ws)
        api.loss_bwd(h, wt, tg, lse, g, tile_tokens=T, dh=dh, dw=dw, workspace=ws)

    step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in evs:
        e[0].record(stream)
        step()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    return {"tile_tokens": T, "step_ms": ms, "model_tflops": model / (ms * 1e-3) / 1e12,
            "workspace_gb_tiled_bwd": api.loss_workspace_bytes(N, D, V, T, "bf16", True) / 1e9}


def _wait(events, label, every_s=30.0):
    """Wait for the recorded step events, printing progress to stderr now and
    then (a long run is then never silent); touches nothing on the GPU."""
    t0 = last = time.perf_counter()
    while not events[-1].query():
        time.sleep(0.25)
        now = time.perf_counter()
        if now - last >= every_s:
            done = sum(1 for e in events if e.query())
            print(f"# {label}: {done} of {len(events)} step events done ({now - t0:.0f} s)", file=sys.stderr,
                  flush=True)
            last = now
    events[-1].synchronize()


def attention_bench(dev, name, w, chunk, steps, warmup, sweep_steps, prof_steps, sweep):
    """Time the step at one workload: the headline chunk size (no per-kernel
    events), a profiled run of prof_steps steps (kernel table and roofline),
    and the chunk sweep."""
    import numpy as np
    import torch

    from headwise_chunked_attention_amd import api
    from headwise_chunked_attention_amd.synth import LayerInputs

    N, D, hq, hkv, d, theta = (w[k] for k in ("n_tokens", "d_model", "n_q_heads", "n_kv_heads", "head_dim",
                                              "rope_theta"))
    norm = bool(w.get("qk_norm", False))
    t0 = time.perf_counter()
    t = {}
    inp = LayerInputs(N, D, hq, hkv, d, "bf16", seed=0, with_x=False, with_dy=False,
                      qk_norm="random" if norm else None)
    for k in ("wq", "wk", "wv", "wo") + (("q_norm", "k_norm") if norm else ()):
        t[k] = torch.from_numpy(getattr(inp, k)).to(dev).to(torch.bfloat16)
    from headwise_chunked_attention_amd.synth import gen_rows
    for k in ("x", "dy"):
        t[k] = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
        step = 262144
        for r0 in range(0, N, step):
            r1 = min(N, r0 + step)
            t[k][r0:r1].copy_(torch.from_numpy(gen_rows(k, N, D, 1.0, "bf16", 0, r0, r1)))
    del inp
    torch.cuda.synchronize()
    print(f"# {name}: inputs generated and resident in HBM in {time.perf_counter() - t0:.1f} s", file=sys.stderr,
          flush=True)
    fl = model_flops(N, D, hq, hkv, d)
    stream = torch.cuda.current_stream(dev)

    def run_chunk(C, steps, warmup, profile):
        kw = dict(n_q_heads=hq, n_kv_heads=hkv, head_dim=d, rope_theta=theta, chunk_heads=C)
        if norm:
            kw.update(q_norm=t["q_norm"], k_norm=t["k_norm"])
        ws_f = api.workspace_bytes(N, D, hq, hkv, d, C, norm, "bf16", False)
        ws_b = api.workspace_bytes(N, D, hq, hkv, d, C, norm, "bf16", True)
        ws = api.alloc_workspace(max(ws_f, ws_b), dev)
        y = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((hq, N), dtype=torch.float32, device=dev)
        f32 = torch.float32
        out = (torch.empty((N, D), dtype=torch.bfloat16, device=dev),
               torch.empty(t["wq"].shape, dtype=f32, device=dev), torch.empty(t["wk"].shape, dtype=f32, device=dev),
               torch.empty(t["wv"].shape, dtype=f32, device=dev), torch.empty(t["wo"].shape, dtype=f32, device=dev),
               torch.empty((d,), dtype=f32, device=dev) if norm else None,
               torch.empty((d,), dtype=f32, device=dev) if norm else None)

        def fwd():
            api.attn_fwd(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], y=y, lse=lse, workspace=ws, **kw)

        def bwd():
            api.attn_bwd(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], t["dy"], lse, out=out, workspace=ws, **kw)

        wev = []
        for _ in range(warmup):
            fwd()
            bwd()
            wev.append(torch.cuda.Event())
            wev[-1].record(stream)
        if wev:
            _wait(wev, f"{name} C={C} warmup")
        torch.cuda.synchronize()
        mem0 = torch.cuda.memory_allocated(dev)
        free0, _ = torch.cuda.mem_get_info(dev)
        if profile:
            api.profile_start()
        # events before each step, between its fwd and bwd, and after the last step
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        ev_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        for i in range(steps):
            evs[i][0].record(stream)
            fwd()
            evs[i][1].record(stream)
            bwd()
        ev_end.record(stream)
        _wait([e[0] for e in evs] + [ev_end], f"{name} C={C}")
        torch.cuda.synchronize()
        ms = evs[0][0].elapsed_time(ev_end) / steps
        t_f = [evs[i][0].elapsed_time(evs[i][1]) for i in range(steps)]
        t_b = [evs[i][1].elapsed_time(evs[i + 1][0] if i + 1 < steps else ev_end) for i in range(steps)]
        t_s = [a + b for a, b in zip(t_f, t_b)]
        prof = api.profile_stop() if profile else None
        free1, _ = torch.cuda.mem_get_info(dev)
        assert torch.cuda.memory_allocated(dev) == mem0, "the library must not allocate"
        res = {"chunk_heads": C, "ms_per_step": ms, "tflops": fl / (ms * 1e-3) / 1e12,
               "step_ms": {"median": float(np.median(t_s)), "min": float(np.min(t_s))},
               "fwd_ms": {"median": float(np.median(t_f)), "min": float(np.min(t_f))},
               "bwd_ms": {"median": float(np.median(t_b)), "min": float(np.min(t_b))},
               "ws_fwd_gb": ws_f / 1e9, "ws_bwd_gb": ws_b / 1e9, "hidden_alloc_bytes": int(free0 - free1)}
        print(f"# {name} C={C}: {ms:.2f} ms/step, {res['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        del ws, y, lse, out
        torch.cuda.empty_cache()
        return res, prof

    # the headline run carries no per-kernel events; a short second run with
    # the library's per-kernel timing on gives the kernel table
    head, _ = run_chunk(chunk, steps, warmup, profile=False)
    _, prof = run_chunk(chunk, prof_steps, 0, profile=True)
    res_sweep = []
    if sweep:
        for C in w["chunks"]:
            if C == chunk:
                res_sweep.append(head)
                continue
            r, _ = run_chunk(C, sweep_steps, 1, profile=False)
            res_sweep.append(r)
    del t
    torch.cuda.empty_cache()

    kernels = {}
    for k, v in prof.items():
        if v["launches"]:
            kernels[k] = {"ms_per_step": v["ms"] / prof_steps, "launches_per_step": v["launches"] / prof_steps,
                          "avg_launch_ms": v["ms"] / v["launches"],
                          "tflops": (v["flops"] / (v["ms"] * 1e-3) / 1e12) if v["flops"] else None}
    # attention-core rate: the core's model flops over the time of the kernels
    # that do them (forward attention, dK/dV and dQ; the recompute is extra work)
    core_ms = sum(prof[k]["ms"] for k in ("attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq")) / prof_steps
    # dominant kernel of the step: the attention kernel kind with the most time
    dom = max(("attn_fwd", "attn_recompute", "attn_bwd_dkdv", "attn_bwd_dq"), key=lambda k: prof[k]["ms"])
    ab = prof[dom]
    achieved = ab["flops"] / ab["launches"] / (ab["ms"] / ab["launches"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": TRAFFIC_BYTES.get((name, dom)),
                "kernel": KERNEL_NAMES[dom],
                "algorithmic_flops_per_launch": ab["flops"] / ab["launches"],
                "avg_launch_ms": ab["ms"] / ab["launches"]}
    return {"workload": name, "n_tokens": N, "chunk_heads": chunk, "head": head, "model_flops_per_step": fl,
            "attention_core_tflops": attn_core_flops(N, hq, d) / (core_ms * 1e-3) / 1e12,
            "hardware_tflops": hardware_flops(N, D, hq, hkv, d) / (head["ms_per_step"] * 1e-3) / 1e12,
            "chunk_sweep": res_sweep, "kernels": kernels, "roofline": roofline}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=1)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-mlp", action="store_true", help="skip the sequence-tiled MLP and loss measurements")
    ap.add_argument("--no-block", action="store_true", help="skip the transformer-block measurement")
    ap.add_argument("--no-secondary", action="store_true", help="skip the N = 131072 measurement")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default=HEADLINE,
                    help="the workload timed (default: the Llama3-8B share at N = 1048576; the 131072-token, "
                         "5M-token and Qwen3-32B-shaped shares on request)")
    ap.add_argument("--prof-steps", type=int, default=2, help="steps of the per-kernel timing run")
    ap.add_argument("--mlp-only", action="store_true",
                    help="run only the sequence-tiled MLP and loss measurements and print their JSON "
                         "(for profiling those GEMMs; not a bench line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain elementwise copy of 1 GiB (reads 1 GiB, writes 1 GiB) so that "
                         "profiler byte counters can be scaled against a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU's Ulysses share: multi-GPU runs (all-to-all over RCCL) are not part "
              "of this build; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from headwise_chunked_attention_amd import api

    dev = torch.device("cuda:0")
    api.load()
    peak_dev = api.device_peak(0)
    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print("# calibration copy: 3 x (1 GiB read + 1 GiB written)", file=sys.stderr, flush=True)
        del src, dst

    if args.mlp_only:
        mlp = mlp_bench(dev, max(2, args.steps // 2), 1)
        torch.cuda.empty_cache()
        loss = loss_bench(dev, max(2, args.steps // 2), 1)
        print(json.dumps({"mlp": mlp, "loss": loss}), flush=True)
        return

    name = args.workload
    w = WORKLOADS[name]
    sweep_steps = max(2, args.steps // 4)
    res = attention_bench(dev, name, w, args.chunk, args.steps, args.warmup, sweep_steps, args.prof_steps,
                          not args.no_sweep)
    head = res["head"]
    secondary = None
    if not args.no_secondary and name != SECONDARY:
        sec = attention_bench(dev, SECONDARY, WORKLOADS[SECONDARY], args.chunk, max(3, args.steps // 2), 2,
                              max(3, args.steps // 2), args.prof_steps, not args.no_sweep)
        secondary = {"workload": SECONDARY, "value": sec["head"]["tflops"], "unit": "TFLOP/s",
                     "ms_per_step": sec["head"]["ms_per_step"],
                     "frac_of_peak": sec["head"]["tflops"] / PEAK_BF16_TFLOPS,
                     "step_ms": sec["head"]["step_ms"], "fwd_ms": sec["head"]["fwd_ms"],
                     "bwd_ms": sec["head"]["bwd_ms"], "attention_core_tflops": sec["attention_core_tflops"],
                     "chunk_sweep": sec["chunk_sweep"], "kernels": sec["kernels"], "roofline": sec["roofline"]}

    mlp = loss = None
    steps = args.steps
    if not args.no_mlp:
        mlp = mlp_bench(dev, max(2, steps // 2), 1)
        print(f"# mlp: fwd {mlp['fwd_ms']:.2f} ms, bwd {mlp['bwd_ms']:.2f} ms, {mlp['model_tflops']:.0f} TFLOP/s",
              file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        loss = loss_bench(dev, max(2, steps // 2), 1)
        print(f"# loss: fwd {loss['fwd_ms']:.2f} ms, bwd {loss['bwd_ms']:.2f} ms, {loss['model_tflops']:.0f} TFLOP/s",
              file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    block = stack = None
    if not args.no_block:
        block = block_bench(dev, max(2, steps // 3), 1)
        print(f"# block: fwd {block['fwd_ms']:.1f} ms, bwd {block['bwd_ms']:.1f} ms (kept h: {block['bwd_kept_ms']:.1f}),"
              f" {block['model_tflops']:.0f} model TFLOP/s", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        stack = stack_bench(dev, 2)
        print(f"# stack of {stack['n_layers']}: offloaded {stack['step_ms_offloaded']:.1f} ms, resident "
              f"{stack['step_ms_resident']:.1f} ms ({100 * stack['offload_overhead']:+.1f}%)", file=sys.stderr,
              flush=True)
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        print("# cpu baseline: the fp64 oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w)
        # GPU speedups: against the workload's projected oracle time, and
        # against the oracle's tiny-configuration run (timed on the GPU here)
        main_row = cpu["rows"][0]
        main_row["gpu_speedup_vs_projected"] = main_row["projected_seconds_at_n"]["seconds"] / (head["ms_per_step"] * 1e-3)
        tiny_row = cpu["rows"][1]
        tiny_row["gpu_seconds"] = tiny_gpu_seconds(dev)
        tiny_row["gpu_speedup"] = tiny_row["seconds"] / tiny_row["gpu_seconds"]

    N, D, hq, hkv, d = (w[k] for k in ("n_tokens", "d_model", "n_q_heads", "n_kv_heads", "head_dim"))
    line = {
        "metric": METRIC,
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded host Gaussian inputs, random-init weights; no dataset)",
        "config": {"workload": name, "n_tokens": N, "d_model": D, "n_q_heads": hq, "n_kv_heads": hkv,
                   "head_dim": d, "rope_theta": w["rope_theta"], "causal": True, "chunk_heads": args.chunk,
                   "qk_norm": bool(w.get("qk_norm", False)),
                   "parallelism": "one GPU's Ulysses head share (no collectives)"},
        "frac_of_peak": head["tflops"] / PEAK_BF16_TFLOPS,
        "peak_from_device": dict(peak_dev, frac_of_peak=head["tflops"] / peak_dev["bf16_dense_tflops"]),
        "model_flops_per_step": res["model_flops_per_step"],
        "step_ms": head["step_ms"],
        "fwd_ms": head["fwd_ms"],
        "bwd_ms": head["bwd_ms"],
        "attention_core_tflops": res["attention_core_tflops"],
        "hardware_tflops": res["hardware_tflops"],
        "workspace_gb": {"fwd": head["ws_fwd_gb"], "bwd": head["ws_bwd_gb"]},
        "peak_workspace_gb_vs_chunk": {str(r["chunk_heads"]): {"fwd": r["ws_fwd_gb"], "bwd": r["ws_bwd_gb"]}
                                       for r in res["chunk_sweep"]},
        "chunk_sweep": res["chunk_sweep"],
        "kernels": res["kernels"],
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "secondary": secondary,
        "mlp": mlp,
        "loss": loss,
        "block": block,
        "stack": stack,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
