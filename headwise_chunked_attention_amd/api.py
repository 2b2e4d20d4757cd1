"""Thin Python binding of libupipe.so (ctypes): argument marshalling only.

PyTorch supplies device memory and the stream; every step of the attention
layer runs in the library's HIP kernels. There is no fallback: if the library
is missing or the tensors are not on a GPU, the call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libupipe.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "upipe.h")

UPIPE_F32, UPIPE_BF16 = 0, 1
_DTYPES = {torch.float32: UPIPE_F32, torch.bfloat16: UPIPE_BF16}

_lib = None


class BlockShape(ctypes.Structure):
    """upipe_block_shape_t."""
    _fields_ = [("n_tokens", ctypes.c_int64), ("d_model", ctypes.c_int64), ("d_ff", ctypes.c_int64),
                ("tile_tokens", ctypes.c_int64), ("n_q_heads", ctypes.c_int), ("n_kv_heads", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("chunk_heads", ctypes.c_int), ("rope_theta", ctypes.c_double),
                ("norm_eps", ctypes.c_float), ("qk_norm_eps", ctypes.c_float)]


_BLOCK_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "q_norm", "k_norm", "mlp_norm", "w_gate", "w_up",
                  "w_down")


class BlockWeights(ctypes.Structure):
    """upipe_block_weights_t (device pointers)."""
    _fields_ = [(n, ctypes.c_void_p) for n in _BLOCK_TENSORS]


class BlockGrads(ctypes.Structure):
    """upipe_block_grads_t (device pointers to fp32)."""
    _fields_ = [(n, ctypes.c_void_p) for n in _BLOCK_TENSORS]


class UpipeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


def load():
    """Load libupipe.so (built in-tree by headwise_chunked_attention_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m headwise_chunked_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, dbl, flt, vp, sz = (ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_float,
                                  ctypes.c_void_p, ctypes.c_size_t)
    lib.upipe_attn_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32, i32, i32, i32]
    lib.upipe_attn_workspace_bytes.restype = sz
    lib.upipe_attn_fwd.argtypes = [i32, i64, i64, i32, i32, i32, dbl, i32,
                                   vp, vp, vp, vp, vp, vp, vp, flt, vp, vp, vp, sz, vp]
    lib.upipe_attn_fwd.restype = i32
    lib.upipe_attn_bwd.argtypes = [i32, i64, i64, i32, i32, i32, dbl, i32,
                                   vp, vp, vp, vp, vp, vp, vp, flt, vp, vp, vp,
                                   vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.upipe_attn_bwd.restype = i32
    lib.upipe_attn_fwd_noalloc.argtypes = [i32, i64, i64, i32, i32, i32, dbl, i32,
                                           vp, vp, vp, vp, vp, vp, vp, flt, vp, vp, vp]
    lib.upipe_attn_fwd_noalloc.restype = i32
    lib.upipe_attn_bwd_deterministic.argtypes = lib.upipe_attn_bwd.argtypes
    lib.upipe_attn_bwd_deterministic.restype = i32
    lib.upipe_choose_chunk_heads.argtypes = [i64, i64, i32, i32, i32, i32, i32, i32, sz,
                                             ctypes.POINTER(ctypes.c_size_t)]
    lib.upipe_choose_chunk_heads.restype = i32
    lib.upipe_mlp_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, i32]
    lib.upipe_mlp_workspace_bytes.restype = sz
    lib.upipe_mlp_fwd.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.upipe_mlp_fwd.restype = i32
    lib.upipe_mlp_bwd.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.upipe_mlp_bwd.restype = i32
    lib.upipe_loss_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, i32]
    lib.upipe_loss_workspace_bytes.restype = sz
    lib.upipe_loss_fwd.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.upipe_loss_fwd.restype = i32
    lib.upipe_loss_bwd.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.upipe_loss_bwd.restype = i32
    bp = ctypes.POINTER(BlockShape)
    lib.upipe_block_workspace_bytes.argtypes = [bp, i32, i32, i32]
    lib.upipe_block_workspace_bytes.restype = sz
    lib.upipe_block_fwd.argtypes = [i32, bp, vp, ctypes.POINTER(BlockWeights), vp, vp, vp, vp, sz, vp]
    lib.upipe_block_fwd.restype = i32
    lib.upipe_block_bwd.argtypes = [i32, bp, vp, ctypes.POINTER(BlockWeights), vp, vp, vp, vp,
                                    ctypes.POINTER(BlockGrads), vp, sz, vp]
    lib.upipe_block_bwd.restype = i32
    lib.upipe_stack_workspace_bytes.argtypes = [bp, i32, i32]
    lib.upipe_stack_workspace_bytes.restype = sz
    lib.upipe_stack_fwd.argtypes = [i32, bp, i32, ctypes.POINTER(BlockWeights), vp, vp, vp, vp, sz, vp, vp]
    lib.upipe_stack_fwd.restype = i32
    lib.upipe_stack_bwd.argtypes = [i32, bp, i32, ctypes.POINTER(BlockWeights), vp, vp, vp,
                                    ctypes.POINTER(BlockGrads), vp, sz, vp, vp]
    lib.upipe_stack_bwd.restype = i32
    lib.upipe_strerror.argtypes = [i32]
    lib.upipe_strerror.restype = ctypes.c_char_p
    lib.upipe_device_peak.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int),
                                       ctypes.POINTER(ctypes.c_int)]
    lib.upipe_device_peak.restype = i32
    lib.upipe_version.argtypes = []
    lib.upipe_version.restype = i32
    lib.upipe_profile_start.argtypes = []
    lib.upipe_profile_start.restype = i32
    lib.upipe_profile_stop.argtypes = [vp, vp, vp, i32]
    lib.upipe_profile_stop.restype = i32
    _lib = lib
    return lib


def header_symbols() -> list[str]:
    """Names of the functions include/upipe.h declares."""
    txt = open(HEADER_PATH).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(upipe_[a-z_]+)\s*\(", txt)))


def strerror(code: int) -> str:
    return load().upipe_strerror(int(code)).decode()


def dtype_code(dtype) -> int:
    if dtype in _DTYPES:
        return _DTYPES[dtype]
    if dtype in ("fp32", "f32", "float32"):
        return UPIPE_F32
    if dtype in ("bf16", "bfloat16"):
        return UPIPE_BF16
    raise ValueError(f"unsupported dtype {dtype}")


def workspace_bytes(n_tokens, d_model, n_q_heads, n_kv_heads, head_dim, chunk_heads, qk_norm,
                    dtype, backward) -> int:
    return int(load().upipe_attn_workspace_bytes(int(n_tokens), int(d_model), int(n_q_heads),
                                                  int(n_kv_heads), int(head_dim), int(chunk_heads),
                                                  int(bool(qk_norm)), dtype_code(dtype), int(bool(backward))))


def choose_chunk_heads(n_tokens, d_model, n_q_heads, n_kv_heads, head_dim, qk_norm, dtype, backward,
                       budget_bytes) -> tuple[int, int]:
    """Largest accepted chunk_heads whose workspace fits budget_bytes, and that workspace.

    Raises UpipeError (code UPIPE_ERR_WORKSPACE) when not even one head per chunk fits.
    """
    ws = ctypes.c_size_t(0)
    c = int(load().upipe_choose_chunk_heads(int(n_tokens), int(d_model), int(n_q_heads), int(n_kv_heads),
                                            int(head_dim), int(bool(qk_norm)), dtype_code(dtype),
                                            int(bool(backward)), int(budget_bytes), ctypes.byref(ws)))
    if c < 0:
        raise UpipeError(c, "upipe_choose_chunk_heads")
    return c, int(ws.value)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype, shape, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _alloc_on(stream):
    """Context for the tensors a call allocates itself (outputs, workspace):
    they belong to the stream the library enqueues on, so the caching
    allocator does not hand their memory to other work before that stream
    is done with it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """A 256-byte aligned device buffer of at least nbytes (torch's allocator aligns to 512)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def attn_fwd(x, wq, wk, wv, wo, *, n_q_heads, n_kv_heads, head_dim, rope_theta, chunk_heads,
             q_norm=None, k_norm=None, eps=1e-6, y=None, lse=None, workspace=None, stream=None):
    """Forward of the headwise-chunked attention layer; returns ``(y, lse)``."""
    lib = load()
    N, D = x.shape
    dev = x.device
    dt = x.dtype
    d = head_dim
    _check(x, "x", dt, (N, D), dev)
    _check(wq, "wq", dt, (n_q_heads * d, D), dev)
    _check(wk, "wk", dt, (n_kv_heads * d, D), dev)
    _check(wv, "wv", dt, (n_kv_heads * d, D), dev)
    _check(wo, "wo", dt, (D, n_q_heads * d), dev)
    if (q_norm is None) != (k_norm is None):
        raise ValueError("q_norm and k_norm must both be given or both be None")
    if q_norm is not None:
        _check(q_norm, "q_norm", dt, (d,), dev)
        _check(k_norm, "k_norm", dt, (d,), dev)
    need = workspace_bytes(N, D, n_q_heads, n_kv_heads, d, chunk_heads, q_norm is not None, dt, False)
    with _alloc_on(stream):
        if y is None:
            y = torch.empty((N, D), dtype=dt, device=dev)
        if lse is None:
            lse = torch.empty((n_q_heads, N), dtype=torch.float32, device=dev)
        if workspace is None:
            workspace = alloc_workspace(need, dev)
    _check(y, "y", dt, (N, D), dev)
    _check(lse, "lse", torch.float32, (n_q_heads, N), dev)
    rc = lib.upipe_attn_fwd(dtype_code(dt), N, D, n_q_heads, n_kv_heads, d, float(rope_theta), chunk_heads,
                            _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(q_norm), _ptr(k_norm),
                            float(eps), _ptr(y), _ptr(lse), _ptr(workspace), workspace.numel(),
                            _stream_handle(dev, stream))
    if rc != 0:
        raise UpipeError(rc, "upipe_attn_fwd")
    return y, lse


NOALLOC_SCRATCH_BYTES = 64 << 20  # UPIPE_NOALLOC_SCRATCH_BYTES


def attn_fwd_noalloc(x, wq, wk, wv, wo, y, lse, *, n_q_heads, n_kv_heads, head_dim, rope_theta, chunk_heads,
                     q_norm=None, k_norm=None, eps=1e-6, stream=None):
    """upipe_attn_fwd_noalloc: the forward into the caller's y and lse, with the
    chunk buffers in the library's static device scratch (nothing allocated,
    here or in the library)."""
    lib = load()
    N, D = x.shape
    dev = x.device
    dt = x.dtype
    d = head_dim
    _check(x, "x", dt, (N, D), dev)
    _check(wq, "wq", dt, (n_q_heads * d, D), dev)
    _check(wk, "wk", dt, (n_kv_heads * d, D), dev)
    _check(wv, "wv", dt, (n_kv_heads * d, D), dev)
    _check(wo, "wo", dt, (D, n_q_heads * d), dev)
    if (q_norm is None) != (k_norm is None):
        raise ValueError("q_norm and k_norm must both be given or both be None")
    if q_norm is not None:
        _check(q_norm, "q_norm", dt, (d,), dev)
        _check(k_norm, "k_norm", dt, (d,), dev)
    _check(y, "y", dt, (N, D), dev)
    _check(lse, "lse", torch.float32, (n_q_heads, N), dev)
    with torch.cuda.device(dev):  # the library takes the current device's scratch
        rc = lib.upipe_attn_fwd_noalloc(dtype_code(dt), N, D, n_q_heads, n_kv_heads, d, float(rope_theta),
                                        chunk_heads, _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(q_norm),
                                        _ptr(k_norm), float(eps), _ptr(y), _ptr(lse), _stream_handle(dev, stream))
    if rc != 0:
        raise UpipeError(rc, "upipe_attn_fwd_noalloc")
    return y, lse


def attn_bwd(x, wq, wk, wv, wo, dy, lse, *, n_q_heads, n_kv_heads, head_dim, rope_theta, chunk_heads,
             q_norm=None, k_norm=None, eps=1e-6, out=None, workspace=None, stream=None, deterministic=False):
    """Backward of the layer; returns ``(dx, dwq, dwk, dwv, dwo, dq_norm, dk_norm)``.
    ``deterministic=True`` calls upipe_attn_bwd_deterministic (bitwise reproducible)."""
    lib = load()
    N, D = x.shape
    dev = x.device
    dt = x.dtype
    d = head_dim
    _check(x, "x", dt, (N, D), dev)
    _check(wq, "wq", dt, (n_q_heads * d, D), dev)
    _check(wk, "wk", dt, (n_kv_heads * d, D), dev)
    _check(wv, "wv", dt, (n_kv_heads * d, D), dev)
    _check(wo, "wo", dt, (D, n_q_heads * d), dev)
    _check(dy, "dy", dt, (N, D), dev)
    _check(lse, "lse", torch.float32, (n_q_heads, N), dev)
    norm = q_norm is not None
    if (q_norm is None) != (k_norm is None):
        raise ValueError("q_norm and k_norm must both be given or both be None")
    if norm:
        _check(q_norm, "q_norm", dt, (d,), dev)
        _check(k_norm, "k_norm", dt, (d,), dev)
    f32 = torch.float32
    need = workspace_bytes(N, D, n_q_heads, n_kv_heads, d, chunk_heads, norm, dt, True)
    with _alloc_on(stream):
        if out is None:
            out = (torch.empty((N, D), dtype=dt, device=dev),
                   torch.empty(wq.shape, dtype=f32, device=dev), torch.empty(wk.shape, dtype=f32, device=dev),
                   torch.empty(wv.shape, dtype=f32, device=dev), torch.empty(wo.shape, dtype=f32, device=dev),
                   torch.empty((d,), dtype=f32, device=dev) if norm else None,
                   torch.empty((d,), dtype=f32, device=dev) if norm else None)
        if workspace is None:
            workspace = alloc_workspace(need, dev)
    dx, dwq, dwk, dwv, dwo, dqn, dkn = out
    _check(dx, "dx", dt, (N, D), dev)
    for t, n, ref in ((dwq, "dwq", wq), (dwk, "dwk", wk), (dwv, "dwv", wv), (dwo, "dwo", wo)):
        _check(t, n, f32, tuple(ref.shape), dev)
    if norm:
        _check(dqn, "dq_norm", f32, (d,), dev)
        _check(dkn, "dk_norm", f32, (d,), dev)
    fn = lib.upipe_attn_bwd_deterministic if deterministic else lib.upipe_attn_bwd
    rc = fn(dtype_code(dt), N, D, n_q_heads, n_kv_heads, d, float(rope_theta), chunk_heads,
                            _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(q_norm), _ptr(k_norm),
                            float(eps), _ptr(dy), _ptr(lse), _ptr(dx), _ptr(dwq), _ptr(dwk), _ptr(dwv),
                            _ptr(dwo), _ptr(dqn), _ptr(dkn), _ptr(workspace), workspace.numel(),
                            _stream_handle(dev, stream))
    if rc != 0:
        raise UpipeError(rc, "upipe_attn_bwd")
    return dx, dwq, dwk, dwv, dwo, dqn, dkn


KERNEL_KINDS = ("projection", "out_gemm", "attn_fwd", "attn_recompute", "attn_bwd_dkdv", "attn_bwd_dq", "wgrad",
                "other", "mlp_gemm", "mlp_wgrad", "loss_gemm", "loss_wgrad", "block_norm")


def loss_workspace_bytes(n_tokens, d_model, vocab, tile_tokens, dtype, backward) -> int:
    return int(load().upipe_loss_workspace_bytes(int(n_tokens), int(d_model), int(vocab), int(tile_tokens),
                                                  dtype_code(dtype), int(bool(backward))))


def loss_fwd(h, w, targets, *, tile_tokens, loss=None, lse=None, workspace=None, stream=None):
    """Per-token cross-entropy of the LM head h W^T, tile_tokens rows at a time
    (upipe_loss_fwd). Returns (loss [N], lse [N]), both fp32."""
    lib = load()
    dev, dt = h.device, h.dtype
    N, D = h.shape
    V = w.shape[0]
    _check(h, "h", dt, (N, D), dev)
    _check(w, "w", dt, (V, D), dev)
    _check(targets, "targets", torch.int32, (N,), dev)
    f32 = torch.float32
    with _alloc_on(stream):
        loss = torch.empty((N,), dtype=f32, device=dev) if loss is None else loss
        lse = torch.empty((N,), dtype=f32, device=dev) if lse is None else lse
        if workspace is None:
            workspace = alloc_workspace(loss_workspace_bytes(N, D, V, tile_tokens, dt, False), dev)
    _check(loss, "loss", f32, (N,), dev)
    _check(lse, "lse", f32, (N,), dev)
    rc = lib.upipe_loss_fwd(dtype_code(dt), N, D, V, int(tile_tokens), _ptr(h), _ptr(w), _ptr(targets), _ptr(loss),
                            _ptr(lse), _ptr(workspace), workspace.numel(), _stream_handle(dev, stream))
    if rc != 0:
        raise UpipeError(rc, "upipe_loss_fwd")
    return loss, lse


def loss_bwd(h, w, targets, lse, g, *, tile_tokens, dh=None, dw=None, workspace=None, stream=None):
    """(dh, dW) of the per-token losses for upstream gradients g [N] (upipe_loss_bwd)."""
    lib = load()
    dev, dt = h.device, h.dtype
    N, D = h.shape
    V = w.shape[0]
    f32 = torch.float32
    _check(h, "h", dt, (N, D), dev)
    _check(w, "w", dt, (V, D), dev)
    _check(targets, "targets", torch.int32, (N,), dev)
    _check(lse, "lse", f32, (N,), dev)
    _check(g, "g", f32, (N,), dev)
    with _alloc_on(stream):
        dh = torch.empty((N, D), dtype=dt, device=dev) if dh is None else dh
        dw = torch.empty((V, D), dtype=f32, device=dev) if dw is None else dw
        if workspace is None:
            workspace = alloc_workspace(loss_workspace_bytes(N, D, V, tile_tokens, dt, True), dev)
    _check(dh, "dh", dt, (N, D), dev)
    _check(dw, "dw", f32, (V, D), dev)
    rc = lib.upipe_loss_bwd(dtype_code(dt), N, D, V, int(tile_tokens), _ptr(h), _ptr(w), _ptr(targets), _ptr(lse),
                            _ptr(g), _ptr(dh), _ptr(dw), _ptr(workspace), workspace.numel(),
                            _stream_handle(dev, stream))
    if rc != 0:
        raise UpipeError(rc, "upipe_loss_bwd")
    return dh, dw


def mlp_workspace_bytes(n_tokens, d_model, d_ff, tile_tokens, dtype, backward) -> int:
    return int(load().upipe_mlp_workspace_bytes(int(n_tokens), int(d_model), int(d_ff), int(tile_tokens),
                                                 dtype_code(dtype), int(bool(backward))))


def mlp_fwd(x, w_gate, w_up, w_down, *, tile_tokens, y=None, workspace=None, stream=None):
    """y = (silu(x Wg^T) * (x Wu^T)) Wd^T, tile_tokens rows at a time (upipe_mlp_fwd)."""
    lib = load()
    dev, dt = x.device, x.dtype
    N, D = x.shape
    F = w_gate.shape[0]
    _check(x, "x", dt, (N, D), dev)
    _check(w_gate, "w_gate", dt, (F, D), dev)
    _check(w_up, "w_up", dt, (F, D), dev)
    _check(w_down, "w_down", dt, (D, F), dev)
    with _alloc_on(stream):
        if y is None:
            y = torch.empty((N, D), dtype=dt, device=dev)
        if workspace is None:
            workspace = alloc_workspace(mlp_workspace_bytes(N, D, F, tile_tokens, dt, False), dev)
    _check(y, "y", dt, (N, D), dev)
    rc = lib.upipe_mlp_fwd(dtype_code(dt), N, D, F, int(tile_tokens), _ptr(x), _ptr(w_gate), _ptr(w_up),
                           _ptr(w_down), _ptr(y), _ptr(workspace), workspace.numel(), _stream_handle(dev, stream))
    if rc != 0:
        raise UpipeError(rc, "upipe_mlp_fwd")
    return y


def mlp_bwd(x, w_gate, w_up, w_down, dy, *, tile_tokens, out=None, workspace=None, stream=None):
    """(dx, dw_gate, dw_up, dw_down) of ``mlp_fwd`` for upstream gradient dy (upipe_mlp_bwd)."""
    lib = load()
    dev, dt = x.device, x.dtype
    N, D = x.shape
    F = w_gate.shape[0]
    _check(x, "x", dt, (N, D), dev)
    _check(w_gate, "w_gate", dt, (F, D), dev)
    _check(w_up, "w_up", dt, (F, D), dev)
    _check(w_down, "w_down", dt, (D, F), dev)
    _check(dy, "dy", dt, (N, D), dev)
    f32 = torch.float32
    with _alloc_on(stream):
        if out is None:
            out = (torch.empty((N, D), dtype=dt, device=dev), torch.empty((F, D), dtype=f32, device=dev),
                   torch.empty((F, D), dtype=f32, device=dev), torch.empty((D, F), dtype=f32, device=dev))
        if workspace is None:
            workspace = alloc_workspace(mlp_workspace_bytes(N, D, F, tile_tokens, dt, True), dev)
    dx, dwg, dwu, dwd = out
    _check(dx, "dx", dt, (N, D), dev)
    _check(dwg, "dw_gate", f32, (F, D), dev)
    _check(dwu, "dw_up", f32, (F, D), dev)
    _check(dwd, "dw_down", f32, (D, F), dev)
    rc = lib.upipe_mlp_bwd(dtype_code(dt), N, D, F, int(tile_tokens), _ptr(x), _ptr(w_gate), _ptr(w_up),
                           _ptr(w_down), _ptr(dy), _ptr(dx), _ptr(dwg), _ptr(dwu), _ptr(dwd), _ptr(workspace),
                           workspace.numel(), _stream_handle(dev, stream))
    if rc != 0:
        raise UpipeError(rc, "upipe_mlp_bwd")
    return dx, dwg, dwu, dwd


def block_shape(n_tokens, d_model, d_ff, tile_tokens, n_q_heads, n_kv_heads, head_dim, chunk_heads, rope_theta,
                norm_eps=1e-5, qk_norm_eps=1e-6) -> BlockShape:
    return BlockShape(int(n_tokens), int(d_model), int(d_ff), int(tile_tokens), int(n_q_heads), int(n_kv_heads),
                      int(head_dim), int(chunk_heads), float(rope_theta), float(norm_eps), float(qk_norm_eps))


def block_workspace_bytes(shape: BlockShape, qk_norm, dtype, backward) -> int:
    return int(load().upipe_block_workspace_bytes(ctypes.byref(shape), int(bool(qk_norm)), dtype_code(dtype),
                                                   int(bool(backward))))


def _block_weight_shapes(s: BlockShape):
    D, F, d = s.d_model, s.d_ff, s.head_dim
    return {"attn_norm": (D,), "wq": (s.n_q_heads * d, D), "wk": (s.n_kv_heads * d, D),
            "wv": (s.n_kv_heads * d, D), "wo": (D, s.n_q_heads * d), "q_norm": (d,), "k_norm": (d,),
            "mlp_norm": (D,), "w_gate": (F, D), "w_up": (F, D), "w_down": (D, F)}


def _block_weights(shape: BlockShape, weights: dict, dt, dev):
    if (weights.get("q_norm") is None) != (weights.get("k_norm") is None):
        raise ValueError("q_norm and k_norm must both be given or both be None")
    shapes = _block_weight_shapes(shape)
    w = BlockWeights()
    for n in _BLOCK_TENSORS:
        t = weights.get(n)
        if t is None and n in ("q_norm", "k_norm"):
            continue
        _check(t, n, dt, shapes[n], dev)
        setattr(w, n, t.data_ptr())
    return w


def block_fwd(x, weights: dict, shape: BlockShape, *, y=None, h_mid=None, lse=None, workspace=None, stream=None):
    """Forward of the pre-norm transformer block (upipe_block_fwd).

    ``weights`` maps attn_norm, wq, wk, wv, wo, [q_norm, k_norm], mlp_norm,
    w_gate, w_up, w_down to tensors of x's dtype. h_mid and lse are optional
    outputs (pass tensors to keep them). Returns (y, h_mid, lse)."""
    lib = load()
    dev, dt = x.device, x.dtype
    N, D = shape.n_tokens, shape.d_model
    _check(x, "x", dt, (N, D), dev)
    w = _block_weights(shape, weights, dt, dev)
    qk = weights.get("q_norm") is not None
    with _alloc_on(stream):
        y = torch.empty((N, D), dtype=dt, device=dev) if y is None else y
        if workspace is None:
            workspace = alloc_workspace(block_workspace_bytes(shape, qk, dt, False), dev)
    _check(y, "y", dt, (N, D), dev)
    if h_mid is not None:
        _check(h_mid, "h_mid", dt, (N, D), dev)
    if lse is not None:
        _check(lse, "lse", torch.float32, (shape.n_q_heads, N), dev)
    rc = lib.upipe_block_fwd(dtype_code(dt), ctypes.byref(shape), _ptr(x), ctypes.byref(w), _ptr(y), _ptr(h_mid),
                             _ptr(lse), _ptr(workspace), workspace.numel(), _stream_handle(dev, stream))
    if rc != 0:
        raise UpipeError(rc, "upipe_block_fwd")
    return y, h_mid, lse


def block_bwd(x, weights: dict, shape: BlockShape, dy, *, h_mid=None, lse=None, dx=None, grads=None,
              workspace=None, stream=None):
    """Backward of the block (upipe_block_bwd): returns (dx, grads) with grads a
    dict of fp32 tensors named like ``weights``. h_mid and lse: both None
    (recompute from x) or both from block_fwd."""
    lib = load()
    dev, dt = x.device, x.dtype
    N, D = shape.n_tokens, shape.d_model
    _check(x, "x", dt, (N, D), dev)
    _check(dy, "dy", dt, (N, D), dev)
    w = _block_weights(shape, weights, dt, dev)
    if (h_mid is None) != (lse is None):
        raise ValueError("h_mid and lse must both be given or both be None")
    if h_mid is not None:
        _check(h_mid, "h_mid", dt, (N, D), dev)
        _check(lse, "lse", torch.float32, (shape.n_q_heads, N), dev)
    qk = weights.get("q_norm") is not None
    shapes = _block_weight_shapes(shape)
    f32 = torch.float32
    with _alloc_on(stream):
        if grads is None:
            grads = {n: torch.empty(shapes[n], dtype=f32, device=dev) for n in _BLOCK_TENSORS
                     if qk or n not in ("q_norm", "k_norm")}
        dx = torch.empty((N, D), dtype=dt, device=dev) if dx is None else dx
        if workspace is None:
            workspace = alloc_workspace(block_workspace_bytes(shape, qk, dt, True), dev)
    g = BlockGrads()
    for n in _BLOCK_TENSORS:
        t = grads.get(n)
        if t is None and not qk and n in ("q_norm", "k_norm"):
            continue
        _check(t, "grad " + n, f32, shapes[n], dev)
        setattr(g, n, t.data_ptr())
    _check(dx, "dx", dt, (N, D), dev)
    rc = lib.upipe_block_bwd(dtype_code(dt), ctypes.byref(shape), _ptr(x), ctypes.byref(w), _ptr(h_mid), _ptr(lse),
                             _ptr(dy), _ptr(dx), ctypes.byref(g), _ptr(workspace), workspace.numel(),
                             _stream_handle(dev, stream))
    if rc != 0:
        raise UpipeError(rc, "upipe_block_bwd")
    return dx, grads


def stack_workspace_bytes(shape: BlockShape, qk_norm, dtype) -> int:
    return int(load().upipe_stack_workspace_bytes(ctypes.byref(shape), int(bool(qk_norm)), dtype_code(dtype)))


def _check_host(t, name, dtype, shape):
    if t is None or t.is_cuda:
        raise ValueError(f"{name} must be a host tensor (pinned: torch.empty(..., pin_memory=True))")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")


def _stream_ptr(dev, stream):
    return None if stream is None else ctypes.c_void_p(stream.cuda_stream)


def stack_fwd(x, layers, shape: BlockShape, host_inputs, *, y=None, workspace=None, stream=None,
              copy_stream=None):
    """Forward of a stack of blocks (upipe_stack_fwd); ``layers`` is a list of
    weight dicts as for ``block_fwd``; ``host_inputs`` a host tensor
    [n_layers][N][D] of x's dtype that receives each block's input. Returns y."""
    lib = load()
    dev, dt = x.device, x.dtype
    N, D, L = shape.n_tokens, shape.d_model, len(layers)
    _check(x, "x", dt, (N, D), dev)
    _check_host(host_inputs, "host_inputs", dt, (L, N, D))
    ws = (BlockWeights * L)(*[_block_weights(shape, w, dt, dev) for w in layers])
    qk = layers[0].get("q_norm") is not None
    with _alloc_on(stream):
        y = torch.empty((N, D), dtype=dt, device=dev) if y is None else y
        if workspace is None:
            workspace = alloc_workspace(stack_workspace_bytes(shape, qk, dt), dev)
    _check(y, "y", dt, (N, D), dev)
    rc = lib.upipe_stack_fwd(dtype_code(dt), ctypes.byref(shape), L, ws, _ptr(x), _ptr(y),
                             ctypes.c_void_p(host_inputs.data_ptr()), _ptr(workspace), workspace.numel(),
                             _stream_handle(dev, stream), _stream_ptr(dev, copy_stream))
    if rc != 0:
        raise UpipeError(rc, "upipe_stack_fwd")
    return y


def stack_bwd(layers, shape: BlockShape, host_inputs, dy, *, dx=None, grads=None, workspace=None, stream=None,
              copy_stream=None):
    """Backward of a stack of blocks (upipe_stack_bwd) from the inputs the
    forward left in ``host_inputs``. Returns (dx, grads), grads a list of
    per-layer dicts of fp32 tensors."""
    lib = load()
    dev, dt = dy.device, dy.dtype
    N, D, L = shape.n_tokens, shape.d_model, len(layers)
    _check(dy, "dy", dt, (N, D), dev)
    _check_host(host_inputs, "host_inputs", dt, (L, N, D))
    ws = (BlockWeights * L)(*[_block_weights(shape, w, dt, dev) for w in layers])
    qk = layers[0].get("q_norm") is not None
    shapes = _block_weight_shapes(shape)
    f32 = torch.float32
    with _alloc_on(stream):
        if grads is None:
            grads = [{n: torch.empty(shapes[n], dtype=f32, device=dev) for n in _BLOCK_TENSORS
                      if qk or n not in ("q_norm", "k_norm")} for _ in range(L)]
        dx = torch.empty((N, D), dtype=dt, device=dev) if dx is None else dx
        if workspace is None:
            workspace = alloc_workspace(stack_workspace_bytes(shape, qk, dt), dev)
    gs = (BlockGrads * L)()
    for i, gd in enumerate(grads):
        for n in _BLOCK_TENSORS:
            t = gd.get(n)
            if t is None and not qk and n in ("q_norm", "k_norm"):
                continue
            _check(t, f"layer {i} grad {n}", f32, shapes[n], dev)
            setattr(gs[i], n, t.data_ptr())
    _check(dx, "dx", dt, (N, D), dev)
    rc = lib.upipe_stack_bwd(dtype_code(dt), ctypes.byref(shape), L, ws, ctypes.c_void_p(host_inputs.data_ptr()),
                             _ptr(dy), _ptr(dx), gs, _ptr(workspace), workspace.numel(), _stream_handle(dev, stream),
                             _stream_ptr(dev, copy_stream))
    if rc != 0:
        raise UpipeError(rc, "upipe_stack_bwd")
    return dx, grads


def device_peak(device: int = 0) -> dict:
    """Dense bf16 MFMA peak of a device from its properties (upipe_device_peak)."""
    tf, cu, clk = ctypes.c_double(0), ctypes.c_int(0), ctypes.c_int(0)
    rc = load().upipe_device_peak(int(device), ctypes.byref(tf), ctypes.byref(cu), ctypes.byref(clk))
    if rc != 0:
        raise UpipeError(rc, "upipe_device_peak")
    return {"bf16_dense_tflops": tf.value, "compute_units": cu.value, "clock_khz": clk.value}


def profile_start():
    """Start per-kernel event timing inside the library (see upipe_profile_start)."""
    rc = load().upipe_profile_start()
    if rc != 0:
        raise UpipeError(rc, "upipe_profile_start")


def profile_stop():
    """Stop timing; returns {kind: {"ms": total, "launches": n, "flops": f}}."""
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    fl = (ctypes.c_double * n)()
    rc = load().upipe_profile_stop(ctypes.cast(ms, ctypes.c_void_p), ctypes.cast(cnt, ctypes.c_void_p),
                                   ctypes.cast(fl, ctypes.c_void_p), n)
    if rc != 0:
        raise UpipeError(rc, "upipe_profile_stop")
    return {k: {"ms": ms[i], "launches": int(cnt[i]), "flops": fl[i]} for i, k in enumerate(KERNEL_KINDS)}
