"""Headwise-chunked causal RoPE/GQA attention (Untied Ulysses / UPipe) for MI355X.

The compute path is the HIP library ``libupipe.so`` (C ABI in
``include/upipe.h``); ``api`` is its ctypes binding and ``synth`` the seeded
input generator shared with the tests.
"""
from .api import (  # noqa: F401
    UPIPE_BF16,
    UPIPE_F32,
    UpipeError,
    attn_bwd,
    attn_fwd,
    load,
    strerror,
    workspace_bytes,
)

__all__ = ["attn_fwd", "attn_bwd", "workspace_bytes", "load", "strerror", "UpipeError"]
