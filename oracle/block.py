"""Plain fp64 CPU oracle of one checkpointed pre-norm transformer block.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` (and nothing in the product
path).

What it computes
----------------
The talk trains Llama-family models and stacks its memory techniques around
the transformer block: the attention op with chunked heads, activation
checkpointing that recomputes a block's activations from its input in the
backward pass, CPU offload of those block inputs, and sequence tiling of the
MLP ("Road to 5 Million Tokens", talk transcript, the memory-optimization
progression; liquidgold.cc notes, "Progression of Techniques", items 4-6).
The pages do not write the block out. The plainest reading is the Llama
pre-norm block without biases:

    a = rmsnorm(x; g_attn)          h = x + attn(a)
    b = rmsnorm(h; g_mlp)           y = h + mlp(b)

with ``attn`` the attention layer of ``oracle.attention`` (RoPE, GQA, causal,
optional q/k norm) and ``mlp`` the gated-SiLU MLP of ``oracle.mlp``;
``rmsnorm(u; g) = g * u / sqrt(mean(u^2) + eps)`` over d_model. Checkpointing
and tiling are schedules: the backward below is the exact gradient of this
forward for an upstream gradient dy,

    db = mlp_bwd(b, dy).dx,          dh = dy + rmsnorm_bwd(h, g_mlp, db)
    da = attn_bwd(a, dh).dx,         dx = dh + rmsnorm_bwd(x, g_attn, da)

plus the weight gradients of both sublayers and of the two norm weights.

``stack_fwd`` / ``stack_bwd`` chain blocks: the stack keeps only each
block's input between the passes (what the talk offloads to the CPU), and
block l's backward starts from that input and from the gradient block l + 1
passes down.

Parity pins: ``tests/test_oracle_block.py`` checks the composition through
special cases that reduce it to the pinned sublayer oracles (zero output
weights give y = x; a zero attention norm weight removes the attention
branch), exact homogeneity identities of the weight gradients, and central
finite differences of every gradient, and the stack's chain rule by
finite differences through two blocks; none is "parity unpinned".

Layouts: x, y, h, dy, dx [N][D]; g_attn, g_mlp [D]; attention weights as in
``oracle.attention``; MLP weights as in ``oracle.mlp``; lse [Hq][N].
"""
from __future__ import annotations

import numpy as np

from .attention import layer_bwd, layer_fwd, rmsnorm, rmsnorm_bwd
from .mlp import mlp_bwd, mlp_fwd

F64 = np.float64


def block_fwd(x, g_attn, wq, wk, wv, wo, g_mlp, wg, wu, wd, n_q_heads, n_kv_heads, head_dim,
              rope_theta, chunk_heads=1, q_norm=None, k_norm=None, qk_eps=1e-6, eps=1e-5,
              tile=None):
    """Forward of the block: ``(y, h, lse)`` with h the residual stream after attention."""
    x = np.asarray(x, dtype=F64)
    a = rmsnorm(x, g_attn, eps)
    att, lse = layer_fwd(a, wq, wk, wv, wo, n_q_heads, n_kv_heads, head_dim, rope_theta,
                         chunk_heads, q_norm, k_norm, qk_eps)
    h = x + att
    b = rmsnorm(h, g_mlp, eps)
    y = h + mlp_fwd(b, wg, wu, wd, tile)
    return y, h, lse


def block_bwd(x, g_attn, wq, wk, wv, wo, g_mlp, wg, wu, wd, dy, n_q_heads, n_kv_heads, head_dim,
              rope_theta, chunk_heads=1, q_norm=None, k_norm=None, qk_eps=1e-6, eps=1e-5,
              tile=None):
    """Exact backward of ``block_fwd`` from the block input alone (checkpointing).

    Returns a dict with ``dx`` and the gradients of every weight: ``g_attn,
    wq, wk, wv, wo, q_norm, k_norm, g_mlp, wg, wu, wd`` (the q/k norm entries
    are None without q/k norm).
    """
    x = np.asarray(x, dtype=F64)
    dy = np.asarray(dy, dtype=F64)
    # recompute the forward from x
    a = rmsnorm(x, g_attn, eps)
    att, _ = layer_fwd(a, wq, wk, wv, wo, n_q_heads, n_kv_heads, head_dim, rope_theta,
                       chunk_heads, q_norm, k_norm, qk_eps)
    h = x + att
    b = rmsnorm(h, g_mlp, eps)
    # MLP branch, then its norm; the residual passes dy through unchanged
    db, dwg, dwu, dwd = mlp_bwd(b, wg, wu, wd, dy, tile)
    dh_n, dg_mlp = rmsnorm_bwd(h, g_mlp, eps, db)
    dh = dy + dh_n
    # attention branch, then its norm
    da, dwq, dwk, dwv, dwo, dqn, dkn = layer_bwd(a, wq, wk, wv, wo, dh, n_q_heads, n_kv_heads,
                                                 head_dim, rope_theta, chunk_heads, q_norm,
                                                 k_norm, qk_eps)
    dx_n, dg_attn = rmsnorm_bwd(x, g_attn, eps, da)
    return {"dx": dh + dx_n, "g_attn": dg_attn, "wq": dwq, "wk": dwk, "wv": dwv, "wo": dwo,
            "q_norm": dqn, "k_norm": dkn, "g_mlp": dg_mlp, "wg": dwg, "wu": dwu, "wd": dwd}


def stack_fwd(x, layers, n_q_heads, n_kv_heads, head_dim, rope_theta, chunk_heads=1, qk_eps=1e-6,
              eps=1e-5, tile=None):
    """A stack of blocks: ``(y, inputs)`` with ``inputs[l]`` the input of block l.

    ``layers`` is a list of dicts with the keys ``g_attn, wq, wk, wv, wo,
    q_norm, k_norm, g_mlp, wg, wu, wd``. Checkpointing keeps exactly the
    block inputs (the talk offloads them to the CPU between the passes).
    """
    inputs = []
    h = np.asarray(x, dtype=F64)
    for w in layers:
        inputs.append(h)
        h, _, _ = block_fwd(h, w["g_attn"], w["wq"], w["wk"], w["wv"], w["wo"], w["g_mlp"], w["wg"], w["wu"],
                            w["wd"], n_q_heads, n_kv_heads, head_dim, rope_theta, chunk_heads, w["q_norm"],
                            w["k_norm"], qk_eps, eps, tile)
    return h, inputs


def stack_bwd(x, layers, dy, n_q_heads, n_kv_heads, head_dim, rope_theta, chunk_heads=1, qk_eps=1e-6,
              eps=1e-5, tile=None):
    """Backward of ``stack_fwd``: ``(dx, grads)`` with ``grads[l]`` the dict
    ``block_bwd`` returns for block l (without its ``dx``). Block l's backward
    starts from its kept input and the gradient that block l + 1 passed down."""
    _, inputs = stack_fwd(x, layers, n_q_heads, n_kv_heads, head_dim, rope_theta, chunk_heads, qk_eps, eps, tile)
    g = np.asarray(dy, dtype=F64)
    grads = [None] * len(layers)
    for i in range(len(layers) - 1, -1, -1):
        w = layers[i]
        r = block_bwd(inputs[i], w["g_attn"], w["wq"], w["wk"], w["wv"], w["wo"], w["g_mlp"], w["wg"], w["wu"],
                      w["wd"], g, n_q_heads, n_kv_heads, head_dim, rope_theta, chunk_heads, w["q_norm"],
                      w["k_norm"], qk_eps, eps, tile)
        g = r.pop("dx")
        grads[i] = r
    return g, grads
