"""CPU fp64 oracle for headwise-chunked causal RoPE/GQA attention, the
sequence-tiled gated-SiLU MLP, the sequence-tiled cross-entropy loss and the
checkpointed pre-norm transformer block built from the first two.

TEST INFRASTRUCTURE ONLY. Nothing in the product package imports this; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.
"""
from .attention import (  # noqa: F401
    rope_cos_sin,
    apply_rope,
    rope_transpose,
    rmsnorm,
    rmsnorm_bwd,
    causal_attention,
    causal_attention_bwd,
    layer_fwd,
    layer_bwd,
    layer_fwd_rows,
    layer_bwd_tail_dx,
    chunk_plan,
)
from .mlp import (  # noqa: F401
    sigmoid,
    silu,
    silu_grad,
    mlp_fwd,
    mlp_bwd,
    mlp_rows,
    mlp_dx_rows,
)
from .loss import (  # noqa: F401
    ce_fwd,
    ce_bwd,
    ce_rows,
    ce_dh_rows,
)
from .block import (  # noqa: F401
    block_fwd,
    block_bwd,
    stack_fwd,
    stack_bwd,
)
