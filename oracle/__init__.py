"""CPU fp64 oracle of the attention layer's forward pass and the steps around it.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product library.
"""

from .qknorm_rope_attn import (  # noqa: F401
    split_qkv,
    rms_norm,
    rope_frequencies,
    rope_rotate_half,
    qk_norm_rope,
    softmax,
    causal_gqa_attention,
    attend_prefix,
    prefill,
    prefill_rows,
    decode,
    prefill_append,
    round_to_bf16,
)
from . import paged  # noqa: F401
from .layer_ops import (  # noqa: F401
    fused_add_rms_norm,
    last_positions,
    gather_last,
    greedy_argmax,
)
