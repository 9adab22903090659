"""CPU fp64 oracle for DFlash draft block attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute it. It shares no code with the HIP
library and never imports it.
"""
from .dflash_oracle import (  # noqa: F401
    rms_norm,
    rope_inv_freq,
    rope_neox,
    qk_norm_rope,
    context_projection,
    context_kv,
    attention_visibility,
    block_attention,
    draft_block_attention,
    paged_context_rows,
    residual_rms_norm,
    block_qkv,
    output_projection,
    draft_layer_attention,
    PAD_SLOT,
    prepare_dflash_inputs,
    fc_combine,
    bf16_round,
)
