"""Test-infrastructure oracle (CPU float64).  Importable only from tests/, the smoke check and
the bench's cpu_baseline leg; the product path never imports it."""
from .gqa_oracle import (ROPE_KINDS, ROT_STYLES, allowed_mask, attn_decode, attn_decode_one,  # noqa: F401
                         attn_prefill, rms_norm, rope_angles, rope_attention_factor,
                         rope_inv_freq, rotate, softmax_attention, yarn_softmax_scale)
