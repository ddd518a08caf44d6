"""Test-infrastructure oracle (CPU float64).  Importable only from tests/, the smoke check and
the bench's cpu_baseline leg; the product path never imports it."""
from .gqa_oracle import (ROPE_KINDS, ROT_STYLES, allowed_mask, append_rows,  # noqa: F401
                         attn_decode, attn_decode_one, attn_decode_paged, attn_prefill,
                         mla_decode, mla_decode_one, MLA_LATENT, MLA_ROPE,
                         paged_rows, paged_update, rms_norm, rope_angles, rope_attention_factor,
                         rope_inv_freq, rotate, softmax_attention, yarn_softmax_scale)
