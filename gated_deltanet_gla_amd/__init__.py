"""MI355X (gfx950) gated linear-attention state recurrence: GLA and Gated
DeltaNet chunked prefill, slot-indexed decode, and the causal conv prelude.

The computation runs in the HIP library ``libgla_mi355x.so`` (C ABI in
include/gla.h); ``ops`` is its thin torch binding.
"""
from .ops import (gla_chunk_fwd, gdn_chunk_fwd, gla_decode_step, gdn_decode_step,  # noqa: F401
                  gla_chunk_fwd_ckpt, gdn_chunk_fwd_ckpt, gdn_chunk_prep, gdn_chunk_run, gla_decode_multi, gdn_decode_multi,
                  gla_state_copy, gla_slot_copy, lin_attn_chunk_fwd, lin_attn_decode_step, causal_conv1d_fwd,
                  workspace_bytes, gla_hbm_probe, gla_chunk_fwd_noalloc)

__version__ = "0.2.0"
