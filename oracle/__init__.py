"""fp64 CPU oracle for the gated linear-attention state recurrence.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the tests, the smoke check and the benchmark's CPU-baseline leg call it.
It shares no code with the HIP library.

What it computes follows "Inference for linear attention and hybrid
architectures", section "Two ways to write the same computation":

* GLA:  S_t = alpha_t S_{t-1} + k_t^T v_t,  o_t = q_t S_t (state read after
  the update).
* Gated DeltaNet: S_t = alpha_t (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t
  (the gate multiplies the old-state term only; that placement is a reading,
  the page only says a decay gate is multiplied in as well).
* the short causal convolution in front of the layer, with its per-request
  cache of the last width-1 inputs (same section, last paragraph; section
  "The real model's ledger" for the width-1 cache).

The definition is the token-by-token recurrence (``recurrence``); the chunked
forms in ``chunked`` evaluate the same recurrence chunk by chunk (GLA from
direct products of the gates, and a derived chunked form for Gated
DeltaNet) and exist only to pin the recurrence.

Parity status of every function is listed in ``PINS`` below: each entry names
the pin tests that fix it against something other than itself.
"""
from .recurrence import (gla_sequence, gdn_sequence, gla_varlen, gdn_varlen,
                         gla_decode, gdn_decode, gla_decode_multi, gdn_decode_multi, state_copy,
                         gla_varlen_ckpt, gdn_varlen_ckpt)
from .conv import causal_conv1d
from .linear import phi, lin_attn_sequence, lin_attn_varlen, lin_attn_decode
from .chunked import gla_chunked, gdn_chunked

PINS = {
    "gla_sequence": "brute-force O(T^2) sum, alpha=1 masked matmul, scipy lfilter (d=1), "
                    "page toy example recurrent==chunked at 1e-5, segmentation",
    "gdn_sequence": "literal d_k x d_k matrix update, beta=0 closed form, orthogonal-key "
                    "reduction to GLA, retrieval identity, chunked WY form",
    "gla_varlen / gdn_varlen": "per-sequence equality with *_sequence, untouched slots, "
                               "empty sequences; zero_init against the brute-force sum (GLA) and "
                               "the literal matrix update (GDN) run from zero with a nonzero pool",
    "gla_decode / gdn_decode": "one step of *_sequence",
    "gla_decode_multi / gdn_decode_multi": "each kept state equals the varlen prefill of the "
                                           "same prefix, closed form of the GLA state after j "
                                           "tokens, rollback-and-replay, untouched slots",
    "state_copy": "element values and untouched slots by construction of the pool",
    "gla_varlen_ckpt / gdn_varlen_ckpt": "checkpoints against the GLA closed form and the "
                                         "literal GDN matrix update; continuing from a copy "
                                         "of a checkpoint equals the uncut run (the page's "
                                         "prefix-cache demonstration); outputs equal "
                                         "*_varlen",
    "lin_attn_sequence": "the page's parallel kernelised formula (O(T^2) double sum), "
                         "the closed form from a given (S0, z0), convex-combination bounds, "
                         "constant values, phi against torch's elu + 1",
    "lin_attn_varlen": "segmentation through the pool; zero_init against the double sum from "
                       "zero with nonzero pools",
    "lin_attn_decode": "one step's closed form S0 + phi(k)^T v, z0 + phi(k), "
                       "phi(q)S / (phi(q).z + eps) on each slot; untouched slots",
    "causal_conv1d": "numpy.convolve per channel, segmented == one pass == token by token; "
                     "zero_init against numpy.convolve with a nonzero cache",
    "gla_chunked": "page toy example; equality with the recurrence",
    "gdn_chunked": "equality with the recurrence (the chunked GDN form itself is not on the "
                   "page; it is pinned only through the recurrence)",
}
