"""One mixed serving step of a Gated DeltaNet layer: the causal conv
prelude over every request, the chunked prefill for the prompts and the
recurrent decode for the one-token requests.

"Inference for linear attention and hybrid architectures": prefill uses the
chunked form and decode the recurrent form (section "Two ways to write the
same computation"; the short conv and its cache in the same section), and
both read and write each request's state by pool slot (section "Speculative
decoding and PD disaggregation").  Prompts are packed first, then the decode
tokens.  This module only sequences the library's entry points; the
prefill and decode parts touch disjoint slots, so the decode runs on a
second stream concurrently with the prefill.
"""
from __future__ import annotations

import torch

from .ops import causal_conv1d_fwd, gdn_chunk_fwd, gdn_decode_step


class MixedStep:
    """Holds the fixed-size buffers of one mixed step so repeated calls do
    not allocate.  Shapes: x [N, H*dv]; q, k [N, H, dk]; alpha, beta [N, H];
    cu_all [B+1] (prompts then decodes); slots [B]; n_prefill prompts whose
    tokens are rows [0, n_prefill_tokens)."""

    def __init__(self, x, conv_w, conv_cache, q, k, alpha, beta, cu_all, cu_prefill, pool, slots,
                 n_prefill, n_prefill_tokens, *, chunk=64, out_dtype=torch.bfloat16):
        self.x, self.conv_w, self.conv_cache = x, conv_w, conv_cache
        self.q, self.k, self.alpha, self.beta = q, k, alpha, beta
        self.cu_all, self.cu_prefill = cu_all, cu_prefill
        self.pool, self.slots = pool, slots
        self.P, self.NP = n_prefill, n_prefill_tokens
        N, H, dk = q.shape
        self.H = H
        self.dv = x.shape[1] // H
        self.chunk = chunk
        self.y = torch.empty_like(x)
        self.o = torch.empty((N, H, self.dv), dtype=out_dtype, device=x.device)
        self.side = torch.cuda.Stream(device=x.device)
        self.ev = torch.cuda.Event()
        self.done = torch.cuda.Event()
        from . import ops
        need = ops.workspace_bytes("gdn", n_prefill, n_prefill_tokens, H, dk, self.dv, chunk)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)

    def __call__(self):
        NP, P = self.NP, self.P
        N, H, dv = self.o.shape
        causal_conv1d_fwd(self.x, self.conv_w, self.cu_all, self.conv_cache, self.slots, y=self.y)
        v = self.y.view(N, H, dv)
        main = torch.cuda.current_stream(self.x.device)
        self.ev.record(main)
        with torch.cuda.stream(self.side):
            self.side.wait_event(self.ev)
            if N > NP:
                gdn_decode_step(self.q[NP:], self.k[NP:], v[NP:], self.alpha[NP:], self.beta[NP:],
                                self.pool, self.slots[P:], o=self.o[NP:])
            self.done.record(self.side)
        if P > 0:
            gdn_chunk_fwd(self.q[:NP], self.k[:NP], v[:NP], self.alpha[:NP], self.beta[:NP],
                          self.cu_prefill, self.pool, self.slots[:P], chunk=self.chunk,
                          o=self.o[:NP], workspace=self.ws)
        main.wait_event(self.done)
        return self.o
