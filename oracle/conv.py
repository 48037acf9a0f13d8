"""Depthwise causal convolution with a per-request cache (oracle; test
infrastructure only).

Source: "Inference for linear attention and hybrid architectures",
section "Two ways to write the same computation" (a short causal convolution,
window about 4, precedes the layer and keeps the inputs of the last few
tokens of each request), and section "The real model's ledger" (an engine
needs to keep width-1 columns).

Reading (the pages fix no tap order, bias or activation): for width W,
  y[t, c] = sum_{i=0}^{W-1} w[c, i] * xx[t + i, c]
where xx is the sequence's inputs preceded by the W-1 cached rows, so
w[:, W-1] multiplies the current token.  No bias, no activation.  After the
call the cache holds the last W-1 rows of xx.
"""
from __future__ import annotations

import numpy as np


def causal_conv1d(x, w, cu_seqlens, cache, slot_idx, zero_init=False):
    """x [N, C]; w [C, W]; cache [n_slots, W-1, C]; returns (y [N, C] fp64,
    cache_out fp64).  Sequence b uses and updates cache[slot_idx[b]]
    (treated as zeros if ``zero_init``)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    cache_out = np.asarray(cache, dtype=np.float64).copy()
    W = w.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    y = np.zeros_like(x)
    for b in range(cu.shape[0] - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        slot = int(slot_idx[b])
        prev = np.zeros((W - 1, x.shape[1])) if zero_init else cache_out[slot]
        xx = np.concatenate([prev, x[s:e]], axis=0)
        for t in range(e - s):
            acc = np.zeros(x.shape[1])
            for i in range(W):
                acc += w[:, i] * xx[t + i]
            y[s + t] = acc
        cache_out[slot] = xx[xx.shape[0] - (W - 1):]
    return y, cache_out
