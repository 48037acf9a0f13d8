"""Token-by-token recurrences in fp64 (oracle; test infrastructure only).

Source: "Inference for linear attention and hybrid architectures",
section "Two ways to write the same computation":
  - softmax-free attention accumulates sum_s k_s^T v_s into a d_k x d_v state;
  - GLA update S_t = alpha_t S_{t-1} + k_t^T v_t with one scalar gate per token;
  - DeltaNet update (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t, and the
    gated variant multiplies in alpha_t as well (read: on the old state);
  - the recurrent algorithm: for each t, update S, then o_t = q_t S.
Section "Speculative decoding and PD disaggregation": batched decode reads
and writes each request's state in a pool by slot index; verifying draft
tokens needs the state of every draft position kept (or a replay), since an
applied update cannot be taken back.  Section "Prefix caching has to be
redone": a saved state is reused whole, and each continuation needs its own
copy.

Shapes (packed, token-major): q, k [T, H, dk]; v [T, H, dv]; alpha, beta
[T, H]; S [H, dk, dv].  Inputs of any float dtype are upcast to fp64.
Heads are independent; the loops vectorise over heads only.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def gla_sequence(q, k, v, alpha, S0=None):
    """GLA over one sequence: returns (o [T,H,dv], S_T [H,dk,dv]) in fp64."""
    q, k, v, alpha = _f64(q), _f64(k), _f64(v), _f64(alpha)
    T, H, dk = q.shape
    dv = v.shape[2]
    S = np.zeros((H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((T, H, dv))
    for t in range(T):
        # S_t = alpha_t S_{t-1} + k_t^T v_t  (outer product of the row vectors)
        S = alpha[t][:, None, None] * S + k[t][:, :, None] * v[t][:, None, :]
        # o_t = q_t S_t
        o[t] = np.einsum("hd,hde->he", q[t], S)
    return o, S


def gdn_sequence(q, k, v, alpha, beta, S0=None):
    """Gated DeltaNet over one sequence: returns (o, S_T) in fp64.

    S_t = alpha_t (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t, applied
    as erase-then-write: p = k_t S_{t-1} is what the state currently returns
    for key k_t, so (I - beta k^T k) S = S - beta k^T p.
    """
    q, k, v, alpha, beta = _f64(q), _f64(k), _f64(v), _f64(alpha), _f64(beta)
    T, H, dk = q.shape
    dv = v.shape[2]
    S = np.zeros((H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((T, H, dv))
    for t in range(T):
        a = alpha[t][:, None, None]
        b = beta[t][:, None, None]
        p = np.einsum("hd,hde->he", k[t], S)                        # k_t S_{t-1}
        erased = S - b * (k[t][:, :, None] * p[:, None, :])         # (I - b k^T k) S
        S = a * erased + b * (k[t][:, :, None] * v[t][:, None, :])  # gate, then write
        o[t] = np.einsum("hd,hde->he", q[t], S)
    return o, S


def _varlen(step_fn, q, k, v, gates, cu_seqlens, pool, slot_idx, zero_init):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    slots = np.asarray(slot_idx, dtype=np.int64)
    T, H, _ = np.shape(q)
    dv = np.shape(v)[2]
    o = np.zeros((T, H, dv))
    pool_out = _f64(pool).copy()
    for b in range(cu.shape[0] - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        S0 = None if zero_init else pool_out[slots[b]]
        if e == s:       # an empty sequence leaves its state as it was
            pool_out[slots[b]] = np.zeros_like(pool_out[slots[b]]) if zero_init else S0
            continue
        ob, Sb = step_fn(q[s:e], k[s:e], v[s:e], *[g[s:e] for g in gates], S0=S0)
        o[s:e] = ob
        pool_out[slots[b]] = Sb
    return o, pool_out


def gla_varlen(q, k, v, alpha, cu_seqlens, pool, slot_idx, zero_init=False):
    """Packed variable-length GLA: sequence b is rows cu[b]:cu[b+1]; its
    initial state is pool[slot_idx[b]] (zeros if ``zero_init``) and its final
    state is written back to the same slot.  Returns (o, pool_out) in fp64;
    slots not named in slot_idx are copied unchanged."""
    return _varlen(gla_sequence, q, k, v, [_f64(alpha)], cu_seqlens, pool, slot_idx, zero_init)


def gdn_varlen(q, k, v, alpha, beta, cu_seqlens, pool, slot_idx, zero_init=False):
    """Packed variable-length Gated DeltaNet; same contract as gla_varlen."""
    return _varlen(gdn_sequence, q, k, v, [_f64(alpha), _f64(beta)], cu_seqlens, pool,
                   slot_idx, zero_init)


def gla_decode(q, k, v, alpha, pool, slot_idx):
    """One decode token per request r (rows of q): a single GLA step on
    pool[slot_idx[r]].  Returns (o [R,H,dv], pool_out)."""
    R = np.shape(q)[0]
    cu = np.arange(R + 1)
    return gla_varlen(q, k, v, alpha, cu, pool, slot_idx, zero_init=False)


def gdn_decode(q, k, v, alpha, beta, pool, slot_idx):
    """One Gated DeltaNet decode step per request on pool[slot_idx[r]]."""
    R = np.shape(q)[0]
    cu = np.arange(R + 1)
    return gdn_varlen(q, k, v, alpha, beta, cu, pool, slot_idx, zero_init=False)


def _decode_multi(step_fn, q, k, v, gates, pool, slot_idx, pos_slots):
    """n_tok tokens per request r (axis 1 of q), starting from
    pool[slot_idx[r]]; after token j the state is stored in
    pool[pos_slots[r, j]] when that index is in range.  The request's own
    slot is not written unless pos_slots names it.  Returns (o, pool_out)."""
    q = _f64(q)
    R, J, H, _ = q.shape
    dv = np.shape(v)[3]
    n_slots = np.shape(pool)[0]
    pool_in = _f64(pool)
    pool_out = pool_in.copy()
    o = np.zeros((R, J, H, dv))
    for r in range(R):
        S = pool_in[int(slot_idx[r])].copy()
        for j in range(J):
            # one recurrence step = the sequence function over one token
            o1, S = step_fn(q[r, j:j + 1], k[r, j:j + 1], v[r, j:j + 1],
                            *[g[r, j:j + 1] for g in gates], S0=S)
            o[r, j] = o1[0]
            ps = int(pos_slots[r, j])
            if 0 <= ps < n_slots:
                pool_out[ps] = S
    return o, pool_out


def gla_decode_multi(q, k, v, alpha, pool, slot_idx, pos_slots):
    """Several GLA tokens per request with every position's state kept:
    q, k [R, J, H, dk]; v [R, J, H, dv]; alpha [R, J, H]; pos_slots [R, J]."""
    return _decode_multi(gla_sequence, q, k, v, [_f64(alpha)], pool, slot_idx, pos_slots)


def gdn_decode_multi(q, k, v, alpha, beta, pool, slot_idx, pos_slots):
    """Gated DeltaNet form of gla_decode_multi; beta [R, J, H]."""
    return _decode_multi(gdn_sequence, q, k, v, [_f64(alpha), _f64(beta)], pool, slot_idx,
                         pos_slots)


def state_copy(pool, src_slots, dst_slots):
    """pool[dst[i]] <- pool[src[i]] for every pair with both slots in range
    (all reads before any write).  Returns the new pool (fp64)."""
    pool_in = _f64(pool)
    out = pool_in.copy()
    n = pool_in.shape[0]
    for s, d in zip(np.asarray(src_slots).tolist(), np.asarray(dst_slots).tolist()):
        if 0 <= s < n and 0 <= d < n:
            out[d] = pool_in[s]
    return out


def _varlen_ckpt(step_fn, q, k, v, gates, cu_seqlens, pool, slot_idx, ckpt_slots, interval,
                 zero_init):
    """Packed varlen recurrence that also saves the state after every
    ``interval`` tokens of sequence b into pool[ckpt_slots[b, j]] (j-th
    checkpoint; entries outside the pool save nothing).  Each sequence is
    run piece by piece, handing only the state on, and the state at the end
    of each full piece is the checkpoint."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    slots = np.asarray(slot_idx, dtype=np.int64)
    ck = np.asarray(ckpt_slots, dtype=np.int64)
    T, H, _ = np.shape(q)
    dv = np.shape(v)[2]
    o = np.zeros((T, H, dv))
    pool_in = _f64(pool)
    pool_out = pool_in.copy()
    n_slots = pool_in.shape[0]
    for b in range(cu.shape[0] - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        S = np.zeros_like(pool_in[slots[b]]) if zero_init else pool_in[slots[b]].copy()
        for j, p in enumerate(range(s, e, interval)):
            pe = min(p + interval, e)
            o[p:pe], S = step_fn(q[p:pe], k[p:pe], v[p:pe], *[g[p:pe] for g in gates], S0=S)
            if pe - p == interval and j < ck.shape[1] and 0 <= ck[b, j] < n_slots:
                pool_out[ck[b, j]] = S
        pool_out[slots[b]] = S
    return o, pool_out


def gla_varlen_ckpt(q, k, v, alpha, cu_seqlens, pool, slot_idx, ckpt_slots, interval,
                    zero_init=False):
    """gla_varlen plus state checkpoints every ``interval`` tokens
    (ckpt_slots [B, stride])."""
    return _varlen_ckpt(gla_sequence, q, k, v, [_f64(alpha)], cu_seqlens, pool, slot_idx,
                        ckpt_slots, interval, zero_init)


def gdn_varlen_ckpt(q, k, v, alpha, beta, cu_seqlens, pool, slot_idx, ckpt_slots, interval,
                    zero_init=False):
    """gdn_varlen plus state checkpoints every ``interval`` tokens."""
    return _varlen_ckpt(gdn_sequence, q, k, v, [_f64(alpha), _f64(beta)], cu_seqlens, pool,
                        slot_idx, ckpt_slots, interval, zero_init)
