"""Normalised kernelised linear attention in fp64 (oracle; test
infrastructure only).

Source: page "Long context, fast inference, smart decoding, and life beyond
attention", chapter "Long-context architectures", section "Linear
attention: removing softmax entirely" (the kernelised formula, and its
statement that the same result can be kept as a running state): with the
feature map
phi(x) = elu(x) + 1 (positive, so the normaliser cannot vanish),
    S_i = S_{i-1} + phi(k_i)^T v_i,     z_i = z_{i-1} + phi(k_i),
    o_i = phi(q_i) S_i / (phi(q_i) . z_i + eps),   eps = 1e-6 on the page,
which equals the kernelised attention
    o_i = sum_{j<=i} (phi(q_i).phi(k_j)) v_j / (sum_{j<=i} phi(q_i).phi(k_j) + eps)
when S and z start at zero.  There is no gate.  A d_k x d_v state S and a
d_k normaliser z per head; starting values may come from a pool slot.

Shapes (packed, token-major): q, k [T, H, dk]; v [T, H, dv]; S [H, dk, dv];
z [H, dk].
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def phi(x):
    """elu(x) + 1: x + 1 for x > 0, exp(x) otherwise."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def lin_attn_sequence(q, k, v, S0=None, z0=None, eps=EPS, block=64):
    """One sequence.  Returns (o [T,H,dv], S_T, z_T).

    The state and normaliser after token i are prefix sums over the tokens
    so far, S_i = S_0 + sum_{j<=i} phi(k_j)^T v_j and z_i = z_0 + sum_{j<=i}
    phi(k_j), taken with a sequential cumulative sum (so cutting the sequence
    anywhere and carrying (S, z) gives bit-identical results); the output
    reads them after the token's own write, o_i = phi(q_i) S_i / (phi(q_i) .
    z_i + eps).  Tokens are taken ``block`` at a time only to bound memory.
    """
    q, k, v = np.asarray(q, np.float64), np.asarray(k, np.float64), np.asarray(v, np.float64)
    T, H, dk = q.shape
    dv = v.shape[2]
    S = np.zeros((H, dk, dv)) if S0 is None else np.asarray(S0, np.float64).copy()
    z = np.zeros((H, dk)) if z0 is None else np.asarray(z0, np.float64).copy()
    fq, fk = phi(q), phi(k)
    o = np.zeros((T, H, dv))
    for s in range(0, T, block):
        e = min(s + block, T)
        writes = fk[s:e, :, :, None] * v[s:e, :, None, :]                  # phi(k_j)^T v_j
        S_run = np.cumsum(np.concatenate([S[None], writes]), axis=0)[1:]    # [n, H, dk, dv]
        z_run = np.cumsum(np.concatenate([z[None], fk[s:e]]), axis=0)[1:]   # [n, H, dk]
        num = np.zeros((e - s, H, dv))
        den = np.full((e - s, H), eps)
        for d in range(dk):
            num += fq[s:e, :, d, None] * S_run[:, :, d, :]
            den += fq[s:e, :, d] * z_run[:, :, d]
        o[s:e] = num / den[:, :, None]
        S, z = S_run[-1], z_run[-1]
    return o, S, z


def lin_attn_varlen(q, k, v, cu_seqlens, pool, zpool, slot_idx, zero_init=False, eps=EPS):
    """Packed varlen form: sequence b starts from pool[slot_idx[b]] and
    zpool[slot_idx[b]] (zeros if zero_init) and writes both back.  Returns
    (o, pool_out, zpool_out) in fp64."""
    cu = np.asarray(cu_seqlens, np.int64)
    slots = np.asarray(slot_idx, np.int64)
    T, H, _ = np.shape(q)
    o = np.zeros((T, H, np.shape(v)[2]))
    pool_out = np.asarray(pool, np.float64).copy()
    zpool_out = np.asarray(zpool, np.float64).copy()
    for b in range(cu.shape[0] - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        sl = slots[b]
        S0 = None if zero_init else pool_out[sl]
        z0 = None if zero_init else zpool_out[sl]
        ob, Sb, zb = lin_attn_sequence(q[s:e], k[s:e], v[s:e], S0, z0, eps)
        o[s:e] = ob
        pool_out[sl], zpool_out[sl] = Sb, zb
    return o, pool_out, zpool_out


def lin_attn_decode(q, k, v, pool, zpool, slot_idx, eps=EPS):
    """One token per request r on pool[slot_idx[r]], zpool[slot_idx[r]]."""
    R = np.shape(q)[0]
    return lin_attn_varlen(q, k, v, np.arange(R + 1), pool, zpool, slot_idx, False, eps)
