"""Pins for the oracle: checks against facts that do not come from the
oracle itself (brute-force sums, closed forms, textbook/library routines,
the worked example of "Inference for linear attention and hybrid
architectures").  Each check takes the implementation under test as an
argument and returns the largest deviation it sees, so the same checks can
be run on deliberately broken copies of the oracle (see
test_oracle_mutants.py).
"""
from __future__ import annotations

import numpy as np
from scipy.signal import lfilter

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(seed, T=24, H=2, dk=6, dv=5, unit_k=False, state=True):
    r = _rng(seed)
    q = r.standard_normal((T, H, dk))
    k = r.standard_normal((T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    else:
        k *= 0.5
    v = r.standard_normal((T, H, dv))
    a = 1.0 / (1.0 + np.exp(-(r.standard_normal((T, H)) + 2.0)))
    b = 1.0 / (1.0 + np.exp(-r.standard_normal((T, H))))
    S0 = r.standard_normal((H, dk, dv)) * 0.3 if state else np.zeros((H, dk, dv))
    return q, k, v, a, b, S0


# ---------------------------------------------------------------- GLA pins
def gla_bruteforce(gla_sequence, seed=1):
    """o_t = sum_{s<=t} (prod_{r=s+1..t} alpha_r)(q_t.k_s) v_s
           + (prod_{r<=t} alpha_r) q_t S_0,  products taken directly."""
    q, k, v, a, _, S0 = _inputs(seed, dk=5, dv=5)   # square heads: a transposed outer product stays shape-valid
    o, S = gla_sequence(q, k, v, a, S0)
    T, H, _ = q.shape
    err = 0.0
    for h in range(H):
        for t in range(T):
            ref = np.prod(a[: t + 1, h]) * (q[t, h] @ S0[h])
            for s in range(t + 1):
                ref = ref + np.prod(a[s + 1: t + 1, h]) * (q[t, h] @ k[s, h]) * v[s, h]
            err = max(err, np.abs(o[t, h] - ref).max())
        Sref = np.prod(a[:, h]) * S0[h]
        for s in range(T):
            Sref = Sref + np.prod(a[s + 1:, h]) * np.outer(k[s, h], v[s, h])
        err = max(err, np.abs(S[h] - Sref).max())
    return err


def gla_linear_attention(gla_sequence, seed=2):
    """alpha = 1, S_0 = 0: plain causal linear attention, tril(Q K^T) V."""
    q, k, v, a, _, _ = _inputs(seed, state=False)
    ones = np.ones_like(a)
    o, S = gla_sequence(q, k, v, ones, None)
    err = 0.0
    for h in range(q.shape[1]):
        ref = np.tril(q[:, h] @ k[:, h].T) @ v[:, h]
        err = max(err, np.abs(o[:, h] - ref).max(), np.abs(S[h] - k[:, h].T @ v[:, h]).max())
    return err


def gla_lfilter(gla_sequence, seed=3):
    """d_k = d_v = 1 with a constant gate: the state is the first-order IIR
    filter y_t = a y_{t-1} + x_t (scipy.signal.lfilter) of x_t = k_t v_t."""
    r = _rng(seed)
    T = 40
    k = r.standard_normal((T, 1, 1))
    v = r.standard_normal((T, 1, 1))
    q = r.standard_normal((T, 1, 1))
    a0 = 0.87
    o, S = gla_sequence(q, k, v, np.full((T, 1), a0), None)
    y = lfilter([1.0], [1.0, -a0], (k * v)[:, 0, 0])
    return max(np.abs(o[:, 0, 0] - q[:, 0, 0] * y).max(), abs(S[0, 0, 0] - y[-1]))


# ---------------------------------------------------------------- GDN pins
def gdn_matrix_form(gdn_sequence, seed=4):
    """Literal update with the d_k x d_k matrix alpha (I - beta k^T k)."""
    q, k, v, a, b, S0 = _inputs(seed)
    o, S = gdn_sequence(q, k, v, a, b, S0)
    T, H, dk = q.shape
    err = 0.0
    for h in range(H):
        St = S0[h].copy()
        for t in range(T):
            kk = k[t, h][:, None]
            M = a[t, h] * (np.eye(dk) - b[t, h] * (kk @ kk.T))
            St = M @ St + b[t, h] * (kk @ v[t, h][None, :])
            err = max(err, np.abs(o[t, h] - q[t, h] @ St).max())
        err = max(err, np.abs(S[h] - St).max())
    return err


def gdn_unrolled(gdn_sequence, seed=5):
    """Unrolled closed form S_T = M_T..M_1 S_0 + sum_t M_T..M_{t+1} beta_t k_t^T v_t,
    with M_t = alpha_t (I - beta_t k_t^T k_t), products formed explicitly."""
    q, k, v, a, b, S0 = _inputs(seed, T=10, H=1)
    _, S = gdn_sequence(q, k, v, a, b, S0)
    dk = q.shape[2]
    Ms = [a[t, 0] * (np.eye(dk) - b[t, 0] * np.outer(k[t, 0], k[t, 0])) for t in range(q.shape[0])]

    def prod(lo, hi):          # M_hi ... M_lo (inclusive), identity if empty
        P = np.eye(dk)
        for t in range(lo, hi + 1):
            P = Ms[t] @ P
        return P
    T = q.shape[0]
    ref = prod(0, T - 1) @ S0[0]
    for t in range(T):
        ref = ref + prod(t + 1, T - 1) @ (b[t, 0] * np.outer(k[t, 0], v[t, 0]))
    return np.abs(S[0] - ref).max()


def gdn_beta_zero(gdn_sequence, seed=6):
    """beta = 0: no erase and no write, o_t = (prod_{r<=t} alpha_r) q_t S_0."""
    q, k, v, a, _, S0 = _inputs(seed)
    o, S = gdn_sequence(q, k, v, a, np.zeros_like(a), S0)
    err = 0.0
    for h in range(q.shape[1]):
        for t in range(q.shape[0]):
            err = max(err, np.abs(o[t, h] - np.prod(a[: t + 1, h]) * (q[t, h] @ S0[h])).max())
    return err


def _orthogonal_keys(seed, T, H, dk, unit=False):
    r = _rng(seed)
    k = np.zeros((T, H, dk))
    for h in range(H):
        Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
        scale = np.ones(T) if unit else r.uniform(0.5, 1.4, T)
        k[:, h] = Qm[:T] * scale[:, None]
    return k


def gdn_orthogonal_keys(gdn_sequence, gla_sequence, seed=7):
    """Mutually orthogonal keys and S_0 = 0: nothing is erased, so Gated
    DeltaNet equals GLA fed with values beta_t v_t."""
    q, _, v, a, b, _ = _inputs(seed, T=8, dk=8)
    k = _orthogonal_keys(seed, 8, q.shape[1], 8)
    o1, S1 = gdn_sequence(q, k, v, a, b, None)
    o2, S2 = gla_sequence(q, k, b[:, :, None] * v, a, None)
    return max(np.abs(o1 - o2).max(), np.abs(S1 - S2).max())


def gdn_linear_attention(gdn_sequence, seed=8):
    """Orthonormal keys, alpha = beta = 1, S_0 = 0: plain causal linear
    attention tril(Q K^T) V."""
    q, _, v, a, _, _ = _inputs(seed, T=8, dk=8)
    k = _orthogonal_keys(seed, 8, q.shape[1], 8, unit=True)
    ones = np.ones_like(a)
    o, _ = gdn_sequence(q, k, v, ones, ones, None)
    err = 0.0
    for h in range(q.shape[1]):
        err = max(err, np.abs(o[:, h] - np.tril(q[:, h] @ k[:, h].T) @ v[:, h]).max())
    return err


def gdn_retrieval(gdn_sequence, seed=9):
    """k_t S_t = alpha_t (1 - beta_t |k_t|^2) k_t S_{t-1} + beta_t |k_t|^2 v_t at
    every step, from states obtained by running one token at a time."""
    q, k, v, a, b, S0 = _inputs(seed)
    err = 0.0
    S = S0.copy()
    for t in range(q.shape[0]):
        _, Sn = gdn_sequence(q[t:t + 1], k[t:t + 1], v[t:t + 1], a[t:t + 1], b[t:t + 1], S)
        for h in range(q.shape[1]):
            kk = k[t, h] @ k[t, h]
            ref = a[t, h] * (1 - b[t, h] * kk) * (k[t, h] @ S[h]) + b[t, h] * kk * v[t, h]
            err = max(err, np.abs(k[t, h] @ Sn[h] - ref).max())
        S = Sn
    return err


def gdn_overwrite(gdn_sequence, seed=10):
    """alpha = beta = 1 and |k| = 1: exact overwrite, k_t S_t = v_t."""
    q, k, v, a, _, S0 = _inputs(seed, unit_k=True)
    ones = np.ones_like(a)
    err = 0.0
    S = S0.copy()
    for t in range(q.shape[0]):
        _, S = gdn_sequence(q[t:t + 1], k[t:t + 1], v[t:t + 1], ones[t:t + 1], ones[t:t + 1], S)
        for h in range(q.shape[1]):
            err = max(err, np.abs(k[t, h] @ S[h] - v[t, h]).max())
    return err


# ---------------------------------------------------------------- conv pin
def conv_numpy_convolve(causal_conv1d, seed=11):
    """Zero cache: channel c is numpy.convolve(x[:, c], w[c, ::-1]) truncated
    to the causal part (w[c, W-1] multiplies the current input)."""
    r = _rng(seed)
    N, Cch, W = 17, 5, 4
    x = r.standard_normal((N, Cch))
    w = r.standard_normal((Cch, W))
    cache = np.zeros((1, W - 1, Cch))
    y, cache_out = causal_conv1d(x, w, np.array([0, N]), cache, np.array([0]))
    err = 0.0
    for c in range(Cch):
        ref = np.convolve(x[:, c], w[c, ::-1])[:N]
        err = max(err, np.abs(y[:, c] - ref).max())
    return max(err, np.abs(cache_out[0] - x[N - (W - 1):]).max())


# ---------------------------------------------------------------- normalised linear attention
def _phi(x):
    """elu(x) + 1 written out for the pins: x + 1 above zero, e^x below."""
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def lin_parallel_form(lin_attn_sequence, seed=12):
    """o_i = sum_{j<=i} (phi(q_i).phi(k_j)) v_j / (sum_{j<=i} phi(q_i).phi(k_j) + eps)
    as a double sum, plus S = phi(K)^T V and z = sum_j phi(k_j)."""
    r = _rng(seed)
    T, H, dk, dv = 18, 2, 5, 4
    q, k, v = r.standard_normal((T, H, dk)), r.standard_normal((T, H, dk)), r.standard_normal((T, H, dv))
    o, S, z = lin_attn_sequence(q, k, v)
    pq, pk = _phi(q), _phi(k)
    worst = 0.0
    for h in range(H):
        for i in range(T):
            w = np.array([pq[i, h] @ pk[j, h] for j in range(i + 1)])
            ref = (w[:, None] * v[:i + 1, h]).sum(0) / (w.sum() + 1e-6)
            worst = max(worst, np.abs(o[i, h] - ref).max())
        worst = max(worst, np.abs(S[h] - pk[:, h].T @ v[:, h]).max(),
                    np.abs(z[h] - pk[:, h].sum(0)).max())
    return worst


def lin_from_state(lin_attn_sequence, seed=13):
    """Starting from (S0, z0): o_i = phi(q_i)(S0 + sum phi(k)^T v) / (phi(q_i).(z0 + sum phi(k)) + eps)."""
    r = _rng(seed)
    T, H, dk, dv = 9, 2, 4, 3
    q, k, v = r.standard_normal((T, H, dk)), r.standard_normal((T, H, dk)), r.standard_normal((T, H, dv))
    S0 = r.standard_normal((H, dk, dv))
    z0 = r.uniform(1.0, 3.0, (H, dk))
    o, _, _ = lin_attn_sequence(q, k, v, S0, z0)
    pq, pk = _phi(q), _phi(k)
    worst = 0.0
    for h in range(H):
        for i in range(T):
            S = S0[h] + pk[:i + 1, h].T @ v[:i + 1, h]
            z = z0[h] + pk[:i + 1, h].sum(0)
            worst = max(worst, np.abs(o[i, h] - pq[i, h] @ S / (pq[i, h] @ z + 1e-6)).max())
    return worst


# ---------------------------------------------------------------- kept states
def _multi(seed, R=2, J=4, H=2, dk=4, dv=3, n_slots=14):
    r = _rng(seed)
    q, k, v = r.standard_normal((R, J, H, dk)), r.standard_normal((R, J, H, dk)), r.standard_normal((R, J, H, dv))
    a = 1.0 / (1.0 + np.exp(-(r.standard_normal((R, J, H)) + 2.0)))
    pool = r.standard_normal((n_slots, H, dk, dv))
    perm = r.permutation(n_slots)
    return q, k, v, a, pool, perm[:R], perm[R:R + R * J].reshape(R, J)


def multi_closed_form(gla_decode_multi, seed=14):
    """Kept state j of request r = (prod_{i<=j} a_i) S_0 + sum_{s<=j} (prod_{i=s+1..j} a_i) k_s^T v_s;
    o_j = q_j S_j; the request's own slot unchanged."""
    q, k, v, a, pool, slots, pos = _multi(seed)
    o, out = gla_decode_multi(q, k, v, a, pool, slots, pos)
    worst = float(np.abs(out[slots] - pool[slots]).max())
    for r in range(q.shape[0]):
        for j in range(q.shape[1]):
            for h in range(q.shape[2]):
                S = np.prod(a[r, :j + 1, h]) * pool[slots[r], h]
                for s_ in range(j + 1):
                    S = S + np.prod(a[r, s_ + 1:j + 1, h]) * np.outer(k[r, s_, h], v[r, s_, h])
                worst = max(worst, np.abs(out[pos[r, j], h] - S).max(),
                            np.abs(o[r, j, h] - q[r, j, h] @ S).max())
    return worst


def ckpt_closed_form(gla_varlen_ckpt, seed=15):
    """Checkpoint j of sequence b = the GLA state after (j+1)*interval of its
    tokens, from its closed form; unreached checkpoint slots untouched."""
    r = _rng(seed)
    lengths, H, dk, dv, iv, stride = [13, 8, 3], 2, 3, 3, 4, 3
    N = sum(lengths)
    q, k, v = r.standard_normal((N, H, dk)), r.standard_normal((N, H, dk)), r.standard_normal((N, H, dv))
    a = 1.0 / (1.0 + np.exp(-(r.standard_normal((N, H)) + 2.0)))
    B = len(lengths)
    n_slots = B + B * stride
    pool = r.standard_normal((n_slots, H, dk, dv))
    perm = r.permutation(n_slots)
    slots, ck = perm[:B], perm[B:].reshape(B, stride)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    _, out = gla_varlen_ckpt(q, k, v, a, cu, pool, slots, ck, iv)
    worst = 0.0
    for b in range(B):
        s0 = cu[b]
        for j in range(stride):
            p = (j + 1) * iv
            if p > lengths[b]:
                worst = max(worst, np.abs(out[ck[b, j]] - pool[ck[b, j]]).max())
                continue
            for h in range(H):
                S = np.prod(a[s0:s0 + p, h]) * pool[slots[b], h]
                for t in range(s0, s0 + p):
                    S = S + np.prod(a[t + 1:s0 + p, h]) * np.outer(k[t, h], v[t, h])
                worst = max(worst, np.abs(out[ck[b, j], h] - S).max())
    return worst


# ---------------------------------------------------------------- decode and zero-init branches
def lin_decode_closed_form(lin_attn_decode, seed=16):
    """One token per request r from (S0, z0) = slot r of the pools:
    S' = S0 + phi(k)^T v, z' = z0 + phi(k), o = phi(q) S' / (phi(q) . z' + eps);
    slots not named keep their values."""
    r = _rng(seed)
    R, H, dk, dv, n_slots = 4, 2, 5, 3, 9
    q, k, v = r.standard_normal((R, H, dk)), r.standard_normal((R, H, dk)), r.standard_normal((R, H, dv))
    pool = r.standard_normal((n_slots, H, dk, dv))
    zpool = r.uniform(1.0, 3.0, (n_slots, H, dk))
    slots = r.permutation(n_slots)[:R]
    o, P, Z = lin_attn_decode(q, k, v, pool, zpool, slots)
    fq, fk = _phi(q), _phi(k)
    rest = sorted(set(range(n_slots)) - set(slots.tolist()))
    worst = max(np.abs(P[rest] - pool[rest]).max(), np.abs(Z[rest] - zpool[rest]).max())
    for i in range(R):
        for h in range(H):
            S = pool[slots[i], h] + np.outer(fk[i, h], v[i, h])
            z = zpool[slots[i], h] + fk[i, h]
            worst = max(worst, np.abs(P[slots[i], h] - S).max(), np.abs(Z[slots[i], h] - z).max(),
                        np.abs(o[i, h] - fq[i, h] @ S / (fq[i, h] @ z + 1e-6)).max())
    return worst


def _zero_init_case(seed, lengths=(5, 0, 7), H=2, dk=4, dv=3, n_slots=6):
    r = _rng(seed)
    N = sum(lengths)
    q, k, v = r.standard_normal((N, H, dk)), r.standard_normal((N, H, dk)), r.standard_normal((N, H, dv))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    a = 1.0 / (1.0 + np.exp(-(r.standard_normal((N, H)) + 2.0)))
    b = 1.0 / (1.0 + np.exp(-r.standard_normal((N, H))))
    pool = r.standard_normal((n_slots, H, dk, dv)) + 1.0      # nonzero everywhere
    slots = r.permutation(n_slots)[:len(lengths)]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    return q, k, v, a, b, pool, slots, cu


def lin_zero_init(lin_attn_varlen, seed=17):
    """zero_init: nonzero pool slots are ignored.  Outputs are the kernelised
    double sum from zero, the slot receives phi(K)^T V and sum phi(k) (zeros
    for an empty sequence), other slots keep their values."""
    q, k, v, _, _, pool, slots, cu = _zero_init_case(seed)
    zpool = np.abs(pool[:, :, :, 0]) + 1.0
    o, P, Z = lin_attn_varlen(q, k, v, cu, pool, zpool, slots, True)
    fq, fk = _phi(q), _phi(k)
    rest = sorted(set(range(pool.shape[0])) - set(slots.tolist()))
    worst = max(np.abs(P[rest] - pool[rest]).max(), np.abs(Z[rest] - zpool[rest]).max())
    for b in range(len(slots)):
        s, e = cu[b], cu[b + 1]
        for h in range(q.shape[1]):
            for i in range(s, e):
                w = np.array([fq[i, h] @ fk[j, h] for j in range(s, i + 1)])
                ref = (w[:, None] * v[s:i + 1, h]).sum(0) / (w.sum() + 1e-6)
                worst = max(worst, np.abs(o[i, h] - ref).max())
            worst = max(worst, np.abs(P[slots[b], h] - fk[s:e, h].T @ v[s:e, h]).max(),
                        np.abs(Z[slots[b], h] - fk[s:e, h].sum(0)).max())
    return worst


def gla_zero_init(gla_varlen, seed=18):
    """zero_init: each sequence starts from S = 0 whatever its slot holds:
    o_t = sum_{s<=t} (prod_{r=s+1..t} alpha_r)(q_t . k_s) v_s with products
    taken directly; the slot receives the final state (zeros if empty)."""
    q, k, v, a, _, pool, slots, cu = _zero_init_case(seed)
    o, P = gla_varlen(q, k, v, a, cu, pool, slots, True)
    worst = 0.0
    for b in range(len(slots)):
        s, e = cu[b], cu[b + 1]
        for h in range(q.shape[1]):
            Sref = np.zeros(pool.shape[2:])
            for t in range(s, e):
                ref = np.zeros(v.shape[2])
                for j in range(s, t + 1):
                    ref = ref + np.prod(a[j + 1:t + 1, h]) * (q[t, h] @ k[j, h]) * v[j, h]
                worst = max(worst, np.abs(o[t, h] - ref).max())
                Sref = Sref + np.prod(a[t + 1:e, h]) * np.outer(k[t, h], v[t, h])
            worst = max(worst, np.abs(P[slots[b], h] - Sref).max())
    return worst


def gdn_zero_init(gdn_varlen, seed=19):
    """zero_init for Gated DeltaNet: the literal d_k x d_k update
    alpha (I - beta k^T k) S + beta k^T v run from S = 0."""
    q, k, v, a, b_, pool, slots, cu = _zero_init_case(seed)
    o, P = gdn_varlen(q, k, v, a, b_, cu, pool, slots, True)
    dk = q.shape[2]
    worst = 0.0
    for b in range(len(slots)):
        s, e = cu[b], cu[b + 1]
        for h in range(q.shape[1]):
            St = np.zeros(pool.shape[2:])
            for t in range(s, e):
                kk = k[t, h][:, None]
                St = a[t, h] * (np.eye(dk) - b_[t, h] * (kk @ kk.T)) @ St + b_[t, h] * (kk @ v[t, h][None, :])
                worst = max(worst, np.abs(o[t, h] - q[t, h] @ St).max())
            worst = max(worst, np.abs(P[slots[b], h] - St).max())
    return worst


def conv_zero_init(causal_conv1d, seed=20):
    """zero_init: a nonzero cache is read as zeros, so each sequence's output
    is numpy.convolve of its own inputs (w[c, W-1] on the current input); the
    cache receives the last W-1 rows of [zeros(W-1); x] (a 2-token sequence
    leaves one zero row in front of its inputs)."""
    r = _rng(seed)
    lengths, Cch, W = [9, 2], 5, 4
    N = sum(lengths)
    x = r.standard_normal((N, Cch))
    w = r.standard_normal((Cch, W))
    cache = r.standard_normal((4, W - 1, Cch)) + 1.0
    slots = np.array([3, 1])
    cu = np.concatenate([[0], np.cumsum(lengths)])
    y, c = causal_conv1d(x, w, cu, cache, slots, True)
    err = max(np.abs(c[[0, 2]] - cache[[0, 2]]).max(), 0.0)
    for b in range(2):
        s, e = cu[b], cu[b + 1]
        for ch in range(Cch):
            ref = np.convolve(x[s:e, ch], w[ch, ::-1])[:e - s]
            err = max(err, np.abs(y[s:e, ch] - ref).max())
        tail = np.concatenate([np.zeros((W - 1, Cch)), x[s:e]])[-(W - 1):]
        err = max(err, np.abs(c[slots[b]] - tail).max())
    return err
