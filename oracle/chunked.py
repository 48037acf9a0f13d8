"""Chunked evaluation of the recurrences in fp64 (oracle; test
infrastructure only).  Used to pin the recurrence, never as the definition.

GLA: "Inference for linear attention and hybrid architectures", section
"Two ways to write the same computation", the chunked (prefill) form.  Its
content, restated from the recurrence S_t = alpha_t S_{t-1} + k_t^T v_t:
for a chunk of tokens s..e-1 entered with state S, token i of the chunk
(i = 0 .. n-1) sees
  * each earlier token j <= i of the same chunk through the gates that act
    after it, lambda(i, j) = alpha_{j+1} ... alpha_i (an empty product is 1),
    and
  * the entering state through all the chunk's gates up to i,
    lambda_in(i) = alpha_0 ... alpha_i,
so o_i = sum_{j<=i} lambda(i, j) (q_i . k_j) v_j + lambda_in(i) q_i S, and the
state that leaves the chunk is lambda_in(n-1) S + sum_j lambda(n-1, j) k_j^T v_j.
Here the decays are formed as direct products of the gates (the page forms
them from a running sum of log-gates); the sums are written per position.

Gated DeltaNet: the page gives no chunked form (it only says the in-chunk
error-correcting updates must first be put in matrix form).  Derived form,
pinned only through its equality with the recurrence: with
u_t = beta_t (v_t - alpha_t k_t S_{t-1}) the update is a GLA step with value
u_t.  Inside a chunk entered with state S and cumulative decay G_t =
exp(g_t):
    (I + A) U = diag(beta) V - diag(beta G) K S,
    A_tj = beta_t (G_t / G_j) (k_t . k_j) for j < t, 0 otherwise,
and then the GLA chunk formulas with U in place of V.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def _chunks(T, C):
    start = 0
    while start < T:
        yield start, min(start + C, T)
        start += C


def gla_chunked(q, k, v, alpha, C, S0=None):
    """Chunked GLA for one head: q, k [T, dk]; v [T, dv]; alpha [T];
    returns (o [T, dv], S [dk, dv]).  Works in the dtype of the inputs
    (fp64 for the oracle; fp32 to reproduce the page's own check)."""
    dt = np.result_type(q, k, v, alpha)
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv), dt) if S0 is None else np.array(S0, dt)
    o = np.zeros((T, dv), dt)
    for s, e in _chunks(T, C):
        n = e - s
        gates = alpha[s:e]
        # lam[i, j]: gates after position j up to and including i (j <= i)
        lam = np.zeros((n, n), dt)
        for i in range(n):
            for j in range(i + 1):
                lam[i, j] = np.prod(gates[j + 1:i + 1], dtype=dt)
        lam_in = np.array([np.prod(gates[:i + 1], dtype=dt) for i in range(n)], dt)
        for i in range(n):
            acc = lam_in[i] * (q[s + i] @ S)
            for j in range(i + 1):
                acc = acc + lam[i, j] * (q[s + i] @ k[s + j]) * v[s + j]
            o[s + i] = acc
        # the state leaving the chunk, one token's write at a time
        S_out = lam_in[n - 1] * S
        for j in range(n):
            S_out = S_out + lam[n - 1, j] * np.outer(k[s + j], v[s + j])
        S = S_out
    return o, S


def gdn_chunked(q, k, v, alpha, beta, C, S0=None):
    """Chunked Gated DeltaNet for one head (derived form above):
    returns (o [T, dv], S [dk, dv]) in fp64."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    alpha, beta = np.asarray(alpha, np.float64), np.asarray(beta, np.float64)
    S = np.zeros((q.shape[1], v.shape[1])) if S0 is None else np.array(S0, np.float64)
    o = np.zeros((q.shape[0], v.shape[1]))
    for s, e in _chunks(q.shape[0], C):
        Q, K, V, b = q[s:e], k[s:e], v[s:e], beta[s:e]
        n = e - s
        g = np.cumsum(np.log(alpha[s:e]))
        diff = g[:, None] - g[None, :]
        lower = np.tril(np.ones((n, n), dtype=bool))
        D = np.where(lower, np.exp(np.where(lower, diff, 0)), 0)
        strict = np.tril(np.ones((n, n), dtype=bool), -1)
        A = np.where(strict, b[:, None] * D * (K @ K.T), 0)
        rhs = b[:, None] * V - (b * np.exp(g))[:, None] * (K @ S)
        U = solve_triangular(np.eye(n) + A, rhs, lower=True, unit_diagonal=True)
        o[s:e] = ((Q @ K.T) * D) @ U + np.exp(g)[:, None] * (Q @ S)
        S = np.exp(g[-1]) * S + (np.exp(g[-1] - g)[:, None] * K).T @ U
    return o, S
