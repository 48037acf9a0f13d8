"""Chunked evaluation of the recurrences in fp64 (oracle; test
infrastructure only).  Used to pin the recurrence, never as the definition.

GLA: "Inference for linear attention and hybrid architectures", section
"Two ways to write the same computation", the chunked (prefill) algorithm:
per chunk of C tokens, g is the running sum of log alpha restarted at the
chunk start; position i sees position j <= i with decay exp(g_i - g_j); the
chunk output is the decay-masked C x C "attention" applied to V plus
exp(g_i) q_i S for the state that entered the chunk; the state leaving the
chunk is exp(g_last) S + sum_j exp(g_last - g_j) k_j^T v_j.

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
    S = np.zeros((q.shape[1], v.shape[1]), dt) if S0 is None else np.array(S0, dt)
    o = np.zeros((q.shape[0], v.shape[1]), dt)
    for s, e in _chunks(q.shape[0], C):
        Q, K, V = q[s:e], k[s:e], v[s:e]
        g = np.cumsum(np.log(alpha[s:e]))
        diff = g[:, None] - g[None, :]
        causal = np.tril(np.ones((e - s, e - s), dtype=bool))
        D = np.where(causal, np.exp(np.where(causal, diff, 0)), 0).astype(dt)
        o[s:e] = ((Q @ K.T) * D) @ V + np.exp(g)[:, None] * (Q @ S)
        S = np.exp(g[-1]) * S + (np.exp(g[-1] - g)[:, None] * K).T @ V
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
