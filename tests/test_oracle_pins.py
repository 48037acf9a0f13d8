"""The fp64 oracle against facts that do not come from itself.

Citations are to "Inference for linear attention and hybrid architectures"
(section names given per test).
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ GLA
def test_gla_bruteforce():
    """Softmax-free attention written as a double sum ("Two ways to write
    the same computation", first formula, with the GLA gate)."""
    assert pins.gla_bruteforce(oracle.gla_sequence) <= pins.TOL


def test_gla_alpha_one_is_linear_attention():
    assert pins.gla_linear_attention(oracle.gla_sequence) <= pins.TOL


def test_gla_scalar_state_is_iir_filter():
    assert pins.gla_lfilter(oracle.gla_sequence) <= pins.TOL


def test_page_toy_example_recurrent_equals_chunked():
    """The page's worked example: recurrent and chunked agree within
    allclose(atol=1e-5) for outputs and final state (printed True/True).
    The fp64 oracle is compared with the page's chunked algorithm run in
    fp32 (as the page runs it) and in fp64."""
    g = _load("page_toy_example.json")["printed"]
    q, k, v, a = synth.page_toy_example()
    o, S = oracle.gla_sequence(q[:, None], k[:, None], v[:, None], a[:, None])
    o32, S32 = oracle.gla_chunked(q, k, v, a, 16)
    assert o32.dtype == np.float32
    atol = g["allclose_atol"]
    close_o = np.allclose(o[:, 0], o32, atol=atol)
    close_S = np.allclose(S[0], S32, atol=atol)
    assert close_o == g["recurrent_vs_chunked_outputs_allclose"]
    assert close_S == g["recurrent_vs_chunked_final_state_allclose"]
    o64, S64 = oracle.gla_chunked(q.astype(np.float64), k.astype(np.float64),
                                  v.astype(np.float64), a.astype(np.float64), 16)
    assert np.abs(o64 - o[:, 0]).max() <= 1e-12
    assert np.abs(S64 - S[0]).max() <= 1e-12
    # state is d_k x d_v numbers whatever T is; KV of the same length is T x (d_k + d_v)
    assert list(S[0].shape) == g["state_numbers_per_head"]
    assert [q.shape[0], q.shape[1] + v.shape[1]] == g["kv_cache_numbers_same_length"]


@pytest.mark.parametrize("C", [16, 64, 37, 1, 200])
def test_gla_chunked_equals_recurrence(C):
    q, k, v, a, _, S0 = pins._inputs(20, T=150, H=1, dk=16, dv=12)
    o, S = oracle.gla_sequence(q, k, v, a, S0)
    oc, Sc = oracle.gla_chunked(q[:, 0], k[:, 0], v[:, 0], a[:, 0], C, S0[0])
    assert np.abs(o[:, 0] - oc).max() <= 1e-12 and np.abs(S[0] - Sc).max() <= 1e-12


# ------------------------------------------------------------------ GDN
def test_gdn_matrix_form():
    """DeltaNet's update as written on the page, with an explicit d_k x d_k
    matrix, and the decay gate multiplied in."""
    assert pins.gdn_matrix_form(oracle.gdn_sequence) <= pins.TOL


def test_gdn_unrolled_closed_form():
    assert pins.gdn_unrolled(oracle.gdn_sequence) <= pins.TOL


def test_gdn_beta_zero():
    assert pins.gdn_beta_zero(oracle.gdn_sequence) <= pins.TOL


def test_gdn_orthogonal_keys_is_gla():
    assert pins.gdn_orthogonal_keys(oracle.gdn_sequence, oracle.gla_sequence) <= pins.TOL


def test_gdn_orthonormal_alpha_beta_one_is_linear_attention():
    assert pins.gdn_linear_attention(oracle.gdn_sequence) <= pins.TOL


def test_gdn_retrieval_identity():
    assert pins.gdn_retrieval(oracle.gdn_sequence) <= pins.TOL


def test_gdn_exact_overwrite():
    assert pins.gdn_overwrite(oracle.gdn_sequence) <= 1e-12


@pytest.mark.parametrize("C", [16, 64, 37])
def test_gdn_chunked_equals_recurrence(C):
    q, k, v, a, b, S0 = pins._inputs(21, T=150, H=1, dk=16, dv=12, unit_k=True)
    o, S = oracle.gdn_sequence(q, k, v, a, b, S0)
    oc, Sc = oracle.gdn_chunked(q[:, 0], k[:, 0], v[:, 0], a[:, 0], b[:, 0], C, S0[0])
    assert np.abs(o[:, 0] - oc).max() <= 1e-12 and np.abs(S[0] - Sc).max() <= 1e-12


# ------------------------------------------------------------------ state handling
@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_segments_pass_only_the_state(kind):
    """"Chunked prefill comes for free": a prompt cut into segments that
    hand only the state on gives the same result (bitwise in the oracle)."""
    q, k, v, a, b, S0 = pins._inputs(22, T=90, unit_k=True)
    f = oracle.gla_sequence if kind == "gla" else oracle.gdn_sequence
    g = (a,) if kind == "gla" else (a, b)
    o, S = f(q, k, v, *g, S0)
    outs, St = [], S0
    for s, e in [(0, 20), (20, 45), (45, 90)]:
        ob, St = f(q[s:e], k[s:e], v[s:e], *[x[s:e] for x in g], St)
        outs.append(ob)
    assert np.array_equal(np.concatenate(outs), o) and np.array_equal(St, S)


def test_state_size_independent_of_length():
    """Section "The real model's ledger": a 16-head 128x128 fp32 state is
    1 MiB per layer at 100, 1000 and 3000 tokens; 18 layers hold 18 MiB."""
    g = _load("state_ledger.json")["printed"]
    shape = g["linear_layer_state_shape"]
    for T in g["prefill_lengths_tokens"][:2]:
        r = np.random.default_rng(T)
        H, d = 2, 8
        _, S = oracle.gla_sequence(r.standard_normal((T, H, d)), r.standard_normal((T, H, d)),
                                   r.standard_normal((T, H, d)), np.full((T, H), 0.9))
        assert S.shape == (H, d, d)
    per_layer = int(np.prod(shape)) * g["state_dtype_bytes"]
    assert per_layer == g["state_per_layer_MiB"] * 2**20
    assert per_layer * g["linear_layers"] == g["state_total_MiB"] * 2**20
    assert 128 * 128 * 4 == g["head_state_KB"] * 1024
    # the conv cache: 18 layers x channels x 4 columns x bf16 = 864 KiB -> 6144 channels
    ch = g["conv_cache_total_KiB"] * 1024 // (g["linear_layers"] * g["conv_cache_columns_kept"]
                                              * g["conv_cache_dtype_bytes"])
    assert ch == 6144 and g["conv_cache_columns_engine_needs"] == g["conv_cache_columns_kept"] - 1


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_varlen_slots_and_batch_invariance(kind):
    """Batched kernels read and write states by slot index (section
    "Speculative decoding and PD disaggregation"): untouched slots keep their
    bytes, empty sequences keep (or, with zero-init, zero) their state, and a
    request's result does not depend on what else is in the batch."""
    lens = [7, 0, 19, 1, 12]
    w = synth.random_varlen(30, lens, 2, 6, 5, dtype="f32", gdn=(kind == "gdn"), n_slots=9)
    f = oracle.gla_varlen if kind == "gla" else oracle.gdn_varlen
    g = (w.alpha,) if kind == "gla" else (w.alpha, w.beta)
    o, P = f(w.q, w.k, w.v, *g, w.cu_seqlens, w.pool, w.slot_idx, False)
    untouched = sorted(set(range(9)) - set(w.slot_idx.tolist()))
    assert np.array_equal(P[untouched], w.pool[untouched].astype(np.float64))
    assert np.array_equal(P[w.slot_idx[1]], w.pool[w.slot_idx[1]].astype(np.float64))
    seqf = oracle.gla_sequence if kind == "gla" else oracle.gdn_sequence
    for b in range(len(lens)):
        s, e = w.cu_seqlens[b], w.cu_seqlens[b + 1]
        if e == s:
            continue
        ob, Sb = seqf(w.q[s:e], w.k[s:e], w.v[s:e], *[x[s:e] for x in g], w.pool[w.slot_idx[b]])
        assert np.array_equal(ob, o[s:e]) and np.array_equal(Sb, P[w.slot_idx[b]])
    _, Pz = f(w.q, w.k, w.v, *g, w.cu_seqlens, w.pool, w.slot_idx, True)
    assert not Pz[w.slot_idx[1]].any()


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_decode_is_one_step(kind):
    w = synth.random_varlen(31, [1, 1, 1], 2, 6, 5, dtype="f32", gdn=(kind == "gdn"), n_slots=6)
    if kind == "gla":
        o, P = oracle.gla_decode(w.q, w.k, w.v, w.alpha, w.pool, w.slot_idx)
    else:
        o, P = oracle.gdn_decode(w.q, w.k, w.v, w.alpha, w.beta, w.pool, w.slot_idx)
    seqf = oracle.gla_sequence if kind == "gla" else oracle.gdn_sequence
    for r in range(3):
        g = (w.alpha[r:r + 1],) if kind == "gla" else (w.alpha[r:r + 1], w.beta[r:r + 1])
        ob, Sb = seqf(w.q[r:r + 1], w.k[r:r + 1], w.v[r:r + 1], *g, w.pool[w.slot_idx[r]])
        assert np.array_equal(ob[0], o[r]) and np.array_equal(Sb, P[w.slot_idx[r]])


def test_checkpoint_copy_and_rollback():
    """Section "Prefix caching has to be redone": a state saved at the end
    of a shared prefix and copied lets each continuation match a run from
    scratch; section "Speculative decoding and PD disaggregation": rollback
    restores a saved state and replays."""
    q, k, v, a, b, S0 = pins._inputs(23, T=60, unit_k=True)
    f = oracle.gdn_sequence
    _, ck = f(q[:39], k[:39], v[:39], a[:39], b[:39], S0)
    saved = ck.copy()
    o_full, S_full = f(q, k, v, a, b, S0)
    o_tail, S_tail = f(q[39:], k[39:], v[39:], a[39:], b[39:], ck)
    assert np.array_equal(ck, saved)       # continuing works on its own copy
    assert np.array_equal(o_tail, o_full[39:]) and np.array_equal(S_tail, S_full)
    # 4 draft tokens accepted 2: restore the checkpoint and replay the accepted ones
    _, S_draft = f(q[39:43], k[39:43], v[39:43], a[39:43], b[39:43], saved)
    _, S_acc = f(q[39:41], k[39:41], v[39:41], a[39:41], b[39:41], saved)
    _, S_ref = f(q[:41], k[:41], v[:41], a[:41], b[:41], S0)
    assert np.array_equal(S_acc, S_ref) and not np.array_equal(S_draft, S_ref)


# ------------------------------------------------------------------ conv
def test_conv_is_numpy_convolve():
    assert pins.conv_numpy_convolve(oracle.causal_conv1d) <= pins.TOL


def test_conv_segments_and_token_by_token():
    """The conv cache carries the last width-1 inputs across calls, so one
    pass, segments, and one token at a time all agree (bitwise)."""
    r = np.random.default_rng(12)
    N, Cch, W = 23, 6, 4
    x = r.standard_normal((N, Cch))
    w = r.standard_normal((Cch, W))
    cache = r.standard_normal((3, W - 1, Cch))
    slot = np.array([2])
    y, c1 = oracle.causal_conv1d(x, w, np.array([0, N]), cache, slot)
    ys, c = [], cache
    for s, e in [(0, 5), (5, 6), (6, 23)]:
        yb, c = oracle.causal_conv1d(x[s:e], w, np.array([0, e - s]), c, slot)
        ys.append(yb)
    assert np.array_equal(np.concatenate(ys), y) and np.array_equal(c, c1)
    c = cache
    for t in range(N):
        yt, c = oracle.causal_conv1d(x[t:t + 1], w, np.array([0, 1]), c, slot)
        assert np.array_equal(yt[0], y[t])
    assert np.array_equal(c, c1)
    assert np.array_equal(c1[[0, 1]], cache[[0, 1]])


# ------------------------------------------------------------------ multi-token decode, state copy
def _multi_inputs(seed, R=3, J=5, H=2, dk=6, dv=5, n_slots=24):
    r = np.random.default_rng(seed)
    q = r.standard_normal((R, J, H, dk))
    k = r.standard_normal((R, J, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((R, J, H, dv))
    a = 1.0 / (1.0 + np.exp(-(r.standard_normal((R, J, H)) + 2.0)))
    b = 1.0 / (1.0 + np.exp(-r.standard_normal((R, J, H))))
    pool = r.standard_normal((n_slots, H, dk, dv)) * 0.3
    perm = r.permutation(n_slots)
    slots = perm[:R].astype(np.int32)
    pos = perm[R:R + R * J].reshape(R, J).astype(np.int32)
    return q, k, v, a, b, pool, slots, pos


def test_gla_decode_multi_kept_states_closed_form():
    """Speculative decoding ("Speculative decoding and PD disaggregation"):
    the state kept after draft position j is
        S_j = (prod_{i<=j} a_i) S_0 + sum_{s<=j} (prod_{i=s+1..j} a_i) k_s^T v_s,
    with the products taken directly, and o_j = q_j S_j."""
    q, k, v, a, _, pool, slots, pos = _multi_inputs(20)
    o, out = oracle.gla_decode_multi(q, k, v, a, pool, slots, pos)
    R, J, H = a.shape
    worst = 0.0
    for r in range(R):
        for j in range(J):
            for h in range(H):
                S = np.prod(a[r, :j + 1, h]) * pool[slots[r], h]
                for s in range(j + 1):
                    S = S + np.prod(a[r, s + 1:j + 1, h]) * np.outer(k[r, s, h], v[r, s, h])
                worst = max(worst, np.abs(out[pos[r, j], h] - S).max(),
                            np.abs(o[r, j, h] - q[r, j, h] @ S).max())
    assert worst <= pins.TOL
    # the requests' own slots are only read
    assert np.array_equal(out[slots], pool[slots])


def test_gdn_decode_multi_kept_states_matrix_form():
    """Gated DeltaNet draft positions: each kept state is the literal
    a (I - b k^T k) S + b k^T v with d_k x d_k matrices ("Two ways to write
    the same computation", DeltaNet update with the gate)."""
    q, k, v, a, b, pool, slots, pos = _multi_inputs(21)
    o, out = oracle.gdn_decode_multi(q, k, v, a, b, pool, slots, pos)
    R, J, H, dk = q.shape
    worst = 0.0
    for r in range(R):
        for h in range(H):
            S = pool[slots[r], h].copy()
            for j in range(J):
                kk = k[r, j, h][:, None]
                S = a[r, j, h] * (np.eye(dk) - b[r, j, h] * kk @ kk.T) @ S \
                    + b[r, j, h] * kk @ v[r, j, h][None, :]
                worst = max(worst, np.abs(out[pos[r, j], h] - S).max(),
                            np.abs(o[r, j, h] - q[r, j, h] @ S).max())
    assert worst <= pins.TOL


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_decode_multi_rollback_and_prefix_prefill(kind):
    """Each kept state equals a prefill of the same prefix passing only the
    state ("Chunked prefill comes for free"), and rolling back to an
    accepted position then replaying the rejected tokens reproduces the
    later kept states bitwise."""
    q, k, v, a, b, pool, slots, pos = _multi_inputs(22)
    R, J = a.shape[:2]
    if kind == "gla":
        o, out = oracle.gla_decode_multi(q, k, v, a, pool, slots, pos)
    else:
        o, out = oracle.gdn_decode_multi(q, k, v, a, b, pool, slots, pos)
    for r in range(R):
        for j in range(J):
            if kind == "gla":
                op, Sp = oracle.gla_sequence(q[r, :j + 1], k[r, :j + 1], v[r, :j + 1],
                                             a[r, :j + 1], S0=pool[slots[r]])
            else:
                op, Sp = oracle.gdn_sequence(q[r, :j + 1], k[r, :j + 1], v[r, :j + 1],
                                             a[r, :j + 1], b[r, :j + 1], S0=pool[slots[r]])
            assert np.array_equal(out[pos[r, j]], Sp)
            assert np.array_equal(o[r, :j + 1], op)
        # accept 2 tokens, then replay the rest from the kept state
        acc = 2
        rest = slice(acc, J)
        if kind == "gla":
            _, Sr = oracle.gla_sequence(q[r, rest], k[r, rest], v[r, rest], a[r, rest],
                                        S0=out[pos[r, acc - 1]])
        else:
            _, Sr = oracle.gdn_sequence(q[r, rest], k[r, rest], v[r, rest], a[r, rest],
                                        b[r, rest], S0=out[pos[r, acc - 1]])
        assert np.array_equal(Sr, out[pos[r, J - 1]])
    # untouched slots: neither a request's slot nor a kept position
    named = set(slots.tolist()) | set(pos.ravel().tolist())
    for s in range(pool.shape[0]):
        if s not in named:
            assert np.array_equal(out[s], pool[s])


def test_decode_multi_skips_unkept_positions_and_own_slot():
    q, k, v, a, _, pool, slots, pos = _multi_inputs(23)
    pos = pos.copy()
    pos[:, :-1] = -1                       # keep only the last position
    pos[0, -1] = slots[0]                  # request 0 commits in place
    o, out = oracle.gla_decode_multi(q, k, v, a, pool, slots, pos)
    _, S_last = oracle.gla_sequence(q[0], k[0], v[0], a[0], S0=pool[slots[0]])
    assert np.array_equal(out[slots[0]], S_last)
    assert np.array_equal(out[slots[1:]], pool[slots[1:]])


def test_state_copy_reads_before_writes():
    """Prefix reuse ("Prefix caching has to be redone"): a continuation gets
    its own whole copy of the saved state; slots not named are unchanged."""
    r = np.random.default_rng(24)
    pool = r.standard_normal((8, 2, 4, 3))
    out = oracle.state_copy(pool, np.array([1, 5, 2]), np.array([4, 1, 7]))
    assert np.array_equal(out[4], pool[1]) and np.array_equal(out[1], pool[5])
    assert np.array_equal(out[7], pool[2])
    for s in (0, 2, 3, 5, 6):
        assert np.array_equal(out[s], pool[s])
    # out-of-range pairs are skipped
    assert np.array_equal(oracle.state_copy(pool, np.array([-1, 9]), np.array([0, 0])), pool)


# ------------------------------------------------------------------ prefill checkpoints
def _ckpt_inputs(seed, lengths=(37, 0, 64, 50), H=2, dk=5, dv=4, interval=16, stride=3):
    r = np.random.default_rng(seed)
    N = sum(lengths)
    q = r.standard_normal((N, H, dk))
    k = r.standard_normal((N, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((N, H, dv))
    a = 1.0 / (1.0 + np.exp(-(r.standard_normal((N, H)) + 2.0)))
    b = 1.0 / (1.0 + np.exp(-r.standard_normal((N, H))))
    B = len(lengths)
    n_slots = B + B * stride + 2
    pool = r.standard_normal((n_slots, H, dk, dv)) * 0.3
    perm = r.permutation(n_slots)
    slots = perm[:B].astype(np.int32)
    ck = perm[B:B + B * stride].reshape(B, stride).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return q, k, v, a, b, pool, slots, ck, cu, interval


def test_gla_ckpt_states_closed_form():
    """Saved states ("Prefix caching has to be redone": a state can be
    reused only where it was saved) are the GLA state after that many
    tokens, here from its closed form with direct products; outputs and
    final states equal the plain varlen run."""
    q, k, v, a, _, pool, slots, ck, cu, iv = _ckpt_inputs(25)
    o, out = oracle.gla_varlen_ckpt(q, k, v, a, cu, pool, slots, ck, iv)
    o2, out2 = oracle.gla_varlen(q, k, v, a, cu, pool, slots)
    assert np.array_equal(o, o2) and np.array_equal(out[slots], out2[slots])
    worst = 0.0
    n_saved = 0
    for bi in range(len(slots)):
        s0, e0 = int(cu[bi]), int(cu[bi + 1])
        for j in range(ck.shape[1]):
            p = (j + 1) * iv
            if p > e0 - s0:
                assert np.array_equal(out[ck[bi, j]], pool[ck[bi, j]])   # not reached: untouched
                continue
            n_saved += 1
            for h in range(q.shape[1]):
                S = np.prod(a[s0:s0 + p, h]) * pool[slots[bi], h]
                for t in range(s0, s0 + p):
                    S = S + np.prod(a[t + 1:s0 + p, h]) * np.outer(k[t, h], v[t, h])
                worst = max(worst, np.abs(out[ck[bi, j], h] - S).max())
    assert n_saved == 2 + 0 + 3 + 3 and worst <= pins.TOL


def test_gdn_ckpt_states_matrix_form_and_reuse():
    """Gated DeltaNet checkpoints against the literal d_k x d_k update, and
    the page's prefix-cache demonstration: continuing from a copy of a
    checkpoint gives the same as the uncut prompt (there it printed True for
    both requests)."""
    q, k, v, a, b, pool, slots, ck, cu, iv = _ckpt_inputs(26)
    o, out = oracle.gdn_varlen_ckpt(q, k, v, a, b, cu, pool, slots, ck, iv)
    dk = q.shape[2]
    worst = 0.0
    for bi in range(len(slots)):
        s0, e0 = int(cu[bi]), int(cu[bi + 1])
        for h in range(q.shape[1]):
            S = pool[slots[bi], h].copy()
            for t in range(s0, e0):
                kk = k[t, h][:, None]
                S = a[t, h] * (np.eye(dk) - b[t, h] * kk @ kk.T) @ S + b[t, h] * kk @ v[t, h][None, :]
                p = t + 1 - s0
                if p % iv == 0 and p // iv - 1 < ck.shape[1]:
                    worst = max(worst, np.abs(out[ck[bi, p // iv - 1], h] - S).max())
        # reuse: continue from the saved state after 16 tokens
        if e0 - s0 >= iv:
            cut = s0 + iv
            o_rest, S_rest = oracle.gdn_sequence(q[cut:e0], k[cut:e0], v[cut:e0], a[cut:e0],
                                                 b[cut:e0], S0=out[ck[bi, 0]].copy())
            assert np.array_equal(o_rest, o[cut:e0])
            assert np.array_equal(S_rest, out[slots[bi]])
    assert worst <= pins.TOL


# ------------------------------------------------------------------ normalised linear attention
def _lin_inputs(seed, T=20, H=2, dk=5, dv=4):
    r = np.random.default_rng(seed)
    return (r.standard_normal((T, H, dk)), r.standard_normal((T, H, dk)),
            r.standard_normal((T, H, dv)))


def test_phi_is_elu_plus_one():
    """phi(x) = elu(x) + 1 (page "Long context, fast inference, smart
    decoding, and life beyond attention", listing "Linear attention as a
    running state"): torch's elu on the CPU, plus one."""
    import torch
    x = np.linspace(-30, 30, 2001)
    ref = torch.nn.functional.elu(torch.from_numpy(x)).numpy() + 1.0
    assert np.abs(oracle.phi(x) - ref).max() <= 1e-15
    assert (oracle.phi(x) > 0).all()


def test_lin_attn_equals_kernelised_parallel_form():
    """The recurrence equals the kernelised attention written as a double
    sum over j <= i (same page, section "Linear attention: removing softmax
    entirely"), which the listing states it is equivalent to."""
    q, k, v = _lin_inputs(30)
    o, S, z = oracle.lin_attn_sequence(q, k, v)
    T, H, _ = q.shape
    pq, pk = oracle.phi(q), oracle.phi(k)
    worst = 0.0
    for h in range(H):
        for i in range(T):
            w = np.array([pq[i, h] @ pk[j, h] for j in range(i + 1)])
            ref = (w[:, None] * v[:i + 1, h]).sum(0) / (w.sum() + 1e-6)
            worst = max(worst, np.abs(o[i, h] - ref).max())
        worst = max(worst, np.abs(S[h] - pk[:, h].T @ v[:, h]).max(),
                    np.abs(z[h] - pk[:, h].sum(0)).max())
    assert worst <= pins.TOL


def test_lin_attn_convex_combination_and_constants():
    """Positive weights: each output lies between the smallest and largest
    value seen so far (up to eps), and constant values are returned as they
    are (scaled by den / (den + eps))."""
    q, k, v = _lin_inputs(31, T=40)
    o, _, _ = oracle.lin_attn_sequence(q, k, v, eps=0.0)
    lo = np.minimum.accumulate(v, axis=0)
    hi = np.maximum.accumulate(v, axis=0)
    assert (o >= lo - 1e-9).all() and (o <= hi + 1e-9).all()
    vc = np.full_like(v, 2.5)
    oc, _, _ = oracle.lin_attn_sequence(q, k, vc, eps=0.0)
    assert np.abs(oc - 2.5).max() <= 1e-12


def test_lin_attn_segments_through_pool():
    """Splitting a sequence and passing (S, z) through the pool gives the
    same result (state hand-off, "Chunked prefill comes for free")."""
    q, k, v = _lin_inputs(32, T=30)
    o, S, z = oracle.lin_attn_sequence(q, k, v)
    H, dk, dv = 2, 5, 4
    pool, zpool = np.zeros((3, H, dk, dv)), np.zeros((3, H, dk))
    o1, pool, zpool = oracle.lin_attn_varlen(q[:11], k[:11], v[:11], [0, 11], pool, zpool, [2])
    o2, pool, zpool = oracle.lin_attn_varlen(q[11:], k[11:], v[11:], [0, 19], pool, zpool, [2])
    assert np.array_equal(np.concatenate([o1, o2]), o)
    assert np.array_equal(pool[2], S) and np.array_equal(zpool[2], z)


# ------------------------------------------------------------------ decode and zero-init branches
def test_lin_attn_decode_closed_form():
    """Normalised linear attention decode: one running-state step per
    request on its slot of both pools (page "Long context, fast inference,
    smart decoding, and life beyond attention", section "Linear attention:
    removing softmax entirely")."""
    assert pins.lin_decode_closed_form(oracle.lin_attn_decode) <= pins.TOL


def test_zero_init_ignores_the_pool():
    """A fresh request starts from S = 0 whatever its slot holds; the final
    state still goes to the slot (section "Chunked prefill comes for free":
    the hand-off is the state alone)."""
    assert pins.gla_zero_init(oracle.gla_varlen) <= pins.TOL
    assert pins.gdn_zero_init(oracle.gdn_varlen) <= pins.TOL
    assert pins.lin_zero_init(oracle.lin_attn_varlen) <= pins.TOL


def test_conv_zero_init_ignores_the_cache():
    assert pins.conv_zero_init(oracle.causal_conv1d) <= pins.TOL
