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
