"""Planted mistakes: copies of the oracle with one plausible error each
(a dropped term, a wrong sign or index, a transposed operand, the output read
at the wrong time).  Every mutant must be caught by at least one pin."""
import numpy as np
import pytest

import oracle
from tests import pins


def _gla_mutant(kind):
    def f(q, k, v, alpha, S0=None):
        q, k, v, alpha = (np.asarray(x, np.float64) for x in (q, k, v, alpha))
        T, H, dk = q.shape
        dv = v.shape[2]
        S = np.zeros((H, dk, dv)) if S0 is None else np.array(S0, np.float64)
        o = np.zeros((T, H, dv))
        for t in range(T):
            a = alpha[t][:, None, None]
            kv = k[t][:, :, None] * v[t][:, None, :]
            if kind == "read_before_update":
                o[t] = np.einsum("hd,hde->he", q[t], S)
            if kind == "no_decay":
                S = S + kv
            elif kind == "decay_on_write":
                S = a * (S + kv)
            elif kind == "sign":
                S = a * S - kv
            elif kind == "transposed_outer":
                S = a * S + np.swapaxes(kv, 1, 2)
            elif kind == "decay_index":        # uses the previous token's gate
                S = alpha[max(t - 1, 0)][:, None, None] * S + kv
            else:
                S = a * S + kv
            if kind != "read_before_update":
                o[t] = np.einsum("hd,hde->he", q[t], S)
        return o, S
    return f


def _gdn_mutant(kind):
    def f(q, k, v, alpha, beta, S0=None):
        q, k, v, alpha, beta = (np.asarray(x, np.float64) for x in (q, k, v, alpha, beta))
        T, H, dk = q.shape
        dv = v.shape[2]
        S = np.zeros((H, dk, dv)) if S0 is None else np.array(S0, np.float64)
        o = np.zeros((T, H, dv))
        for t in range(T):
            a = alpha[t][:, None, None]
            b = beta[t][:, None, None]
            kk = k[t][:, :, None]
            p = np.einsum("hd,hde->he", k[t], S)
            if kind == "gate_everything":
                S = a * (S - b * kk * p[:, None, :] + b * kk * v[t][:, None, :])
            elif kind == "erase_without_beta":
                S = a * (S - kk * p[:, None, :]) + b * kk * v[t][:, None, :]
            elif kind == "erase_sign":
                S = a * (S + b * kk * p[:, None, :]) + b * kk * v[t][:, None, :]
            elif kind == "write_without_beta":
                S = a * (S - b * kk * p[:, None, :]) + kk * v[t][:, None, :]
            elif kind == "no_gate":
                S = (S - b * kk * p[:, None, :]) + b * kk * v[t][:, None, :]
            elif kind == "query_for_key":
                pq = np.einsum("hd,hde->he", q[t], S)
                S = a * (S - b * kk * pq[:, None, :]) + b * kk * v[t][:, None, :]
            else:
                S = a * (S - b * kk * p[:, None, :]) + b * kk * v[t][:, None, :]
            o[t] = np.einsum("hd,hde->he", q[t], S)
        return o, S
    return f


def _worst(pin_list, f):
    """Largest deviation any pin reports; a pin that cannot even run the
    mutant (shape error) counts as catching it."""
    worst = 0.0
    for p in pin_list:
        try:
            worst = max(worst, p(f))
        except ValueError:
            worst = np.inf
    return worst


GLA_PINS = [pins.gla_bruteforce, pins.gla_linear_attention, pins.gla_lfilter]
GDN_PINS = [pins.gdn_matrix_form, pins.gdn_unrolled, pins.gdn_beta_zero, pins.gdn_retrieval,
            pins.gdn_overwrite, pins.gdn_linear_attention,
            lambda f: pins.gdn_orthogonal_keys(f, oracle.gla_sequence)]


def test_unmutated_copies_pass():
    assert max(p(_gla_mutant("none")) for p in GLA_PINS) <= pins.TOL
    assert max(p(_gdn_mutant("none")) for p in GDN_PINS) <= pins.TOL


@pytest.mark.parametrize("kind", ["read_before_update", "no_decay", "decay_on_write", "sign",
                                  "transposed_outer", "decay_index"])
def test_gla_mutant_caught(kind):
    f = _gla_mutant(kind)
    assert _worst(GLA_PINS, f) > 1e-6


@pytest.mark.parametrize("kind", ["gate_everything", "erase_without_beta", "erase_sign",
                                  "write_without_beta", "no_gate", "query_for_key"])
def test_gdn_mutant_caught(kind):
    f = _gdn_mutant(kind)
    assert _worst(GDN_PINS, f) > 1e-6


@pytest.mark.parametrize("kind", ["tap_order", "cache_rows"])
def test_conv_mutant_caught(kind):
    def f(x, w, cu, cache, slots, zero_init=False):
        y, c = oracle.causal_conv1d(x, w[:, ::-1] if kind == "tap_order" else w, cu, cache,
                                    slots, zero_init)
        if kind == "cache_rows":
            c = c.copy()
            c[int(slots[0])] = np.roll(c[int(slots[0])], 1, axis=0)
        return y, c
    assert pins.conv_numpy_convolve(f) > 1e-6


# ---------------------------------------------------------------- normalised linear attention
def _lin_mutant(kind):
    def phi(x):
        if kind == "phi_without_one":
            return np.where(x > 0, x, np.exp(np.minimum(x, 0.0)) - 1.0)
        if kind == "phi_relu":
            return np.maximum(x, 0.0) + 1.0
        return oracle.phi(x)

    def f(q, k, v, S0=None, z0=None, eps=1e-6):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        T, H, dk = q.shape
        S = np.zeros((H, dk, v.shape[2])) if S0 is None else np.array(S0, np.float64)
        z = np.zeros((H, dk)) if z0 is None else np.array(z0, np.float64)
        o = np.zeros((T, H, v.shape[2]))
        for t in range(T):
            pq, pk = phi(q[t]), phi(k[t])
            if kind == "read_before_update":
                o[t] = np.einsum("hd,hde->he", pq, S) / (np.einsum("hd,hd->h", pq, z) + eps)[:, None]
            S = S + pk[:, :, None] * v[t][:, None, :]
            if kind != "frozen_normaliser":
                z = z + pk
            den = np.einsum("hd,hd->h", pk if kind == "key_in_normaliser" else pq, z) + eps
            if kind != "read_before_update":
                o[t] = np.einsum("hd,hde->he", pq, S) / den[:, None]
        return o, S, z
    return f


LIN_PINS = [pins.lin_parallel_form, pins.lin_from_state]


def test_lin_unmutated_copy_passes():
    assert max(p(_lin_mutant("none")) for p in LIN_PINS) <= pins.TOL


@pytest.mark.parametrize("kind", ["phi_without_one", "phi_relu", "read_before_update",
                                  "frozen_normaliser", "key_in_normaliser"])
def test_lin_mutant_caught(kind):
    assert _worst(LIN_PINS, _lin_mutant(kind)) > 1e-6


# ---------------------------------------------------------------- kept states
def _multi_mutant(kind):
    def f(q, k, v, alpha, pool, slot_idx, pos_slots):
        pos = np.array(pos_slots)
        if kind == "position_shift":
            pos = np.roll(pos, 1, axis=1)
        o, out = oracle.gla_decode_multi(q, k, v, alpha, pool, slot_idx, pos)
        if kind == "commits_own_slot":
            out = out.copy()
            out[np.asarray(slot_idx)] = out[pos[:, -1]]
        if kind == "state_before_update":
            _, prev = oracle.gla_decode_multi(q[:, :-1], k[:, :-1], v[:, :-1], alpha[:, :-1],
                                              pool, slot_idx, pos[:, 1:])
            out = out.copy()
            out[pos[:, 1:]] = prev[pos[:, 1:]]
            out[pos[:, 0]] = np.asarray(pool)[np.asarray(slot_idx)]
        return o, out
    return f


@pytest.mark.parametrize("kind", ["position_shift", "commits_own_slot", "state_before_update"])
def test_multi_mutant_caught(kind):
    assert pins.multi_closed_form(oracle.gla_decode_multi) <= pins.TOL
    assert pins.multi_closed_form(_multi_mutant(kind)) > 1e-6


def _ckpt_mutant(kind):
    def f(q, k, v, alpha, cu, pool, slots, ck, interval, zero_init=False):
        if kind == "interval_plus_one_chunk":
            return oracle.gla_varlen_ckpt(q, k, v, alpha, cu, pool, slots, ck, interval + 1, zero_init)
        if kind == "from_zero_state":
            return oracle.gla_varlen_ckpt(q, k, v, alpha, cu, pool, slots, ck, interval, True)
        if kind == "shifted_table":
            return oracle.gla_varlen_ckpt(q, k, v, alpha, cu, pool, slots, np.roll(ck, 1, axis=1),
                                          interval, zero_init)
        return oracle.gla_varlen_ckpt(q, k, v, alpha, cu, pool, slots, ck, interval, zero_init)
    return f


@pytest.mark.parametrize("kind", ["interval_plus_one_chunk", "from_zero_state", "shifted_table"])
def test_ckpt_mutant_caught(kind):
    assert pins.ckpt_closed_form(_ckpt_mutant("none")) <= pins.TOL
    assert pins.ckpt_closed_form(_ckpt_mutant(kind)) > 1e-6


# ---------------------------------------------------------------- decode and zero-init branches
def _lin_decode_mutant(kind):
    def f(q, k, v, pool, zpool, slot_idx, eps=1e-6):
        slots = np.asarray(slot_idx)
        if kind == "wrong_slot":
            slots = np.roll(slots, 1)
        o, P, Z = oracle.lin_attn_decode(q, k, v, pool, zpool, slots, eps)
        if kind == "normaliser_not_written":
            Z = np.asarray(zpool, np.float64).copy()
        if kind == "output_before_update":
            fq = oracle.phi(q)
            S0 = np.asarray(pool, np.float64)[slots]
            z0 = np.asarray(zpool, np.float64)[slots]
            o = np.einsum("rhd,rhde->rhe", fq, S0) / (np.einsum("rhd,rhd->rh", fq, z0) + eps)[..., None]
        return o, P, Z
    return f


@pytest.mark.parametrize("kind", ["wrong_slot", "normaliser_not_written", "output_before_update"])
def test_lin_decode_mutant_caught(kind):
    assert pins.lin_decode_closed_form(_lin_decode_mutant("none")) <= pins.TOL
    assert pins.lin_decode_closed_form(_lin_decode_mutant(kind)) > 1e-6


def _zero_init_mutants(kind):
    """zero-init handled wrongly: ignored altogether, or (normalised linear
    attention) the state reset but not the normaliser."""
    def gla(q, k, v, a, cu, pool, slots, zero_init=False):
        return oracle.gla_varlen(q, k, v, a, cu, pool, slots, zero_init and kind != "ignored")

    def gdn(q, k, v, a, b, cu, pool, slots, zero_init=False):
        return oracle.gdn_varlen(q, k, v, a, b, cu, pool, slots, zero_init and kind != "ignored")

    def lin(q, k, v, cu, pool, zpool, slots, zero_init=False, eps=1e-6):
        if kind == "normaliser_kept" and zero_init:
            P0 = np.asarray(pool, np.float64).copy()
            P0[np.asarray(slots)] = 0.0
            return oracle.lin_attn_varlen(q, k, v, cu, P0, zpool, slots, False, eps)
        return oracle.lin_attn_varlen(q, k, v, cu, pool, zpool, slots, zero_init and kind != "ignored", eps)
    return gla, gdn, lin


@pytest.mark.parametrize("kind", ["ignored", "normaliser_kept"])
def test_zero_init_mutant_caught(kind):
    gla, gdn, lin = _zero_init_mutants("none")
    assert max(pins.gla_zero_init(gla), pins.gdn_zero_init(gdn), pins.lin_zero_init(lin)) <= pins.TOL
    gla, gdn, lin = _zero_init_mutants(kind)
    assert pins.lin_zero_init(lin) > 1e-6
    if kind == "ignored":
        assert pins.gla_zero_init(gla) > 1e-6 and pins.gdn_zero_init(gdn) > 1e-6


@pytest.mark.parametrize("kind", ["ignored", "cache_not_written", "cache_from_old_rows"])
def test_conv_zero_init_mutant_caught(kind):
    def f(x, w, cu, cache, slots, zero_init=False):
        y, c = oracle.causal_conv1d(x, w, cu, cache, slots, zero_init and kind != "ignored")
        if kind == "cache_not_written":
            c = c.copy()
            c[np.asarray(slots)] = np.asarray(cache)[np.asarray(slots)]
        if kind == "cache_from_old_rows":      # the short sequence keeps old cache rows in front
            _, c_old = oracle.causal_conv1d(x, w, cu, cache, slots, False)
            c = c.copy()
            c[int(slots[1])] = c_old[int(slots[1])]
        return y, c
    assert pins.conv_zero_init(oracle.causal_conv1d) <= pins.TOL
    assert pins.conv_zero_init(f) > 1e-6
