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
