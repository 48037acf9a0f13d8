"""GPU parity of the multi-token decode (per-position states kept for
speculative-decoding verification and rollback) and of the slot copy,
against the fp64 oracle.  Sections "Speculative decoding and PD
disaggregation" (a draft token's update cannot be taken back, so every
draft position's state is kept) and "Prefix caching has to be redone" (a
saved state is reused whole, each continuation on its own copy)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import DEV, check, dev, host, note, rne_bf16

pytestmark = pytest.mark.gpu


def _run(kind, w, pos=None, out_dtype="f32"):
    import gated_deltanet_gla_amd as G
    tin = w.dtype
    q, k, v = dev(w.q, tin), dev(w.k, tin), dev(w.v, tin)
    a = dev(w.alpha)
    pool = dev(w.pool)
    slots = dev(w.slot_idx)
    ps = dev(w.extra["pos_slots"] if pos is None else pos)
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    if kind == "gla":
        o = G.gla_decode_multi(q, k, v, a, pool, slots, ps, out_dtype=od)
    else:
        o = G.gdn_decode_multi(q, k, v, a, dev(w.beta), pool, slots, ps, out_dtype=od)
    torch.cuda.synchronize()
    return o, pool


def _oracle(kind, w, pos=None):
    pos = w.extra["pos_slots"] if pos is None else pos
    if kind == "gla":
        return oracle.gla_decode_multi(w.q, w.k, w.v, w.alpha, w.pool, w.slot_idx, pos)
    return oracle.gdn_decode_multi(w.q, w.k, w.v, w.alpha, w.beta, w.pool, w.slot_idx, pos)


def _check_pool(kind, w, pool, pool_ref, dtype):
    p = host(pool)
    named = sorted(set(w.slot_idx.tolist()) | set(int(x) for x in w.extra["pos_slots"].ravel()
                                                   if x >= 0))
    check(p[named], pool_ref[named], dtype, f"{kind} kept states")
    rest = np.ones(w.pool.shape[0], bool)
    rest[named] = False
    assert np.array_equal(pool.cpu().numpy()[rest], w.pool[rest]), "untouched slots changed"


@pytest.mark.parametrize("kind", ["gla", "gdn"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 128), (64, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_tok", [1, 2, 5])
def test_decode_multi_parity(kind, dk, dv, dtype, n_tok):
    note(f"decode_multi {kind} dk={dk} dv={dv} {dtype} n_tok={n_tok}")
    w = synth.decode_multi(seed=30 + dk + dv + n_tok, n_req=5, n_tok=n_tok, H=3, dk=dk, dv=dv,
                           n_slots=5 * (n_tok + 1) + 4, gdn=(kind == "gdn"), dtype=dtype)
    o, pool = _run(kind, w)
    o_ref, pool_ref = _oracle(kind, w)
    check(host(o), o_ref, dtype, f"{kind} o")
    _check_pool(kind, w, pool, pool_ref, dtype)
    # the requests' own slots are only read
    assert np.array_equal(pool.cpu().numpy()[w.slot_idx], w.pool[w.slot_idx])


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_decode_multi_unkept_positions_own_slot_and_invalid(kind):
    """Negative pos_slots keep nothing; a request may commit its last
    position in place; a request whose slot is out of range is skipped."""
    w = synth.decode_multi(seed=40, n_req=4, n_tok=3, H=2, dk=64, dv=64, n_slots=20,
                           gdn=(kind == "gdn"), dtype="f32")
    pos = w.extra["pos_slots"].copy()
    pos[:, 0] = -1
    pos[1, 2] = w.slot_idx[1]          # in-place commit of the last position
    pos[2, 1] = 999                    # out of range: not kept
    slot_bad = w.slot_idx.copy()
    slot_bad[3] = -5                   # request 3 is skipped entirely
    w.slot_idx = slot_bad
    note(f"decode_multi {kind} unkept/own/invalid")
    import gated_deltanet_gla_amd as G
    q, k, v, a = dev(w.q), dev(w.k), dev(w.v), dev(w.alpha)
    pool = dev(w.pool)
    o = torch.full((4, 3, 2, 64), 77.0, device=DEV)
    if kind == "gla":
        G.gla_decode_multi(q, k, v, a, pool, dev(slot_bad), dev(pos), o=o)
    else:
        G.gdn_decode_multi(q, k, v, a, dev(w.beta), pool, dev(slot_bad), dev(pos), o=o)
    torch.cuda.synchronize()
    assert torch.all(o[3] == 77.0)
    # oracle on the three valid requests
    sub = slice(0, 3)
    if kind == "gla":
        o_ref, p_ref = oracle.gla_decode_multi(w.q[sub], w.k[sub], w.v[sub], w.alpha[sub], w.pool,
                                               slot_bad[sub], pos[sub])
    else:
        o_ref, p_ref = oracle.gdn_decode_multi(w.q[sub], w.k[sub], w.v[sub], w.alpha[sub],
                                               w.beta[sub], w.pool, slot_bad[sub], pos[sub])
    check(host(o)[:3], o_ref, "f32", "o")
    check(host(pool), p_ref, "f32", "pool")
    kept3 = pos[3][pos[3] >= 0]
    assert np.array_equal(pool.cpu().numpy()[kept3], w.pool[kept3])


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_decode_multi_bf16_output_is_rne_of_fp32(kind):
    w = synth.decode_multi(seed=41, n_req=3, n_tok=4, H=4, n_slots=15, gdn=(kind == "gdn"))
    note(f"decode_multi {kind} bf16-out")
    o32, _ = _run(kind, w, out_dtype="f32")
    o16, _ = _run(kind, w, out_dtype="bf16")
    assert torch.equal(o16.cpu(), rne_bf16(o32))


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_decode_multi_full_size(kind):
    """256 requests x 4 draft tokens x 16 heads of 128x128 fp32 states,
    every position kept (1280-slot pool); all kept states and outputs are
    compared with the oracle."""
    note(f"decode_multi full {kind}")
    w = synth.decode_multi(seed=6, n_req=256, n_tok=4, n_slots=1280, gdn=(kind == "gdn"))
    o, pool = _run(kind, w)
    o_ref, pool_ref = _oracle(kind, w)
    check(host(o), o_ref, "bf16", "o")
    _check_pool(kind, w, pool, pool_ref, "bf16")


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_speculative_accept_then_continue(kind):
    """Verify 4 drafts, accept 2 (adopt the kept slot of position 2), then
    one ordinary decode step: equals the recurrence over the accepted
    tokens followed by the next token."""
    import gated_deltanet_gla_amd as G
    w = synth.decode_multi(seed=42, n_req=3, n_tok=4, H=2, dk=32, dv=32, n_slots=16,
                           gdn=(kind == "gdn"), dtype="f32")
    nxt = synth.decode_multi(seed=43, n_req=3, n_tok=1, H=2, dk=32, dv=32, n_slots=16,
                             gdn=(kind == "gdn"), dtype="f32")
    note(f"speculative accept {kind}")
    _, pool = _run(kind, w)
    acc = 2
    live = dev(w.extra["pos_slots"][:, acc - 1].copy())
    sq = lambda x: dev(x[:, 0].copy())  # noqa: E731
    if kind == "gla":
        o2 = G.gla_decode_step(sq(nxt.q), sq(nxt.k), sq(nxt.v), sq(nxt.alpha), pool, live)
    else:
        o2 = G.gdn_decode_step(sq(nxt.q), sq(nxt.k), sq(nxt.v), sq(nxt.alpha), sq(nxt.beta),
                               pool, live)
    torch.cuda.synchronize()
    for r in range(3):
        cat = lambda name: np.concatenate([getattr(w, name)[r, :acc],  # noqa: E731
                                           getattr(nxt, name)[r, :1]])
        if kind == "gla":
            o_ref, S_ref = oracle.gla_sequence(cat("q"), cat("k"), cat("v"), cat("alpha"),
                                               S0=w.pool[w.slot_idx[r]])
        else:
            o_ref, S_ref = oracle.gdn_sequence(cat("q"), cat("k"), cat("v"), cat("alpha"),
                                               cat("beta"), S0=w.pool[w.slot_idx[r]])
        check(host(o2)[r], o_ref[-1], "f32", "o after accept")
        check(host(pool)[w.extra["pos_slots"][r, acc - 1]], S_ref, "f32", "state after accept")


@pytest.mark.parametrize("dk,dv,H", [(128, 128, 16), (16, 32, 3), (64, 16, 1)])
def test_state_copy_matches_oracle(dk, dv, H):
    import gated_deltanet_gla_amd as G
    rng = np.random.default_rng(dk + dv + H)
    n = 40
    pool_h = rng.standard_normal((n, H, dk, dv)).astype(np.float32)
    perm = rng.permutation(n)
    src, dst = perm[:12].astype(np.int32), perm[12:24].astype(np.int32)
    src[3] = -1                       # skipped pair
    dst[5] = n + 3                    # skipped pair
    note(f"state_copy dk={dk} dv={dv} H={H}")
    pool = dev(pool_h)
    G.gla_state_copy(pool, dev(src), dev(dst))
    torch.cuda.synchronize()
    ref = oracle.state_copy(pool_h, src, dst)
    assert np.array_equal(pool.cpu().numpy(), ref.astype(np.float32))


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_speculative_replay_strategy(kind):
    """Verify with no state kept, then commit the accepted prefix by
    replaying it in place (the page's record-and-replay alternative):
    verification outputs match the oracle and leave the pool untouched; the
    committed slot equals the state after the accepted tokens."""
    import gated_deltanet_gla_amd as G
    R, J = 16, 4
    w = synth.decode_multi(seed=44, n_req=R, n_tok=J, H=4, dk=128, dv=128, n_slots=R * (J + 1),
                           gdn=(kind == "gdn"))
    q, k, v, a = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), dev(w.alpha)
    b = dev(w.beta) if kind == "gdn" else None
    pool = dev(w.pool)
    slots = dev(w.slot_idx)

    def run(pos):
        if kind == "gla":
            return G.gla_decode_multi(q, k, v, a, pool, slots, dev(pos), out_dtype=torch.float32)
        return G.gdn_decode_multi(q, k, v, a, b, pool, slots, dev(pos), out_dtype=torch.float32)

    note(f"speculative replay {kind}: verify")
    none = np.full((R, J), -1, np.int32)
    o = run(none)
    torch.cuda.synchronize()
    if kind == "gla":
        o_ref, _ = oracle.gla_decode_multi(w.q, w.k, w.v, w.alpha, w.pool, w.slot_idx, none)
    else:
        o_ref, _ = oracle.gdn_decode_multi(w.q, w.k, w.v, w.alpha, w.beta, w.pool, w.slot_idx, none)
    check(host(o), o_ref, "bf16", "verify outputs")
    assert np.array_equal(pool.cpu().numpy(), w.pool), "verification wrote state"

    acc = np.random.default_rng(45).integers(0, J + 1, size=R)
    commit = none.copy()
    for r in range(R):
        if acc[r] > 0:
            commit[r, acc[r] - 1] = w.slot_idx[r]
    note(f"speculative replay {kind}: commit")
    run(commit)
    torch.cuda.synchronize()
    p = host(pool)
    for r in range(R):
        n = int(acc[r])
        S0 = w.pool[w.slot_idx[r]]
        if n == 0:
            assert np.array_equal(pool[int(w.slot_idx[r])].cpu().numpy(), S0)
            continue
        if kind == "gla":
            _, S = oracle.gla_sequence(w.q[r, :n], w.k[r, :n], w.v[r, :n], w.alpha[r, :n], S0=S0)
        else:
            _, S = oracle.gdn_sequence(w.q[r, :n], w.k[r, :n], w.v[r, :n], w.alpha[r, :n],
                                       w.beta[r, :n], S0=S0)
        check(p[w.slot_idx[r]], S, "bf16", f"committed state of request {r} ({n} accepted)")


def test_slot_copy_conv_cache_and_normaliser():
    """A saved prefix needs the conv cache copied with the state ("Prefix
    caching has to be redone"): bf16 conv-cache slots [n, 3, 2048] and fp32
    normaliser slots [n, 16, 128] copied bitwise."""
    import gated_deltanet_gla_amd as G
    rng = np.random.default_rng(46)
    n = 12
    cache = synth.round_bf16(rng.standard_normal((n, 3, 2048)).astype(np.float32))
    zpool = rng.standard_normal((n, 16, 128)).astype(np.float32)
    src = np.array([3, 7, 0, 11], np.int32)
    dst = np.array([5, 1, 9, 2], np.int32)
    note("slot copy conv cache + normaliser")
    c_dev, z_dev = dev(cache, "bf16"), dev(zpool)
    G.gla_slot_copy(c_dev, dev(src), dev(dst))
    G.gla_slot_copy(z_dev, dev(src), dev(dst))
    torch.cuda.synchronize()
    assert np.array_equal(c_dev.float().cpu().numpy(), oracle.state_copy(cache, src, dst))
    assert np.array_equal(z_dev.cpu().numpy(), oracle.state_copy(zpool, src, dst))
