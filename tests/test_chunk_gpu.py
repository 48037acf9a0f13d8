"""GPU parity of the chunked prefill kernels (GLA and Gated DeltaNet)
against the fp64 oracle.

GLA: "Inference for linear attention and hybrid architectures", section
"Two ways to write the same computation" (chunked form, state hand-off,
segmented prefill).  Gated DeltaNet: the same section's update with the
decay gate; the chunked form is derived (the page has none) and is checked
here only through the recurrence.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import DEV, check, dev, host, note, rel_err, rne_bf16

pytestmark = pytest.mark.gpu


def run_chunk(kind, w, *, out_dtype="f32", pool=None, chunk=None, cu=None, slots=None,
              zero_init=None, rows=None):
    """Run gla/gdn_chunk_fwd on workload w; returns (o tensor, pool tensor)."""
    import gated_deltanet_gla_amd as G
    sl = slice(None) if rows is None else slice(*rows)
    tin = w.dtype
    q, k, v = dev(w.q[sl], tin), dev(w.k[sl], tin), dev(w.v[sl], tin)
    a = dev(w.alpha[sl])
    pool = dev(w.pool) if pool is None else pool
    cu = dev(w.cu_seqlens) if cu is None else dev(cu)
    slots = dev(w.slot_idx) if slots is None else dev(slots)
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    zi = w.zero_init if zero_init is None else zero_init
    C = chunk or w.chunk
    if kind == "gla":
        o = G.gla_chunk_fwd(q, k, v, a, cu, pool, slots, chunk=C, out_dtype=od, zero_init=zi)
    else:
        o = G.gdn_chunk_fwd(q, k, v, a, dev(w.beta[sl]), cu, pool, slots, chunk=C, out_dtype=od,
                            zero_init=zi)
    torch.cuda.synchronize()
    return o, pool


def run_oracle(kind, w):
    if kind == "gla":
        return oracle.gla_varlen(w.q, w.k, w.v, w.alpha, w.cu_seqlens, w.pool, w.slot_idx,
                                 w.zero_init)
    return oracle.gdn_varlen(w.q, w.k, w.v, w.alpha, w.beta, w.cu_seqlens, w.pool, w.slot_idx,
                             w.zero_init)


def test_page_toy_example_chunked():
    """The page's worked example (T=64, d=16, C=16, fp32, zero state):
    outputs and final state within 1e-5 of the recurrence."""
    w = synth.page_toy_workload()
    note("gla chunk toy")
    o, pool = run_chunk("gla", w)
    o_ref, S_ref = oracle.gla_sequence(w.q, w.k, w.v, w.alpha)
    check(host(o), o_ref, "f32", "o")
    check(host(pool)[0, 0], S_ref[0], "f32", "state")


LENS = [1, 2, 15, 16, 17, 63, 0, 64, 65, 129, 200]


@pytest.mark.parametrize("kind", ["gla", "gdn"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("dk,dv", [(16, 16), (128, 128), (64, 32), (32, 128)])
def test_chunk_varlen_parity(kind, dtype, C, dk, dv):
    zero_init = (C == 32)
    note(f"chunk {kind} {dtype} C={C} dk={dk} dv={dv} zero_init={zero_init}")
    w = synth.random_varlen(1000 + C + dk + dv, LENS, 2, dk, dv, dtype=dtype, gdn=(kind == "gdn"),
                            n_slots=14, zero_init=zero_init, chunk=C)
    o, pool = run_chunk(kind, w)
    o_ref, pool_ref = run_oracle(kind, w)
    check(host(o), o_ref, dtype, "o")
    p = pool.cpu().numpy()
    check(p[w.slot_idx], pool_ref[w.slot_idx], dtype, "state")
    untouched = sorted(set(range(14)) - set(w.slot_idx.tolist()))
    assert np.array_equal(p[untouched], w.pool[untouched])


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_bf16_output_is_rne_of_fp32(kind):
    w = synth.random_varlen(11, [70, 5, 130], 3, 128, 128, dtype="bf16", gdn=(kind == "gdn"))
    note(f"chunk {kind} bf16 out")
    o32, p32 = run_chunk(kind, w, out_dtype="f32")
    o16, p16 = run_chunk(kind, w, out_dtype="bf16")
    assert torch.equal(o16.cpu(), rne_bf16(o32))
    assert torch.equal(p16, p32)


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_deterministic_and_batch_invariant(kind):
    """Two runs are bitwise equal, and a sequence's output and final state do
    not depend on what else is in the batch."""
    w = synth.random_varlen(12, [40, 100, 7], 2, 64, 64, dtype="bf16", gdn=(kind == "gdn"), n_slots=5)
    note(f"chunk {kind} determinism")
    o1, p1 = run_chunk(kind, w)
    o2, p2 = run_chunk(kind, w)
    assert torch.equal(o1, o2) and torch.equal(p1, p2)
    # sequence 1 alone
    s, e = int(w.cu_seqlens[1]), int(w.cu_seqlens[2])
    o3, p3 = run_chunk(kind, w, rows=(s, e), cu=np.array([0, e - s], np.int32),
                       slots=w.slot_idx[1:2])
    assert torch.equal(o3, o1[s:e])
    sl = int(w.slot_idx[1])
    assert torch.equal(p3[sl], p1[sl])


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_invalid_slot_skips_sequence(kind):
    w = synth.random_varlen(13, [20, 30], 2, 32, 32, dtype="f32", gdn=(kind == "gdn"), n_slots=3)
    w.slot_idx = np.array([5, 1], np.int32)
    note(f"chunk {kind} invalid slot")
    import gated_deltanet_gla_amd as G
    q, k, v, a = dev(w.q), dev(w.k), dev(w.v), dev(w.alpha)
    pool = dev(w.pool)
    o = torch.full((50, 2, 32), 7.0, device=DEV)
    if kind == "gla":
        G.gla_chunk_fwd(q, k, v, a, dev(w.cu_seqlens), pool, dev(w.slot_idx), chunk=16, o=o)
    else:
        G.gdn_chunk_fwd(q, k, v, a, dev(w.beta), dev(w.cu_seqlens), pool, dev(w.slot_idx),
                        chunk=16, o=o)
    torch.cuda.synchronize()
    assert torch.all(o[:20] == 7.0)
    assert np.array_equal(pool.cpu().numpy()[[0, 2]], w.pool[[0, 2]])
    o_ref, _ = run_oracle(kind, synth.Workload(**{**w.__dict__, "slot_idx": np.array([0, 1], np.int32)}))
    check(host(o)[20:], o_ref[20:], "f32", "o")


@pytest.mark.parametrize("zero_init", [False, True])
def test_gla_segmented_many_sequences(zero_init):
    """The segmented bf16 path (d=128, C=64) with 600 short sequences
    (lengths 0..40, so each thread of a workgroup's segment lookup sums
    several sequences) around three long ones that split into 4, 6 and 7
    segments of 256 tokens (the last one 1 token long): outputs and final
    states against the recurrence, fp32 and bf16 outputs.  The first pass
    indexes only the segments of split sequences, so here its block numbers
    differ from the segments' workspace slots."""
    rng = np.random.Generator(np.random.PCG64(77))
    short = rng.integers(0, 41, size=600).tolist()
    lens = short[:200] + [1500] + short[200:400] + [1537] + short[400:] + [900]
    w = synth.random_varlen(15 + zero_init, lens, 2, 128, 128, dtype="bf16", zero_init=zero_init)
    note(f"gla segmented, {len(lens)} sequences, zero_init={zero_init}")
    o, pool = run_chunk("gla", w)
    o_ref, pool_ref = run_oracle("gla", w)
    check(host(o), o_ref, "bf16", "o")
    p = pool.cpu().numpy()
    check(p[w.slot_idx], pool_ref[w.slot_idx], "bf16", "state")
    spare = sorted(set(range(p.shape[0])) - set(w.slot_idx.tolist()))
    assert np.array_equal(p[spare], w.pool[spare])
    o16, p16 = run_chunk("gla", w, out_dtype="bf16")
    assert torch.equal(o16.cpu(), rne_bf16(o))
    assert torch.equal(p16, pool)


@pytest.mark.parametrize("zero_init,H", [(False, 2), (True, 2), (False, 5)])
def test_gla_segmented_entry_scan(zero_init, H):
    """Few sequences of many segments (here 16, 10 and 13 segments of 256
    tokens, an empty sequence between them, last segments of 160, 1 and 28
    tokens; H = 5 does not divide the 256 workgroups the segment length
    aims at): the entry states are scanned once over the first pass's slots
    instead of folded in every segment of the output pass.  Outputs and final
    states against the recurrence; bf16 outputs are the RNE of the fp32 ones."""
    lens = [4000, 2305, 0, 3100]
    w = synth.random_varlen(23 + zero_init + 3 * H, lens, H, 128, 128, dtype="bf16", zero_init=zero_init)
    note(f"gla segmented entry scan, lengths {lens}, H={H}, zero_init={zero_init}")
    o, pool = run_chunk("gla", w)
    o_ref, pool_ref = run_oracle("gla", w)
    check(host(o), o_ref, "bf16", "o")
    p = pool.cpu().numpy()
    check(p[w.slot_idx], pool_ref[w.slot_idx], "bf16", "state")
    o16, p16 = run_chunk("gla", w, out_dtype="bf16")
    assert torch.equal(o16.cpu(), rne_bf16(o))
    assert torch.equal(p16, pool)


def test_gla_segmented_no_split_sequences():
    """Many prompts of one segment each (1..256 tokens, under the 320-token
    segment at this size): the first pass launches blocks, none of which
    finds a split sequence, and the output pass starts every sequence from
    its pool slot."""
    rng = np.random.Generator(np.random.PCG64(78))
    lens = rng.integers(1, 257, size=300).tolist()
    lens[::50] = [256] * 6
    w = synth.random_varlen(17, lens, 2, 128, 128, dtype="bf16")
    note(f"gla segmented, {len(lens)} one-segment sequences, {sum(lens)} tokens")
    o, pool = run_chunk("gla", w)
    o_ref, pool_ref = run_oracle("gla", w)
    check(host(o), o_ref, "bf16", "o")
    check(pool.cpu().numpy()[w.slot_idx], pool_ref[w.slot_idx], "bf16", "state")


@pytest.mark.parametrize("zero_init", [False, True])
def test_gla_short_prompts_several_heads_per_block(zero_init):
    """Batches of short prompts run the output pass with several heads of
    one segment per block, their chunks in one stream (4 heads per block at
    these sizes): 98 sequences of 0..200 tokens (empty ones included), one
    of 1200 tokens that splits into two segments and one of 3000 that splits
    into four (entry states folded between heads, from the copy of the
    initial state and from up to three segment slots), 16 heads, and one
    sequence whose slot is outside the pool: it is skipped (its outputs and
    the pool untouched), the others match the recurrence."""
    import gated_deltanet_gla_amd as G
    rng = np.random.Generator(np.random.PCG64(79 + zero_init))
    lens = rng.integers(0, 201, size=98).tolist()
    lens[3] = 0
    lens[40] = 0
    lens = lens[:30] + [1200] + lens[30:70] + [3000] + lens[70:]
    w = synth.random_varlen(19 + zero_init, lens, 16, 128, 128, dtype="bf16", zero_init=zero_init)
    bad = 7
    n_slots = w.pool.shape[0]
    slots = w.slot_idx.copy()
    slots[bad] = n_slots + 2
    note(f"gla short prompts, {len(lens)} sequences x 16 heads, zero_init={zero_init}")
    q, k, v, a = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), dev(w.alpha)
    pool = dev(w.pool)
    o = torch.full(w.q.shape, 7.0, device=DEV)
    G.gla_chunk_fwd(q, k, v, a, dev(w.cu_seqlens), pool, dev(slots), chunk=64, o=o, zero_init=zero_init)
    torch.cuda.synchronize()
    s0, s1 = int(w.cu_seqlens[bad]), int(w.cu_seqlens[bad + 1])
    assert torch.all(o[s0:s1] == 7.0)
    o_ref, pool_ref = run_oracle("gla", w)
    keep = np.ones(w.q.shape[0], bool)
    keep[s0:s1] = False
    check(host(o)[keep], o_ref[keep], "bf16", "o")
    p = pool.cpu().numpy()
    good = np.delete(w.slot_idx, bad)
    check(p[good], pool_ref[good], "bf16", "state")
    untouched = sorted(set(range(n_slots)) - set(good.tolist()))
    assert np.array_equal(p[untouched], w.pool[untouched])


@pytest.mark.parametrize("zero_init", [False, True])
def test_gdn_short_prompts_several_heads_per_block(zero_init):
    """The Gated DeltaNet counterpart: pass 2 of unsplit short prompts runs
    several heads of a segment per block (4 at these sizes), their chunks
    in one stream, next to split sequences handled by the scan and phase B;
    empty sequences and a skipped one (slot outside the pool) included."""
    import gated_deltanet_gla_amd as G
    rng = np.random.Generator(np.random.PCG64(81 + zero_init))
    lens = rng.integers(0, 201, size=98).tolist()
    lens[3] = 0
    lens[40] = 0
    lens = lens[:30] + [1200] + lens[30:70] + [1200] + lens[70:]
    w = synth.random_varlen(21 + zero_init, lens, 16, 128, 128, dtype="bf16", gdn=True, zero_init=zero_init)
    bad = 7
    n_slots = w.pool.shape[0]
    slots = w.slot_idx.copy()
    slots[bad] = n_slots + 2
    note(f"gdn short prompts, {len(lens)} sequences x 16 heads, zero_init={zero_init}")
    q, k, v, a, bt = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), dev(w.alpha), dev(w.beta)
    pool = dev(w.pool)
    o = torch.full(w.q.shape, 7.0, device=DEV)
    G.gdn_chunk_fwd(q, k, v, a, bt, dev(w.cu_seqlens), pool, dev(slots), chunk=64, o=o, zero_init=zero_init)
    torch.cuda.synchronize()
    s0, s1 = int(w.cu_seqlens[bad]), int(w.cu_seqlens[bad + 1])
    assert torch.all(o[s0:s1] == 7.0)
    o_ref, pool_ref = run_oracle("gdn", w)
    keep = np.ones(w.q.shape[0], bool)
    keep[s0:s1] = False
    check(host(o)[keep], o_ref[keep], "bf16", "o")
    p = pool.cpu().numpy()
    good = np.delete(w.slot_idx, bad)
    check(p[good], pool_ref[good], "bf16", "state")
    untouched = sorted(set(range(n_slots)) - set(good.tolist()))
    assert np.array_equal(p[untouched], w.pool[untouched])


def test_gdn_first_segments_run_before_the_scan():
    """A Gated DeltaNet batch of many (sequence, head) pairs (40 x 16) with
    three prompts cut into 4, 4 and 3 segments: there the first segment of
    a cut prompt runs its outputs next to the other segments' first pass
    and its end state seeds the scan, which then starts one segment later.
    Outputs and final states against the recurrence."""
    rng = np.random.Generator(np.random.PCG64(83))
    lens = rng.integers(260, 341, size=37).tolist()
    lens = lens[:5] + [2000] + lens[5:20] + [1990] + lens[20:] + [1500]
    w = synth.random_varlen(23, lens, 16, 128, 128, dtype="bf16", gdn=True)
    note(f"gdn large batch with cut prompts, {len(lens)} sequences x 16 heads, {sum(lens)} tokens")
    o, pool = run_chunk("gdn", w)
    o_ref, pool_ref = run_oracle("gdn", w)
    cu = w.cu_seqlens
    cut = np.zeros(o_ref.shape[0], bool)
    for b in (5, 21, 39):
        cut[cu[b]:cu[b + 1]] = True
    oh = host(o)
    print(f"rel err o: cut prompts {rel_err(oh[cut], o_ref[cut]):.2e}, others {rel_err(oh[~cut], o_ref[~cut]):.2e}")
    check(oh, o_ref, "bf16", "o")
    p = pool.cpu().numpy()
    check(p[w.slot_idx], pool_ref[w.slot_idx], "bf16", "state")
    spare = sorted(set(range(p.shape[0])) - set(w.slot_idx.tolist()))
    assert np.array_equal(p[spare], w.pool[spare])
    o16, p16 = run_chunk("gdn", w, out_dtype="bf16")
    assert torch.equal(o16.cpu(), rne_bf16(o))


def test_gla_prefill_full_size():
    """GLA prefill: 4 x 4096 tokens, 16 heads, d=128, C=64, bf16 inputs,
    zero initial state: every output and final state against the oracle."""
    w = synth.prefill_gla()
    note("gla prefill full size")
    o, pool = run_chunk("gla", w)
    o_ref, pool_ref = run_oracle("gla", w)
    e_o = check(host(o), o_ref, "bf16", "o")
    e_s = check(host(pool), pool_ref, "bf16", "state")
    print(f"gla full: rel err o {e_o:.2e} state {e_s:.2e}")
    o16, _ = run_chunk("gla", w, out_dtype="bf16")
    print(f"gla full: bf16-stored o rel err {rel_err(host(o16), o_ref):.2e} (information)")


def test_gdn_prefill_full_size_and_segments():
    """Gated DeltaNet prefill: 2 x 8192 tokens, 16 heads, d=128, C=64, bf16,
    initial states ~ N(0, 0.05); one pass, and three calls over tokens
    [0,2000), [2000,5000), [5000,8192) that pass only the state."""
    w = synth.prefill_gdn()
    note("gdn prefill full size")
    o, pool = run_chunk("gdn", w)
    o_ref, pool_ref = run_oracle("gdn", w)
    e_o = check(host(o), o_ref, "bf16", "o")
    e_s = check(host(pool), pool_ref, "bf16", "state")
    print(f"gdn full: rel err o {e_o:.2e} state {e_s:.2e}")
    note("gdn prefill segmented")
    T = 8192
    segs = w.extra["segments"]
    pool_s = dev(w.pool)
    outs = []
    for a_, b_ in zip(segs[:-1], segs[1:]):
        # the same token range of both sequences, packed
        idx = np.concatenate([np.arange(a_, b_), T + np.arange(a_, b_)])
        ws = synth.Workload(**{**w.__dict__, "q": w.q[idx], "k": w.k[idx], "v": w.v[idx],
                               "alpha": w.alpha[idx], "beta": w.beta[idx],
                               "cu_seqlens": np.array([0, b_ - a_, 2 * (b_ - a_)], np.int32)})
        os_, pool_s = run_chunk("gdn", ws, pool=pool_s)
        outs.append((idx, host(os_)))
    o_seg = np.zeros_like(o_ref)
    for idx, x in outs:
        o_seg[idx] = x
    check(o_seg, o_ref, "bf16", "o (segments)")
    check(host(pool_s), pool_ref, "bf16", "state (segments)")


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_prefill_then_decode(kind):
    """Prefill T tokens, then decode token T+1 from the same slot: equal to
    the recurrence over T+1 tokens."""
    import gated_deltanet_gla_amd as G
    w = synth.random_varlen(14, [97], 2, 128, 128, dtype="bf16", gdn=(kind == "gdn"), n_slots=2)
    note(f"{kind} prefill then decode")
    wp = synth.Workload(**{**w.__dict__, "cu_seqlens": np.array([0, 96], np.int32)})
    _, pool = run_chunk(kind, wp, rows=(0, 96))
    t = slice(96, 97)
    args = [dev(w.q[t], "bf16"), dev(w.k[t], "bf16"), dev(w.v[t], "bf16"), dev(w.alpha[t])]
    if kind == "gla":
        od = G.gla_decode_step(*args, pool, dev(w.slot_idx), out_dtype=torch.float32)
    else:
        od = G.gdn_decode_step(*args, dev(w.beta[t]), pool, dev(w.slot_idx), out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, pool_ref = run_oracle(kind, w)
    check(host(od)[0], o_ref[96], "bf16", "decode o")
    check(host(pool)[w.slot_idx], pool_ref[w.slot_idx], "bf16", "state")


@pytest.mark.parametrize("kind", ["gla", "gdn"])
@pytest.mark.parametrize("reset", [False, True])
def test_degenerate_gates_many_segments(kind, reset):
    """The gates of test_degenerate_gates (alpha = 1 on a tenth of the
    tokens, with ``reset`` alpha = 0 on another tenth; for Gated DeltaNet
    beta = 0 or 1 on a tenth each) in two long bf16 sequences cut into
    many segments (GLA: 11 and 7 segments of 256 tokens, entry states
    scanned): segment decay totals that underflow to zero and state scales
    restarted mid-segment, against the recurrence."""
    w = synth.random_varlen(31 + reset, [2600, 1700], 2, 128, 128, dtype="bf16", gdn=(kind == "gdn"),
                            chunk=64)
    rng = np.random.Generator(np.random.PCG64(32))
    u = rng.random(w.alpha.shape)
    w.alpha = np.where(u < 0.1, 0.0 if reset else w.alpha, np.where(u > 0.9, 1.0, w.alpha)).astype(np.float32)
    if kind == "gdn":
        u = rng.random(w.beta.shape)
        w.beta = np.where(u < 0.1, 0.0, np.where(u > 0.9, 1.0, w.beta)).astype(np.float32)
    note(f"chunk {kind} bf16 many segments, degenerate gates reset={reset}")
    o, pool = run_chunk(kind, w)
    o_ref, pool_ref = run_oracle(kind, w)
    p = pool.cpu().numpy()[w.slot_idx]
    assert np.all(np.isfinite(host(o))) and np.all(np.isfinite(p))
    check(host(o), o_ref, "bf16", "o")
    check(p, pool_ref[w.slot_idx], "bf16", "state")


@pytest.mark.parametrize("kind", ["gla", "gdn"])
@pytest.mark.parametrize("dtype,d,C", [("bf16", 128, 64), ("f32", 32, 16)])
@pytest.mark.parametrize("reset", [False, True])
def test_degenerate_gates(kind, dtype, d, C, reset):
    """Gates at the ends of their range, against the recurrence: alpha = 1
    (no decay) on a tenth of the tokens and, for Gated DeltaNet, beta
    exactly 0 (no write) or 1 on a tenth each, all inside the parity
    contract; with ``reset`` also alpha exactly 0 (a complete reset) on a
    tenth of the tokens.  A zero gate lies outside the parity contract the
    header states (alpha in (0, 1]): it is taken as 2^-126, which shifts the
    chunk's running log2 decay by -126 per reset, and fp32 keeps log values
    near 126..252 to 2^-17..2^-16, so decays between later tokens of that
    chunk carry ~1e-5 relative error.  That case is held to finite results
    within 5e-5 (fp32); everything else to the contract's bars."""
    w = synth.random_varlen(21 + d, [300, 77, 129], 2, d, d, dtype=dtype, gdn=(kind == "gdn"),
                            chunk=C)
    rng = np.random.Generator(np.random.PCG64(22))
    u = rng.random(w.alpha.shape)
    w.alpha = np.where(u < 0.1, 0.0 if reset else w.alpha, np.where(u > 0.9, 1.0, w.alpha)).astype(np.float32)
    if kind == "gdn":
        u = rng.random(w.beta.shape)
        w.beta = np.where(u < 0.1, 0.0, np.where(u > 0.9, 1.0, w.beta)).astype(np.float32)
    note(f"chunk {kind} {dtype} d={d} C={C} degenerate gates reset={reset}")
    o, pool = run_chunk(kind, w)
    o_ref, pool_ref = run_oracle(kind, w)
    p = pool.cpu().numpy()[w.slot_idx]
    assert np.all(np.isfinite(host(o))) and np.all(np.isfinite(p))
    if dtype == "f32" and reset:
        e_o = float(np.max(np.abs(host(o) - o_ref)))
        e_s = float(np.max(np.abs(p - pool_ref[w.slot_idx])))
        assert e_o <= 5e-5 and e_s <= 5e-5, (e_o, e_s)
    else:
        check(host(o), o_ref, dtype, "o")
        check(p, pool_ref[w.slot_idx], dtype, "state")


@pytest.mark.parametrize("dtype,dk,C", [("bf16", 128, 64), ("f32", 32, 16)])
def test_gdn_prep_then_run_equals_fwd(dtype, dk, C):
    """gdn_chunk_prep followed by gdn_chunk_run gives gdn_chunk_fwd's
    outputs and states bit for bit."""
    import gated_deltanet_gla_amd as G
    w = synth.random_varlen(90 + dk, [300, 1, 0, 129], 2, dk, dk, dtype=dtype, gdn=True, chunk=C)
    note(f"gdn prep+run {dtype} dk={dk} C={C}")
    q, k, v = dev(w.q, dtype), dev(w.k, dtype), dev(w.v, dtype)
    a, b, cu, sl = dev(w.alpha), dev(w.beta), dev(w.cu_seqlens), dev(w.slot_idx)
    p1, p2 = dev(w.pool), dev(w.pool)
    ws = torch.empty(max(1, G.workspace_bytes("gdn", w.n_seqs, w.n_tokens, 2, dk, dk, C)),
                     dtype=torch.uint8, device="cuda:0")
    o1 = G.gdn_chunk_fwd(q, k, v, a, b, cu, p1, sl, chunk=C, out_dtype=torch.float32)
    G.gdn_chunk_prep(q, k, a, b, cu, ws, n_dv=dk, chunk=C)
    o2 = G.gdn_chunk_run(q, k, v, a, b, cu, p2, sl, ws, chunk=C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(p1, p2)


@pytest.mark.parametrize("dk,dv,C,H", [(128, 128, 64, 2), (64, 64, 32, 4), (128, 32, 64, 8)])
def test_gdn_wide_columns_parity(dk, dv, C, H):
    """Many (sequence, head) pairs: the bf16 serial kernel runs 32 state
    columns per workgroup (at least 1024 sixteen-column workgroups' worth of
    work); varlen batch with empty, one-token and partial-chunk sequences."""
    import gated_deltanet_gla_amd as G
    rng = np.random.default_rng(dk + dv + C)
    B = max(8, 1024 // (H * (dv // 16)))
    lengths = rng.integers(0, 3 * C + 7, size=B)
    lengths[:3] = [0, 1, C]
    w = synth.random_varlen(120 + dk + C, lengths.tolist(), H, dk, dv, dtype="bf16", gdn=True,
                            chunk=C)
    note(f"gdn wide dk={dk} dv={dv} C={C} H={H} B={B}")
    pool = dev(w.pool)
    o = G.gdn_chunk_fwd(dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), dev(w.alpha),
                        dev(w.beta), dev(w.cu_seqlens), pool, dev(w.slot_idx), chunk=C,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, p_ref = oracle.gdn_varlen(w.q, w.k, w.v, w.alpha, w.beta, w.cu_seqlens, w.pool,
                                     w.slot_idx)
    check(host(o), o_ref, "bf16", "o")
    check(host(pool)[w.slot_idx], p_ref[w.slot_idx], "bf16", "state")


def test_gdn_batch_invariance_across_column_widths():
    """A sequence prefilled alone (16-column serial workgroups) and inside a
    batch big enough for 32-column workgroups gets bitwise the same outputs
    and final state: both widths accumulate every product in the same order."""
    import gated_deltanet_gla_amd as G
    H, d = 4, 128
    lengths = [333] + [70] * 40           # 41 x 4 heads x 8 tiles > 1024: the wide path
    w = synth.random_varlen(130, lengths, H, d, d, dtype="bf16", gdn=True, n_slots=44)
    note("gdn batch invariance across widths")
    q, k, v = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16")
    a, b = dev(w.alpha), dev(w.beta)
    pool_all = dev(w.pool)
    o_all = G.gdn_chunk_fwd(q, k, v, a, b, dev(w.cu_seqlens), pool_all, dev(w.slot_idx),
                            out_dtype=torch.float32)
    n0 = lengths[0]
    pool_one = dev(w.pool)
    o_one = G.gdn_chunk_fwd(q[:n0].contiguous(), k[:n0].contiguous(), v[:n0].contiguous(),
                            a[:n0].contiguous(), b[:n0].contiguous(),
                            dev(np.array([0, n0], np.int32)), pool_one, dev(w.slot_idx[:1]),
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    s0 = int(w.slot_idx[0])
    assert torch.equal(o_all[:n0], o_one)
    assert torch.equal(pool_all[s0], pool_one[s0])
