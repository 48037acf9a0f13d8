"""GPU parity of normalised kernelised linear attention (phi = elu + 1,
normaliser z, eps) against the fp64 oracle: page "Long context, fast
inference, smart decoding, and life beyond attention", section "Linear
attention: removing softmax entirely" and its running-state listing."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import DEV, check, dev, host, note, rne_bf16

pytestmark = pytest.mark.gpu


def _chunk(w, out_dtype="f32", eps=1e-6):
    import gated_deltanet_gla_amd as G
    pool, zpool = dev(w.pool), dev(w.extra["zpool"])
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    o = G.lin_attn_chunk_fwd(dev(w.q, w.dtype), dev(w.k, w.dtype), dev(w.v, w.dtype),
                             dev(w.cu_seqlens), pool, zpool, dev(w.slot_idx), chunk=w.chunk,
                             eps=eps, out_dtype=od, zero_init=w.zero_init)
    torch.cuda.synchronize()
    return o, pool, zpool


def _ref(w, eps=1e-6):
    return oracle.lin_attn_varlen(w.q, w.k, w.v, w.cu_seqlens, w.pool, w.extra["zpool"],
                                  w.slot_idx, w.zero_init, eps)


def _check_state(x, ref, dtype, what):
    """fp32 inputs: the normaliser z (a sum of positive features) and S grow
    with the number of tokens, to hundreds here, where one fp32 ulp already
    exceeds 1e-5; they are held to 1e-5 of their scale, max(1, max|ref|).
    bf16 inputs: the usual 3e-3 max relative error."""
    if dtype == "f32":
        e = float(np.abs(x - ref).max() / max(1.0, np.abs(ref).max()))
        assert e <= 1e-5, f"{what}: scaled err {e:.3e} > 1e-05"
    else:
        check(x, ref, dtype, what)


def _check_all(w, o, pool, zpool, ref, dtype):
    o_ref, p_ref, z_ref = ref
    check(host(o), o_ref, dtype, "o")
    _check_state(host(pool)[w.slot_idx], p_ref[w.slot_idx], dtype, "S")
    _check_state(host(zpool)[w.slot_idx], z_ref[w.slot_idx], dtype, "z")
    rest = sorted(set(range(w.pool.shape[0])) - set(w.slot_idx.tolist()))
    assert np.array_equal(pool.cpu().numpy()[rest], w.pool[rest])
    assert np.array_equal(zpool.cpu().numpy()[rest], w.extra["zpool"][rest])


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16)])
@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lin_attn_chunk_parity(dk, dv, C, dtype):
    lengths = [2 * C + 5, 1, 0, C, 3 * C - 1]
    note(f"lin_attn chunk dk={dk} dv={dv} C={C} {dtype} lengths={lengths}")
    w = synth.lin_attn_varlen(600 + dk + dv + C, lengths, 3, dk, dv, dtype=dtype, chunk=C)
    o, pool, zpool = _chunk(w)
    _check_all(w, o, pool, zpool, _ref(w), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lin_attn_chunk_zero_init_and_eps(dtype):
    w = synth.lin_attn_varlen(610, [200, 64, 7], 2, 64, 64, dtype=dtype, chunk=64, zero_init=True)
    note(f"lin_attn zero-init eps {dtype}")
    for eps in (1e-6, 0.5):
        o, pool, zpool = _chunk(w, eps=eps)
        _check_all(w, o, pool, zpool, _ref(w, eps), dtype)


@pytest.mark.parametrize("zero_init", [False, True])
@pytest.mark.parametrize("lengths,H", [([1000, 77, 0, 640, 300], 2), ([2050, 256, 64], 3),
                                       ([257, 1], 1), ([3000, 1800], 2)])
def test_lin_attn_segmented_parity(lengths, H, zero_init):
    """bf16, d = 128, chunk 64: sequences cut into segments of 256 tokens
    (several per sequence here), each segment's sum of phi(k) handed on
    with its state (the last case has 12 and 8 segments a sequence: its
    entry states and normalisers are scanned once instead of folded)."""
    note(f"lin_attn segmented lengths={lengths} H={H} zero_init={zero_init}")
    w = synth.lin_attn_varlen(650 + H + len(lengths), lengths, H, 128, 128, dtype="bf16", chunk=64,
                              zero_init=zero_init)
    o, pool, zpool = _chunk(w)
    _check_all(w, o, pool, zpool, _ref(w), "bf16")


def test_lin_attn_bf16_output_is_rne_of_fp32():
    w = synth.lin_attn_varlen(611, [300, 40], 4, 128, 128, dtype="bf16")
    note("lin_attn bf16-out")
    o32, _, _ = _chunk(w, "f32")
    o16, _, _ = _chunk(w, "bf16")
    assert torch.equal(o16.cpu(), rne_bf16(o32))


@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 128), (128, 128), (128, 16)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lin_attn_decode_parity(dk, dv, dtype):
    import gated_deltanet_gla_amd as G
    w = synth.lin_attn_varlen(620 + dk + dv, [1] * 9, 3, dk, dv, dtype=dtype, n_slots=13)
    note(f"lin_attn decode dk={dk} dv={dv} {dtype}")
    pool, zpool = dev(w.pool), dev(w.extra["zpool"])
    o = G.lin_attn_decode_step(dev(w.q, dtype), dev(w.k, dtype), dev(w.v, dtype), pool, zpool,
                               dev(w.slot_idx), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.lin_attn_decode(w.q, w.k, w.v, w.pool, w.extra["zpool"], w.slot_idx)
    _check_all(w, o, pool, zpool, ref, dtype)


def test_lin_attn_prefill_then_decode_equals_sequence():
    """Prefill 100 tokens, then decode 20 one at a time through the pool:
    the same as the recurrence over all 120 (fp32, 1e-5)."""
    import gated_deltanet_gla_amd as G
    w = synth.lin_attn_varlen(630, [120], 2, 32, 32, dtype="f32", chunk=16, zero_init=True)
    note("lin_attn prefill + decode")
    pool, zpool = dev(w.pool), dev(w.extra["zpool"])
    slots = dev(w.slot_idx)
    o1 = G.lin_attn_chunk_fwd(dev(w.q[:100]), dev(w.k[:100]), dev(w.v[:100]),
                              dev(np.array([0, 100], np.int32)), pool, zpool, slots, chunk=16,
                              zero_init=True)
    outs = [G.lin_attn_decode_step(dev(w.q[t:t + 1]), dev(w.k[t:t + 1]), dev(w.v[t:t + 1]), pool,
                                   zpool, slots) for t in range(100, 120)]
    torch.cuda.synchronize()
    o_ref, S_ref, z_ref = oracle.lin_attn_sequence(w.q, w.k, w.v)
    check(np.concatenate([host(o1)] + [host(x) for x in outs]), o_ref, "f32", "o")
    _check_state(host(pool)[w.slot_idx[0]], S_ref, "f32", "S")
    _check_state(host(zpool)[w.slot_idx[0]], z_ref, "f32", "z")


def test_lin_attn_full_size():
    """4 sequences x 4096 tokens, 16 heads, d = 128, chunk 64, bf16 (the
    prefill benchmark shape), from pool states."""
    note("lin_attn full size")
    w = synth.lin_attn_varlen(640, [4096] * 4, 16, 128, 128, dtype="bf16", chunk=64)
    o, pool, zpool = _chunk(w)
    _check_all(w, o, pool, zpool, _ref(w), "bf16")
