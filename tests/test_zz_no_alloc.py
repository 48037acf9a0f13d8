"""gla_chunk_fwd_noalloc, the entry point for callers that cannot allocate:
its results must equal gla_chunk_fwd's (same kernels, the library's fixed
per-GPU scratch array in place of the caller's workspace), on two calls in
a row where the second is smaller and finds the first call's segment
states still in the array; calls that need more than the array are refused
before anything runs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import check, dev, host, note

pytestmark = pytest.mark.gpu


def _both(w, out_dtype=torch.float32):
    """The same workload through gla_chunk_fwd_noalloc and gla_chunk_fwd,
    each on its own copy of the pool; returns host copies of both."""
    import gated_deltanet_gla_amd as G
    t = w.dtype
    q, k, v, a = dev(w.q, t), dev(w.k, t), dev(w.v, t), dev(w.alpha)
    cu, sl = dev(w.cu_seqlens), dev(w.slot_idx)
    N, H, dv = w.v.shape
    p1, p2 = dev(w.pool), dev(w.pool)
    o1 = torch.full((N, H, dv), float("nan"), dtype=out_dtype, device="cuda:0")
    o2 = torch.full((N, H, dv), float("nan"), dtype=out_dtype, device="cuda:0")
    G.gla_chunk_fwd_noalloc(q, k, v, a, cu, p1, sl, chunk=w.chunk, zero_init=w.zero_init, o=o1)
    G.gla_chunk_fwd(q, k, v, a, cu, p2, sl, chunk=w.chunk, zero_init=w.zero_init, o=o2)
    torch.cuda.synchronize()
    return host(o1), host(o2), p1.cpu().numpy(), p2.cpu().numpy()


def test_noalloc_equals_workspace_call_twice_then_smaller():
    # 1: three long sequences cut into many segments (bf16, d = 128, chunk 64)
    w = synth.random_varlen(71, [2500, 1500, 700], 16, 128, 128, dtype="bf16", n_slots=7)
    note("noalloc gla, 3 sequences 4700 tokens x 16 heads")
    o1, o2, p1, p2 = _both(w)
    assert np.array_equal(o1, o2) and np.array_equal(p1, p2)
    # 2: a smaller call right after it, the scratch holding call 1's states
    w = synth.random_varlen(72, [300, 77, 0, 129], 16, 128, 128, dtype="bf16", n_slots=9)
    note("noalloc gla, 4 sequences 506 tokens x 16 heads (second call)")
    o1, o2, p1, p2 = _both(w)
    assert np.array_equal(o1, o2) and np.array_equal(p1, p2)
    o_ref, p_ref = oracle.gla_varlen(w.q, w.k, w.v, w.alpha, w.cu_seqlens, w.pool, w.slot_idx,
                                     w.zero_init)
    check(o1, o_ref, "bf16", "o")
    check(p1[w.slot_idx], p_ref[w.slot_idx], "bf16", "state")
    rest = sorted(set(range(9)) - set(w.slot_idx.tolist()))
    assert np.array_equal(p1[rest], w.pool[rest])


def test_noalloc_many_segments_scanned():
    """One 5000-token sequence over 16 heads is cut into 16 segments, so the
    entry states are scanned between the passes, in the fixed array too."""
    w = synth.random_varlen(75, [5000], 16, 128, 128, dtype="bf16", n_slots=3)
    note("noalloc gla, 1 sequence of 5000 tokens x 16 heads (scanned entry states)")
    o1, o2, p1, p2 = _both(w)
    assert np.array_equal(o1, o2) and np.array_equal(p1, p2)


def test_noalloc_shapes_without_segments():
    """fp32 inputs and small heads run the generic kernel, which needs no
    workspace: the call is then gla_chunk_fwd with nothing extra."""
    w = synth.random_varlen(73, [90, 33], 2, 32, 32, dtype="f32", chunk=16, n_slots=4)
    note("noalloc gla fp32 d=32 C=16")
    o1, o2, p1, p2 = _both(w)
    assert np.array_equal(o1, o2) and np.array_equal(p1, p2)
    o_ref, p_ref = oracle.gla_varlen(w.q, w.k, w.v, w.alpha, w.cu_seqlens, w.pool, w.slot_idx,
                                     w.zero_init)
    check(o1, o_ref, "f32", "o")
    check(p1[w.slot_idx], p_ref[w.slot_idx], "f32", "state")


def test_noalloc_refuses_calls_beyond_its_scratch():
    """300 sequences of 8 tokens need about 326 MB of segment states, more
    than the fixed array: the call returns GLA_ESCRATCH and touches nothing."""
    import gated_deltanet_gla_amd as G
    from gated_deltanet_gla_amd import _lib
    w = synth.random_varlen(74, [8] * 300, 16, 128, 128, dtype="bf16", n_slots=300)
    need = G.workspace_bytes("gla", 300, 2400, 16, 128, 128, 64)
    assert need > _lib.GLA_NOALLOC_SCRATCH_BYTES
    q, k, v, a = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), dev(w.alpha)
    pool = dev(w.pool)
    o = torch.zeros((2400, 16, 128), dtype=torch.bfloat16, device="cuda:0")
    note("noalloc gla, refused size")
    with pytest.raises(_lib.GlaError) as e:
        G.gla_chunk_fwd_noalloc(q, k, v, a, dev(w.cu_seqlens), pool, dev(w.slot_idx), o=o)
    assert e.value.status == _lib.GLA_ESCRATCH
    torch.cuda.synchronize()
    assert not o.any() and np.array_equal(pool.cpu().numpy(), w.pool)
