"""GPU parity of the decode step against the fp64 oracle (section "Two ways
to write the same computation", recurrent form; slot-indexed pool of section
"Speculative decoding and PD disaggregation")."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import DEV, check, dev, host, note, rne_bf16

pytestmark = pytest.mark.gpu


def _run(kind, w, out_dtype="f32"):
    import gated_deltanet_gla_amd as G
    tin = w.dtype
    q, k, v = dev(w.q, tin), dev(w.k, tin), dev(w.v, tin)
    a = dev(w.alpha)
    pool = dev(w.pool)
    slots = dev(w.slot_idx)
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    if kind == "gla":
        o = G.gla_decode_step(q, k, v, a, pool, slots, out_dtype=od)
    else:
        o = G.gdn_decode_step(q, k, v, a, dev(w.beta), pool, slots, out_dtype=od)
    torch.cuda.synchronize()
    return o, pool


def _oracle(kind, w):
    if kind == "gla":
        return oracle.gla_decode(w.q, w.k, w.v, w.alpha, w.pool, w.slot_idx)
    return oracle.gdn_decode(w.q, w.k, w.v, w.alpha, w.beta, w.pool, w.slot_idx)


@pytest.mark.parametrize("kind", ["gla", "gdn"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (16, 128), (128, 16)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_parity(kind, dk, dv, dtype):
    note(f"decode {kind} dk={dk} dv={dv} {dtype}")
    w = synth.random_varlen(100 + dk + dv, [1] * 9, 3, dk, dv, dtype=dtype, gdn=(kind == "gdn"),
                            n_slots=13)
    o, pool = _run(kind, w)
    o_ref, pool_ref = _oracle(kind, w)
    check(host(o), o_ref, dtype, "o")
    check(host(pool)[w.slot_idx], pool_ref[w.slot_idx], dtype, "state")
    untouched = sorted(set(range(13)) - set(w.slot_idx.tolist()))
    assert np.array_equal(pool.cpu().numpy()[untouched], w.pool[untouched])


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_decode_bf16_output_is_rne_of_fp32(kind):
    w = synth.random_varlen(7, [1] * 5, 4, 128, 128, dtype="bf16", gdn=(kind == "gdn"), n_slots=6)
    note(f"decode {kind} bf16-out")
    o32, _ = _run(kind, w, "f32")
    o16, _ = _run(kind, w, "bf16")
    assert torch.equal(o16.cpu(), rne_bf16(o32))


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_decode_full_size(kind):
    """256 requests x 16 heads on a 1024-slot pool of 128x128 fp32 states
    ~ N(0, 0.05), random distinct slots; all touched slots and outputs are
    compared with the oracle, untouched slots must keep their bytes."""
    note(f"decode full {kind}")
    w = synth.decode(seed=3, gdn=(kind == "gdn"))
    o, pool = _run(kind, w)
    o_ref, pool_ref = _oracle(kind, w)
    check(host(o), o_ref, "bf16", "o")
    p = pool.cpu().numpy()
    check(p[w.slot_idx], pool_ref[w.slot_idx], "bf16", "state")
    mask = np.ones(1024, bool)
    mask[w.slot_idx] = False
    assert np.array_equal(p[mask], w.pool[mask])


def test_decode_repeated_equals_sequence():
    """64 successive decode calls on the page's worked example (T=64, d=16,
    fp32) reproduce the recurrence within 1e-5."""
    import gated_deltanet_gla_amd as G
    w = synth.page_toy_workload()
    note("decode toy x64")
    pool = dev(np.zeros((1, 1, 16, 16), np.float32))
    slots = dev(np.array([0], np.int32))
    outs = []
    for t in range(64):
        outs.append(G.gla_decode_step(dev(w.q[t:t + 1]), dev(w.k[t:t + 1]), dev(w.v[t:t + 1]),
                                      dev(w.alpha[t:t + 1]), pool, slots))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gla_sequence(w.q, w.k, w.v, w.alpha)
    check(np.concatenate([host(x) for x in outs]), o_ref, "f32", "o")
    check(host(pool)[0], S_ref, "f32", "state")


def test_decode_invalid_slot_is_skipped():
    import gated_deltanet_gla_amd as G
    w = synth.random_varlen(8, [1, 1, 1], 2, 32, 32, dtype="f32", n_slots=4)
    w.slot_idx = np.array([0, 7, 2], np.int32)      # 7 is outside the pool
    note("decode invalid slot")
    q, k, v, a = dev(w.q), dev(w.k), dev(w.v), dev(w.alpha)
    pool = dev(w.pool)
    o = torch.full((3, 2, 32), 123.0, device=DEV)
    G.gla_decode_step(q, k, v, a, pool, dev(w.slot_idx), o=o)
    torch.cuda.synchronize()
    assert torch.all(o[1] == 123.0)
    p = pool.cpu().numpy()
    assert np.array_equal(p[[1, 3]], w.pool[[1, 3]])
