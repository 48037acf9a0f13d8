"""Pool offsets beyond 32 bits: a 4.1 GiB pool (4200 slots of 16 heads x
128 x 128 fp32) with the requests' slots near its end, so every state
address exceeds 2^32 bytes (section "Speculative decoding and PD
disaggregation": the pool is addressed by slot index; at 1 MiB per slot a
pool of more than 4096 slots needs 64-bit offsets).  The pool is filled on
the device from a seeded generator; the touched slots are copied to the
host before the call and the oracle runs on those."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import DEV, check, dev, host, note

pytestmark = pytest.mark.gpu

N_SLOTS, H, D = 4200, 16, 128


def _pool():
    g = torch.Generator(device=DEV)
    g.manual_seed(99)
    return torch.randn((N_SLOTS, H, D, D), generator=g, device=DEV) * 0.05


def _sub_pool(pool, slots):
    """Host copy of the named slots, renumbered 0..len-1."""
    return pool[torch.from_numpy(np.asarray(slots, np.int64)).to(DEV)].cpu().numpy()


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_decode_high_slots(kind):
    import gated_deltanet_gla_amd as G
    R = 8
    slots = np.arange(N_SLOTS - R, N_SLOTS, dtype=np.int32)[::-1].copy()
    w = synth.decode(seed=60, n_req=R, H=H, d=D, n_slots=R, gdn=(kind == "gdn"),
                     pool=np.zeros((1,), np.float32))
    pool = _pool()
    before = _sub_pool(pool, slots)
    note(f"large pool decode {kind}")
    args = (dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), dev(w.alpha))
    if kind == "gla":
        o = G.gla_decode_step(*args, pool, dev(slots), out_dtype=torch.float32)
        o_ref, p_ref = oracle.gla_decode(w.q, w.k, w.v, w.alpha, before, np.arange(R))
    else:
        o = G.gdn_decode_step(*args, dev(w.beta), pool, dev(slots), out_dtype=torch.float32)
        o_ref, p_ref = oracle.gdn_decode(w.q, w.k, w.v, w.alpha, w.beta, before, np.arange(R))
    torch.cuda.synchronize()
    check(host(o), o_ref, "bf16", "o")
    check(_sub_pool(pool, slots), p_ref, "bf16", "state")


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_chunk_and_checkpoints_high_slots(kind):
    """bf16 d = 128 C = 64 prefill (segmented GLA passes / GDN serial kernel)
    reading and writing slots above 4 GiB, with checkpoints there too."""
    import gated_deltanet_gla_amd as G
    lengths = [600, 130]
    w = synth.random_varlen(61, lengths, H, D, D, dtype="bf16", gdn=(kind == "gdn"), n_slots=2)
    slots = np.array([N_SLOTS - 1, N_SLOTS - 3], np.int32)
    ck = np.array([[N_SLOTS - 2, N_SLOTS - 4], [N_SLOTS - 5, -1]], np.int32)   # every 256 tokens
    pool = _pool()
    named = np.concatenate([slots, ck.ravel()[ck.ravel() >= 0]])
    before = _sub_pool(pool, named)
    note(f"large pool chunk {kind}")
    q, k, v, a = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), dev(w.alpha)
    cu = dev(w.cu_seqlens)
    if kind == "gla":
        o = G.gla_chunk_fwd_ckpt(q, k, v, a, cu, pool, dev(slots), dev(ck), 256,
                                 out_dtype=torch.float32)
    else:
        o = G.gdn_chunk_fwd_ckpt(q, k, v, a, dev(w.beta), cu, pool, dev(slots), dev(ck), 256,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    # oracle on the renumbered sub-pool: sequence slots 0, 1; checkpoints 2.. in table order
    ck_sub = np.array([[2, 3], [4, -1]])
    if kind == "gla":
        o_ref, p_ref = oracle.gla_varlen_ckpt(w.q, w.k, w.v, w.alpha, w.cu_seqlens, before,
                                              [0, 1], ck_sub, 256)
    else:
        o_ref, p_ref = oracle.gdn_varlen_ckpt(w.q, w.k, w.v, w.alpha, w.beta, w.cu_seqlens, before,
                                              [0, 1], ck_sub, 256)
    check(host(o), o_ref, "bf16", "o")
    check(_sub_pool(pool, named), p_ref, "bf16", "final states and checkpoints")


def test_multi_decode_and_copy_high_slots():
    import gated_deltanet_gla_amd as G
    R, J = 4, 3
    w = synth.decode_multi(seed=62, n_req=R, n_tok=J, H=H, dk=D, dv=D, n_slots=R * (J + 1),
                           gdn=True)
    slots = (N_SLOTS - 1 - np.arange(R)).astype(np.int32)
    pos = (N_SLOTS - 1 - R - np.arange(R * J)).reshape(R, J).astype(np.int32)
    pool = _pool()
    named = np.concatenate([slots, pos.ravel()])
    before = _sub_pool(pool, named)
    note("large pool multi-token decode + copy")
    o = G.gdn_decode_multi(dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), dev(w.alpha),
                           dev(w.beta), pool, dev(slots), dev(pos), out_dtype=torch.float32)
    G.gla_state_copy(pool, dev(pos[:, -1].copy()), dev(np.array([5, 6, 7, 8], np.int32)))
    torch.cuda.synchronize()
    o_ref, p_ref = oracle.gdn_decode_multi(w.q, w.k, w.v, w.alpha, w.beta, before, np.arange(R),
                                           (R + np.arange(R * J)).reshape(R, J))
    check(host(o), o_ref, "bf16", "o")
    check(_sub_pool(pool, named), p_ref, "bf16", "kept states")
    assert np.array_equal(_sub_pool(pool, [5, 6, 7, 8]), _sub_pool(pool, pos[:, -1]))
