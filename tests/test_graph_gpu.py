"""Decode and prefill captured in a HIP graph and replayed (section
"Speculative decoding and PD disaggregation": each request's state has a
fixed pool slot and batched kernels address states by slot index, which is
what lets a decode step be captured once and replayed).  The calls allocate
nothing and record no memset, so the graph holds only their kernels.  Each
test replays several times with new inputs copied into the captured
buffers, with eager work and synchronisation between replays, and checks
every replay against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import DEV, check, dev, host, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_decode_step_graph_replays(kind):
    import gated_deltanet_gla_amd as G
    R, H, d = 64, 4, 128
    w0 = synth.decode(seed=70, n_req=R, H=H, d=d, n_slots=256, gdn=(kind == "gdn"))
    pool = dev(w0.pool)
    slots = dev(w0.slot_idx)
    q, k, v = (torch.empty((R, H, d), dtype=torch.bfloat16, device=DEV) for _ in range(3))
    a = torch.empty((R, H), dtype=torch.float32, device=DEV)
    b = torch.empty((R, H), dtype=torch.float32, device=DEV)
    o = torch.empty((R, H, d), dtype=torch.float32, device=DEV)

    def call():
        if kind == "gla":
            G.gla_decode_step(q, k, v, a, pool, slots, o=o)
        else:
            G.gdn_decode_step(q, k, v, a, b, pool, slots, o=o)

    def load(w):
        q.copy_(dev(w.q, "bf16")); k.copy_(dev(w.k, "bf16")); v.copy_(dev(w.v, "bf16"))
        a.copy_(dev(w.alpha))
        if kind == "gdn":
            b.copy_(dev(w.beta))

    # eager warm-up on a side stream, then capture
    load(w0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref_pool = pool.cpu().numpy().astype(np.float64)
    note(f"graph capture decode {kind}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    # capture does not run the kernels: the pool is still the eager result
    assert np.array_equal(pool.cpu().numpy(), ref_pool.astype(np.float32))
    for step in range(4):
        w = synth.decode(seed=71 + step, n_req=R, H=H, d=d, n_slots=256, gdn=(kind == "gdn"),
                         pool=np.zeros((1,), np.float32))
        load(w)
        _ = torch.ones(1 << 20, device=DEV).sum()        # eager work between replays
        torch.cuda.synchronize()
        note(f"graph replay {step} decode {kind}")
        g.replay()
        torch.cuda.synchronize()
        if kind == "gla":
            o_ref, ref_pool = oracle.gla_decode(w.q, w.k, w.v, w.alpha, ref_pool, w0.slot_idx)
        else:
            o_ref, ref_pool = oracle.gdn_decode(w.q, w.k, w.v, w.alpha, w.beta, ref_pool,
                                                w0.slot_idx)
        check(host(o), o_ref, "bf16", f"o, replay {step}")
        check(host(pool)[w0.slot_idx], ref_pool[w0.slot_idx], "bf16", f"state, replay {step}")


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_chunk_prefill_graph_replays(kind):
    """bf16, d = 128, chunk 64 (the segmented GLA passes / the GDN prep and
    serial kernels), zero-initialised slots refilled from the pool each
    replay by the calls themselves."""
    import gated_deltanet_gla_amd as G
    lengths, H = [700, 64, 300], 2
    w0 = synth.random_varlen(80, lengths, H, 128, 128, dtype="bf16", gdn=(kind == "gdn"),
                             zero_init=True)
    N = w0.n_tokens
    pool = dev(np.zeros_like(w0.pool))
    cu, slots = dev(w0.cu_seqlens), dev(w0.slot_idx)
    q, k, v = (torch.empty((N, H, 128), dtype=torch.bfloat16, device=DEV) for _ in range(3))
    a = torch.empty((N, H), dtype=torch.float32, device=DEV)
    b = torch.empty((N, H), dtype=torch.float32, device=DEV)
    o = torch.empty((N, H, 128), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(1, G.workspace_bytes(kind, len(lengths), N, H, 128, 128, 64)),
                     dtype=torch.uint8, device=DEV)

    def call():
        if kind == "gla":
            G.gla_chunk_fwd(q, k, v, a, cu, pool, slots, zero_init=True, o=o, workspace=ws)
        else:
            G.gdn_chunk_fwd(q, k, v, a, b, cu, pool, slots, zero_init=True, o=o, workspace=ws)

    def load(w):
        q.copy_(dev(w.q, "bf16")); k.copy_(dev(w.k, "bf16")); v.copy_(dev(w.v, "bf16"))
        a.copy_(dev(w.alpha))
        if kind == "gdn":
            b.copy_(dev(w.beta))

    load(w0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    note(f"graph capture prefill {kind}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for step in range(3):
        w = synth.random_varlen(81 + step, lengths, H, 128, 128, dtype="bf16", gdn=(kind == "gdn"),
                                zero_init=True)
        load(w)
        _ = torch.ones(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        note(f"graph replay {step} prefill {kind}")
        g.replay()
        torch.cuda.synchronize()
        # the graph captured w0's slot table (the new draw's slots are not used)
        sl = w0.slot_idx
        if kind == "gla":
            o_ref, p_ref = oracle.gla_varlen(w.q, w.k, w.v, w.alpha, w.cu_seqlens, w.pool, sl, True)
        else:
            o_ref, p_ref = oracle.gdn_varlen(w.q, w.k, w.v, w.alpha, w.beta, w.cu_seqlens, w.pool,
                                             sl, True)
        check(host(o), o_ref, "bf16", f"o, replay {step}")
        check(host(pool)[sl], p_ref[sl], "bf16", f"state, replay {step}")
