"""GPU parity of the mixed varlen Gated DeltaNet step: conv prelude over all
requests, chunked prefill for the prompts (from their pool states) and
decode for the one-token requests, in one step (sections "Two ways to write
the same computation" and "Speculative decoding and PD disaggregation")."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import check, check_bf16_storage, dev, host, note

pytestmark = pytest.mark.gpu


def _run_step(w):
    from gated_deltanet_gla_amd.step import MixedStep
    P = w.extra["n_prefill"]
    lens = w.extra["lengths"]
    NP = int(lens[:P].sum())
    cu_p = np.concatenate([[0], np.cumsum(lens[:P])]).astype(np.int32)
    pool = dev(w.pool)
    cache = dev(w.extra["conv_cache"], "bf16")
    st = MixedStep(dev(w.extra["x"], "bf16"), dev(w.extra["w"]), cache, dev(w.q, "bf16"),
                   dev(w.k, "bf16"), dev(w.alpha), dev(w.beta), dev(w.cu_seqlens), dev(cu_p), pool,
                   dev(w.slot_idx), P, NP, out_dtype=torch.float32)
    o = st()
    torch.cuda.synchronize()
    return o, pool, cache, st


def _oracle(w, heads):
    """Oracle on a subset of heads (heads are independent)."""
    H = w.q.shape[1]
    d = w.q.shape[2]
    ch = np.concatenate([np.arange(h * d, (h + 1) * d) for h in heads])
    y, cache_out = oracle.causal_conv1d(w.extra["x"][:, ch], w.extra["w"][ch], w.cu_seqlens,
                                        w.extra["conv_cache"][:, :, ch], w.slot_idx)
    v = synth.round_bf16(y.astype(np.float32)).reshape(-1, len(heads), d)   # the layer's bf16 v
    o, pool = oracle.gdn_varlen(w.q[:, heads], w.k[:, heads], v, w.alpha[:, heads],
                                w.beta[:, heads], w.cu_seqlens, w.pool[:, heads], w.slot_idx)
    return o, pool, y, cache_out, ch


def test_mixed_step_small():
    """12 prompts (lengths log-uniform in [16, 1024]) + 40 decodes, all heads."""
    w = synth.mixed_varlen(seed=9, n_prefill=12, n_decode=40, max_len=1024, n_slots=64)
    note("mixed small")
    o, pool, cache, st = _run_step(w)
    heads = list(range(16))
    o_ref, pool_ref, y_ref, c_ref, ch = _oracle(w, heads)
    check_bf16_storage(host(st.y), y_ref, "conv y")
    assert np.array_equal(host(cache), c_ref.astype(np.float32).astype(np.float64))
    check(host(o), o_ref, "bf16", "o")
    check(host(pool)[w.slot_idx], pool_ref[w.slot_idx], "bf16", "state")
    untouched = sorted(set(range(64)) - set(w.slot_idx.tolist()))
    assert np.array_equal(pool.cpu().numpy()[untouched], w.pool[untouched])


def test_mixed_step_full_size_sampled_heads():
    """48 prompts of log-uniform length in [16, 32768] + 512 decodes, 16 heads,
    1024-slot pool: heads 0, 7 and 12 of every request against the oracle,
    and every head's outputs and states finite."""
    w = synth.mixed_varlen()
    note(f"mixed full ({int(w.cu_seqlens[-1])} tokens)")
    o, pool, cache, st = _run_step(w)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(pool).all())
    heads = [0, 7, 12]
    o_ref, pool_ref, y_ref, c_ref, ch = _oracle(w, heads)
    check_bf16_storage(host(st.y)[:, ch], y_ref, "conv y")
    check(host(o)[:, heads], o_ref, "bf16", "o")
    check(host(pool)[w.slot_idx][:, heads], pool_ref[w.slot_idx], "bf16", "state")
