"""GPU parity of the causal conv prelude against the oracle (section "Two
ways to write the same computation", last paragraph; cache width from
section "The real model's ledger")."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import check, check_bf16_storage, dev, host, note

pytestmark = pytest.mark.gpu


def _case(seed, lens, C, W, dtype, n_slots):
    r = np.random.default_rng(seed)
    N = int(sum(lens))
    x = r.standard_normal((N, C)).astype(np.float32)
    cache = r.standard_normal((n_slots, W - 1, C)).astype(np.float32)
    if dtype == "bf16":
        x, cache = synth.round_bf16(x), synth.round_bf16(cache)
    w = (r.standard_normal((C, W)) * 0.5).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = r.permutation(n_slots)[: len(lens)].astype(np.int32)
    return x, w, cu, cache, slots


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [2, 3, 4])
@pytest.mark.parametrize("zero_init", [False, True])
def test_conv_parity(dtype, W, zero_init):
    import gated_deltanet_gla_amd as G
    lens = [1, 0, 2, 37, 16, 1, 5, 0, 100, 3]
    x, w, cu, cache, slots = _case(W, lens, 136, W, dtype, 14)
    note(f"conv {dtype} W={W} zero_init={zero_init}")
    xd, cd = dev(x, dtype), dev(cache, dtype)
    y = G.causal_conv1d_fwd(xd, dev(w), dev(cu), cd, dev(slots), zero_init=zero_init)
    torch.cuda.synchronize()
    y_ref, c_ref = oracle.causal_conv1d(x, w, cu, cache, slots, zero_init)
    # fp32 arithmetic of <= 4 products: a bf16 output differs from the exact
    # value only by the final rounding
    if dtype == "f32":
        check(host(y), y_ref, "f32", "y")
    else:
        check_bf16_storage(host(y), y_ref, "y")
    assert np.array_equal(host(cd), c_ref.astype(np.float32).astype(np.float64))


def test_conv_segments_equal_one_pass():
    import gated_deltanet_gla_amd as G
    x, w, cu, cache, slots = _case(5, [50], 64, 4, "f32", 2)
    note("conv segments")
    c1 = dev(cache)
    y1 = G.causal_conv1d_fwd(dev(x), dev(w), dev(cu), c1, dev(slots))
    c2 = dev(cache)
    ys = []
    for s, e in [(0, 1), (1, 2), (2, 19), (19, 50)]:
        ys.append(G.causal_conv1d_fwd(dev(x[s:e]), dev(w), dev(np.array([0, e - s], np.int32)), c2,
                                      dev(slots)))
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(ys), y1) and torch.equal(c1, c2)
