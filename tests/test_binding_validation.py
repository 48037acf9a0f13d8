"""Host-side checks of the Python binding's argument validation: tensors of
the wrong shape, dtype or layout are refused with ValueError before any
call reaches the library (so no kernel can index past a buffer), and the
device check comes last, so CPU tensors with correct shapes are refused
only for not being on the GPU.  No GPU is needed."""
import pytest
import torch

import gated_deltanet_gla_amd as G

N, H, D, B, NS = 10, 2, 16, 2, 5
f32, bf, i32 = torch.float32, torch.bfloat16, torch.int32


def chunk_args(**over):
    a = dict(q=torch.zeros(N, H, D, dtype=bf), k=torch.zeros(N, H, D, dtype=bf),
             v=torch.zeros(N, H, D, dtype=bf), alpha=torch.ones(N, H),
             cu_seqlens=torch.tensor([0, 4, N], dtype=i32), state_pool=torch.zeros(NS, H, D, D),
             slot_idx=torch.tensor([0, 3], dtype=i32))
    a.update(over)
    return a


def decode_args(**over):
    a = dict(q=torch.zeros(B, H, D, dtype=bf), k=torch.zeros(B, H, D, dtype=bf),
             v=torch.zeros(B, H, D, dtype=bf), alpha=torch.ones(B, H), state_pool=torch.zeros(NS, H, D, D),
             slot_idx=torch.tensor([0, 3], dtype=i32))
    a.update(over)
    return a


def _call(fn, a, **kw):
    names = list(a)
    return fn(*[a[n] for n in names], **kw)


CHUNK_BAD = {
    "k rows": dict(k=torch.zeros(N - 1, H, D, dtype=bf)),
    "k width": dict(k=torch.zeros(N, H, 2 * D, dtype=bf)),
    "v rows": dict(v=torch.zeros(N + 1, H, D, dtype=bf)),
    "v heads": dict(v=torch.zeros(N, H + 1, D, dtype=bf)),
    "alpha rows": dict(alpha=torch.ones(N - 1, H)),
    "alpha heads": dict(alpha=torch.ones(N, 1)),
    "pool heads": dict(state_pool=torch.zeros(NS, H + 1, D, D)),
    "pool dk": dict(state_pool=torch.zeros(NS, H, D // 2, D)),
    "pool dv": dict(state_pool=torch.zeros(NS, H, D, D * 2)),
    "slot count": dict(slot_idx=torch.tensor([0, 1, 2], dtype=i32)),
    "slot dtype": dict(slot_idx=torch.tensor([0, 1], dtype=torch.int64)),
    "cu empty": dict(cu_seqlens=torch.zeros(0, dtype=i32)),
    "q non-contiguous": dict(q=torch.zeros(N, D, H, dtype=bf).transpose(1, 2)),
    "mixed dtypes": dict(v=torch.zeros(N, H, D, dtype=f32)),
}


@pytest.mark.parametrize("case", sorted(CHUNK_BAD))
@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_chunk_shape_mismatch_refused(kind, case):
    a = chunk_args(**CHUNK_BAD[case])
    with pytest.raises(ValueError) as e:
        if kind == "gla":
            _call(G.gla_chunk_fwd, a)
        else:
            a = dict(list(a.items())[:4] + [("beta", torch.ones(N, H))] + list(a.items())[4:])
            _call(G.gdn_chunk_fwd, a)
    assert "device tensor" not in str(e.value), e.value


def test_chunk_output_and_beta_shapes_refused():
    with pytest.raises(ValueError, match="o has shape"):
        _call(G.gla_chunk_fwd, chunk_args(), o=torch.zeros(N, H, D + 1, dtype=bf))
    a = chunk_args()
    a = dict(list(a.items())[:4] + [("beta", torch.ones(N, H + 1))] + list(a.items())[4:])
    with pytest.raises(ValueError, match="beta has shape"):
        _call(G.gdn_chunk_fwd, a)


def test_well_formed_host_tensors_refused_only_for_the_device():
    with pytest.raises(ValueError, match="device tensor"):
        _call(G.gla_chunk_fwd, chunk_args())
    with pytest.raises(ValueError, match="device tensor"):
        _call(G.gla_decode_step, decode_args())


DECODE_BAD = {
    "k rows": dict(k=torch.zeros(B + 1, H, D, dtype=bf)),
    "v width": dict(v=torch.zeros(B, H, D + 16, dtype=bf)),
    "alpha": dict(alpha=torch.ones(B, H + 1)),
    "pool": dict(state_pool=torch.zeros(NS, H, D, D + 16)),
    "slots": dict(slot_idx=torch.tensor([0], dtype=i32)),
}


@pytest.mark.parametrize("case", sorted(DECODE_BAD))
def test_decode_shape_mismatch_refused(case):
    with pytest.raises(ValueError) as e:
        _call(G.gla_decode_step, decode_args(**DECODE_BAD[case]))
    assert "device tensor" not in str(e.value)
    a = decode_args(**DECODE_BAD[case])
    a = dict(list(a.items())[:4] + [("beta", torch.ones(B, H))] + list(a.items())[4:])
    with pytest.raises(ValueError) as e:
        _call(G.gdn_decode_step, a)
    assert "device tensor" not in str(e.value)


class _OnDevice0(torch.Tensor):
    """A CPU tensor that reports device index 0, so the decode fast path's
    shape and dtype tests can be exercised without a GPU."""

    def get_device(self):
        return 0


def _dev0(t):
    return torch.Tensor._make_subclass(_OnDevice0, t)


@pytest.mark.parametrize("gdn", [False, True])
def test_decode_fast_path_accepts_only_valid_calls(gdn):
    """The one-pass test that lets a valid decode call skip the per-tensor
    checks accepts the valid call and nothing else: every mismatch of the
    table above, a wrong dtype, a non-contiguous tensor, a missing output
    and a tensor on another device send the call to the detailed checks."""
    from gated_deltanet_gla_amd import ops

    def args(**over):
        a = decode_args(**over)
        a = {n: _dev0(t) for n, t in a.items()}
        a["o"] = _dev0(over.get("o", torch.zeros(B, H, D, dtype=bf)))
        a["beta"] = _dev0(over.get("beta", torch.ones(B, H))) if gdn else None
        return a

    def ok(a, out_dtype=None):
        return ops._decode_fast_ok(a["q"], a["k"], a["v"], a["alpha"], a["state_pool"], a["slot_idx"],
                                   out_dtype, a["o"], a["beta"])

    assert ok(args())
    assert ok(args(), out_dtype=bf)
    assert not ok(args(), out_dtype=f32)
    for case, over in DECODE_BAD.items():
        assert not ok(args(**over)), case
    assert not ok(args(k=torch.zeros(B, H, D, dtype=f32)))
    assert not ok(args(q=torch.zeros(B, H, D, dtype=torch.float16), k=torch.zeros(B, H, D, dtype=torch.float16),
                       v=torch.zeros(B, H, D, dtype=torch.float16)))
    assert not ok(args(alpha=torch.ones(B, H, dtype=torch.float64)))
    assert not ok(args(slot_idx=torch.tensor([0, 3], dtype=torch.int64)))
    assert not ok(args(o=torch.zeros(B, H, D + 16, dtype=bf)))
    assert not ok(args(v=torch.zeros(B, D, H, dtype=bf).transpose(1, 2)))
    if gdn:
        assert not ok(args(beta=torch.ones(B, H + 1)))
    a = args()
    a["o"] = None
    assert not ok(a)
    a = args()
    a["state_pool"] = torch.zeros(NS, H, D, D)          # reports no device
    assert not ok(a)


def test_multi_and_norm_pool_and_conv_shapes_refused():
    J = 3
    q = torch.zeros(B, J, H, D, dtype=bf)
    with pytest.raises(ValueError, match="alpha has shape"):
        G.gla_decode_multi(q, q.clone(), q.clone(), torch.ones(B, J + 1, H), torch.zeros(NS, H, D, D),
                           torch.tensor([0, 1], dtype=i32), torch.zeros(B, J, dtype=i32))
    with pytest.raises(ValueError, match="norm_pool has shape"):
        G.lin_attn_decode_step(torch.zeros(B, H, D, dtype=bf), torch.zeros(B, H, D, dtype=bf),
                               torch.zeros(B, H, D, dtype=bf), torch.zeros(NS, H, D, D),
                               torch.zeros(NS, H, D + 1), torch.tensor([0, 1], dtype=i32))
    with pytest.raises(ValueError, match="norm_pool has shape"):
        G.lin_attn_chunk_fwd(torch.zeros(N, H, D, dtype=bf), torch.zeros(N, H, D, dtype=bf),
                             torch.zeros(N, H, D, dtype=bf), torch.tensor([0, N], dtype=i32),
                             torch.zeros(NS, H, D, D), torch.zeros(NS - 1, H, D),
                             torch.tensor([1], dtype=i32))
    C, W = 32, 4
    x = torch.zeros(N, C, dtype=bf)
    cu = torch.tensor([0, 4, N], dtype=i32)
    sl = torch.tensor([0, 2], dtype=i32)
    for bad in [dict(w=torch.zeros(C + 1, W)), dict(cache=torch.zeros(NS, W, C, dtype=bf)),
                dict(cache=torch.zeros(NS, W - 1, C + 8, dtype=bf)), dict(slots=torch.tensor([0], dtype=i32))]:
        args = dict(w=torch.zeros(C, W), cache=torch.zeros(NS, W - 1, C, dtype=bf), slots=sl)
        args.update(bad)
        with pytest.raises(ValueError) as e:
            G.causal_conv1d_fwd(x, args["w"], cu, args["cache"], args["slots"])
        assert "device tensor" not in str(e.value)
