"""Python binding of the C ABI: torch tensors in, the same names out.

Each function only checks tensor placement/dtype/layout, takes raw device
pointers and the current HIP stream, and calls the library.  Every step of
the computation runs in the HIP kernels; there is no other implementation
here.  Shapes follow include/gla.h.
"""
from __future__ import annotations

import torch

from . import _lib

_DT = {torch.float32: _lib.GLA_F32, torch.bfloat16: _lib.GLA_BF16}


def _ptr(t):
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t):
    """The raw handle of the current HIP stream of t's device.  torch's raw
    accessor skips building a Stream object (about 2 us a call)."""
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(t, name, dtype=None, dims=None):
    """Layout checks of one tensor (dims, dtype, contiguity); the device is
    checked by _devices once every shape has been checked."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, has {t.dim()}")
    if dtype is not None and t.dtype is not dtype and (type(dtype) is not tuple or t.dtype not in dtype):
        raise ValueError(f"{name} has dtype {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t, name, *dims):
    """t.shape must equal dims (None: any size)."""
    s = t.shape
    if s == dims:
        return
    if len(s) == len(dims) and all(d is None or a == d for a, d in zip(s, dims)):
        return
    want = "[" + ", ".join("*" if d is None else str(d) for d in dims) + "]"
    raise ValueError(f"{name} has shape {list(s)}, expected {want}")


def _devices(*named):
    """Every tensor given (None entries skipped) is a device tensor, all on
    the device of the first."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        g = t.get_device()
        if g < 0:
            raise ValueError(f"{name} must be a device tensor")
        if dev is None:
            dev = g
        elif g != dev:
            raise ValueError(f"{name} is on {t.device}, the other arguments on device {dev}")


def _ws_check(workspace):
    if workspace is not None:
        _check(workspace, "workspace")


def _chunk_common(q, k, v, alpha, cu_seqlens, state_pool, slot_idx, out_dtype, o, beta=None,
                  workspace=None, extra=()):
    """Checks of the chunked entry points: q, k [N, H, dk]; v, o [N, H, dv];
    alpha (and beta) [N, H]; cu_seqlens [B + 1]; state_pool
    [n_slots, H, dk, dv]; slot_idx [B]; everything on one device."""
    for t, n, d, nd in [(q, "q", (torch.float32, torch.bfloat16), 3),
                        (k, "k", (torch.float32, torch.bfloat16), 3),
                        (v, "v", (torch.float32, torch.bfloat16), 3),
                        (alpha, "alpha", torch.float32, 2), (cu_seqlens, "cu_seqlens", torch.int32, 1),
                        (state_pool, "state_pool", torch.float32, 4), (slot_idx, "slot_idx", torch.int32, 1)]:
        if t is not None or n != "alpha":     # alpha is None for the ungated operation
            _check(t, n, d, nd)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    N, H, dk = q.shape
    dv = v.shape[2]
    _shape(k, "k", N, H, dk)
    _shape(v, "v", N, H, dv)
    if alpha is not None:
        _shape(alpha, "alpha", N, H)
    if beta is not None:
        _check(beta, "beta", torch.float32, 2)
        _shape(beta, "beta", N, H)
    if cu_seqlens.shape[0] < 1:
        raise ValueError("cu_seqlens must hold n_seqs + 1 entries")
    B = cu_seqlens.shape[0] - 1
    _shape(slot_idx, "slot_idx", B)
    _shape(state_pool, "state_pool", None, H, dk, dv)
    _ws_check(workspace)
    out_dtype = out_dtype or (o.dtype if o is not None else q.dtype)
    if o is not None:
        _check(o, "o", out_dtype, 3)
        _shape(o, "o", N, H, dv)
    _devices(("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta), ("cu_seqlens", cu_seqlens),
             ("state_pool", state_pool), ("slot_idx", slot_idx), ("o", o), ("workspace", workspace),
             *extra)
    if o is None:
        o = torch.empty((N, H, dv), dtype=out_dtype, device=q.device)
    return N, H, dk, dv, out_dtype, o


def gla_chunk_fwd(q, k, v, alpha, cu_seqlens, state_pool, slot_idx, *, chunk=64, out_dtype=None,
                  zero_init=False, o=None, workspace=None):
    """Chunked GLA prefill; updates state_pool[slot_idx] in place, returns o."""
    N, H, dk, dv, out_dtype, o = _chunk_common(q, k, v, alpha, cu_seqlens, state_pool, slot_idx,
                                               out_dtype, o, workspace=workspace)
    B = cu_seqlens.shape[0] - 1
    need = _lib.lib().gla_chunk_workspace_bytes(B, N, H, dk, dv, chunk)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _lib.call("gla_chunk_fwd", q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(),
              cu_seqlens.data_ptr(), B, N, H, dk, dv, chunk, _DT[q.dtype], _DT[out_dtype],
              state_pool.data_ptr(), state_pool.shape[0], slot_idx.data_ptr(),
              _lib.GLA_ZERO_INIT if zero_init else 0, o.data_ptr(), _ptr(workspace),
              0 if workspace is None else workspace.numel() * workspace.element_size(),
              _stream(q))
    return o


def gla_chunk_fwd_noalloc(q, k, v, alpha, cu_seqlens, state_pool, slot_idx, *, chunk=64,
                          out_dtype=None, zero_init=False, o=None):
    """gla_chunk_fwd without a workspace: the library's fixed per-GPU scratch
    array is used instead, so the C call allocates nothing (pass ``o`` to
    allocate nothing here either).  Calls that overlap on one GPU race."""
    N, H, dk, dv, out_dtype, o = _chunk_common(q, k, v, alpha, cu_seqlens, state_pool, slot_idx,
                                               out_dtype, o)
    B = cu_seqlens.shape[0] - 1
    _lib.call("gla_chunk_fwd_noalloc", q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(),
              cu_seqlens.data_ptr(), B, N, H, dk, dv, chunk, _DT[q.dtype], _DT[out_dtype],
              state_pool.data_ptr(), state_pool.shape[0], slot_idx.data_ptr(),
              _lib.GLA_ZERO_INIT if zero_init else 0, o.data_ptr(), _stream(q))
    return o


def gdn_chunk_fwd(q, k, v, alpha, beta, cu_seqlens, state_pool, slot_idx, *, chunk=64,
                  out_dtype=None, zero_init=False, o=None, workspace=None):
    """Chunked Gated DeltaNet prefill; updates state_pool[slot_idx] in place, returns o."""
    N, H, dk, dv, out_dtype, o = _chunk_common(q, k, v, alpha, cu_seqlens, state_pool, slot_idx,
                                               out_dtype, o, beta=beta, workspace=workspace)
    B = cu_seqlens.shape[0] - 1
    need = _lib.lib().gdn_chunk_workspace_bytes(B, N, H, dk, dv, chunk)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _lib.call("gdn_chunk_fwd", q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(),
              beta.data_ptr(), cu_seqlens.data_ptr(), B, N, H, dk, dv, chunk, _DT[q.dtype],
              _DT[out_dtype], state_pool.data_ptr(), state_pool.shape[0], slot_idx.data_ptr(),
              _lib.GLA_ZERO_INIT if zero_init else 0, o.data_ptr(), _ptr(workspace),
              0 if workspace is None else workspace.numel() * workspace.element_size(),
              _stream(q))
    return o


def _ckpt_args(ckpt_slots, ckpt_interval, n_seqs):
    if ckpt_slots.shape[0] != n_seqs:
        raise ValueError("ckpt_slots must be [n_seqs, ckpt_stride]")
    return int(ckpt_interval), ckpt_slots.data_ptr(), ckpt_slots.shape[1]


def gla_chunk_fwd_ckpt(q, k, v, alpha, cu_seqlens, state_pool, slot_idx, ckpt_slots, ckpt_interval,
                       *, chunk=64, out_dtype=None, zero_init=False, o=None, workspace=None):
    """gla_chunk_fwd that also writes the state after every ckpt_interval
    tokens of sequence b to state_pool[ckpt_slots[b, j]] (j-th checkpoint;
    negative = not saved).  ckpt_slots [n_seqs, stride] int32."""
    _check(ckpt_slots, "ckpt_slots", torch.int32, 2)
    N, H, dk, dv, out_dtype, o = _chunk_common(q, k, v, alpha, cu_seqlens, state_pool, slot_idx,
                                               out_dtype, o, workspace=workspace,
                                               extra=(("ckpt_slots", ckpt_slots),))
    B = cu_seqlens.shape[0] - 1
    iv, cp, cs = _ckpt_args(ckpt_slots, ckpt_interval, B)
    need = _lib.lib().gla_chunk_workspace_bytes(B, N, H, dk, dv, chunk)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _lib.call("gla_chunk_fwd_ckpt", q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(),
              cu_seqlens.data_ptr(), B, N, H, dk, dv, chunk, _DT[q.dtype], _DT[out_dtype],
              state_pool.data_ptr(), state_pool.shape[0], slot_idx.data_ptr(),
              _lib.GLA_ZERO_INIT if zero_init else 0, iv, cp, cs, o.data_ptr(), _ptr(workspace),
              0 if workspace is None else workspace.numel() * workspace.element_size(),
              _stream(q))
    return o


def gdn_chunk_fwd_ckpt(q, k, v, alpha, beta, cu_seqlens, state_pool, slot_idx, ckpt_slots,
                       ckpt_interval, *, chunk=64, out_dtype=None, zero_init=False, o=None,
                       workspace=None):
    """Gated DeltaNet form of gla_chunk_fwd_ckpt."""
    _check(ckpt_slots, "ckpt_slots", torch.int32, 2)
    N, H, dk, dv, out_dtype, o = _chunk_common(q, k, v, alpha, cu_seqlens, state_pool, slot_idx,
                                               out_dtype, o, beta=beta, workspace=workspace,
                                               extra=(("ckpt_slots", ckpt_slots),))
    B = cu_seqlens.shape[0] - 1
    iv, cp, cs = _ckpt_args(ckpt_slots, ckpt_interval, B)
    need = _lib.lib().gdn_chunk_workspace_bytes(B, N, H, dk, dv, chunk)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _lib.call("gdn_chunk_fwd_ckpt", q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(),
              beta.data_ptr(), cu_seqlens.data_ptr(), B, N, H, dk, dv, chunk, _DT[q.dtype],
              _DT[out_dtype], state_pool.data_ptr(), state_pool.shape[0], slot_idx.data_ptr(),
              _lib.GLA_ZERO_INIT if zero_init else 0, iv, cp, cs, o.data_ptr(), _ptr(workspace),
              0 if workspace is None else workspace.numel() * workspace.element_size(),
              _stream(q))
    return o


def gdn_chunk_prep(q, k, alpha, beta, cu_seqlens, workspace, *, n_dv, chunk=64):
    """The state-independent part of gdn_chunk_fwd (chunk offsets, inverses,
    planes) into `workspace`; follow it with gdn_chunk_run on the same
    inputs and workspace.  n_dv = d_v of the values that run will get."""
    for t, n in ((q, "q"), (k, "k")):
        _check(t, n, (torch.float32, torch.bfloat16), 3)
    _check(alpha, "alpha", torch.float32, 2)
    _check(beta, "beta", torch.float32, 2)
    _check(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _check(workspace, "workspace")
    if q.dtype != k.dtype:
        raise ValueError("q, k must share a dtype")
    N, H, dk = q.shape
    _shape(k, "k", N, H, dk)
    _shape(alpha, "alpha", N, H)
    _shape(beta, "beta", N, H)
    if cu_seqlens.shape[0] < 1:
        raise ValueError("cu_seqlens must hold n_seqs + 1 entries")
    _devices(("q", q), ("k", k), ("alpha", alpha), ("beta", beta), ("cu_seqlens", cu_seqlens),
             ("workspace", workspace))
    _lib.call("gdn_chunk_prep", q.data_ptr(), k.data_ptr(), alpha.data_ptr(), beta.data_ptr(),
              cu_seqlens.data_ptr(), cu_seqlens.shape[0] - 1, N, H, dk, n_dv, chunk, _DT[q.dtype],
              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
              _stream(q))


def gdn_chunk_run(q, k, v, alpha, beta, cu_seqlens, state_pool, slot_idx, workspace, *, chunk=64,
                  out_dtype=None, zero_init=False, o=None):
    """The serial part of gdn_chunk_fwd, after gdn_chunk_prep on the same
    inputs and workspace; updates state_pool[slot_idx] in place, returns o."""
    _check(workspace, "workspace")
    N, H, dk, dv, out_dtype, o = _chunk_common(q, k, v, alpha, cu_seqlens, state_pool, slot_idx,
                                               out_dtype, o, beta=beta, workspace=workspace)
    _lib.call("gdn_chunk_run", q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(),
              beta.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.shape[0] - 1, N, H, dk, dv, chunk,
              _DT[q.dtype], _DT[out_dtype], state_pool.data_ptr(), state_pool.shape[0],
              slot_idx.data_ptr(), _lib.GLA_ZERO_INIT if zero_init else 0, o.data_ptr(),
              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
              _stream(q))
    return o


def workspace_bytes(kind, n_seqs, n_tokens, n_heads, dk, dv, chunk):
    """Workspace bytes of gla_chunk_fwd ("gla"), gdn_chunk_fwd ("gdn") or
    lin_attn_chunk_fwd ("lin") for these sizes."""
    fn = {"gla": "gla_chunk_workspace_bytes", "gdn": "gdn_chunk_workspace_bytes",
          "lin": "lin_attn_chunk_workspace_bytes"}[kind]
    return getattr(_lib.lib(), fn)(n_seqs, n_tokens, n_heads, dk, dv, chunk)


def _decode_fast_ok(q, k, v, alpha, state_pool, slot_idx, out_dtype, o, beta):
    """The common case of a decode call in one pass of cheap tests: every
    tensor given, contiguous, of the expected dtype and shape, all on one
    device.  False sends the call through the per-tensor checks, which name
    what is wrong."""
    try:
        if o is None or alpha is None or (out_dtype is not None and out_dtype is not o.dtype):
            return False
        dt = q.dtype
        if dt is not torch.bfloat16 and dt is not torch.float32:
            return False
        qs = q.shape
        if len(qs) != 3 or k.shape != qs or k.dtype is not dt or v.dtype is not dt:
            return False
        R, H, dk = qs
        vs = v.shape
        if len(vs) != 3 or vs[0] != R or vs[1] != H or o.shape != vs:
            return False
        ps = state_pool.shape
        if len(ps) != 4 or ps[1] != H or ps[2] != dk or ps[3] != vs[2]:
            return False
        if (alpha.shape != (R, H) or alpha.dtype is not torch.float32 or state_pool.dtype is not torch.float32
                or slot_idx.shape != (R,) or slot_idx.dtype is not torch.int32):
            return False
        ts = (q, k, v, alpha, state_pool, slot_idx, o)
        if beta is not None:
            if beta.shape != (R, H) or beta.dtype is not torch.float32:
                return False
            ts += (beta,)
        g = q.get_device()
        return g >= 0 and all(t.is_contiguous() and t.get_device() == g for t in ts)
    except AttributeError:          # something that is not a tensor
        return False


def _decode_common(q, k, v, alpha, state_pool, slot_idx, out_dtype, o, beta=None, extra=()):
    """Checks of the one-token decode entry points: q, k [R, H, dk]; v, o
    [R, H, dv]; alpha (and beta) [R, H]; state_pool [n_slots, H, dk, dv];
    slot_idx [R]; everything on one device."""
    if _decode_fast_ok(q, k, v, alpha, state_pool, slot_idx, out_dtype, o, beta) and not extra:
        R, H, dk = q.shape
        return R, H, dk, v.shape[2], o.dtype, o
    for t, n, d, nd in [(q, "q", (torch.float32, torch.bfloat16), 3),
                        (k, "k", (torch.float32, torch.bfloat16), 3),
                        (v, "v", (torch.float32, torch.bfloat16), 3),
                        (alpha, "alpha", torch.float32, 2),
                        (state_pool, "state_pool", torch.float32, 4), (slot_idx, "slot_idx", torch.int32, 1)]:
        if t is not None or n != "alpha":     # alpha is None for the ungated operation
            _check(t, n, d, nd)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    R, H, dk = q.shape
    dv = v.shape[2]
    _shape(k, "k", R, H, dk)
    _shape(v, "v", R, H, dv)
    if alpha is not None:
        _shape(alpha, "alpha", R, H)
    if beta is not None:
        _check(beta, "beta", torch.float32, 2)
        _shape(beta, "beta", R, H)
    _shape(slot_idx, "slot_idx", R)
    _shape(state_pool, "state_pool", None, H, dk, dv)
    out_dtype = out_dtype or (o.dtype if o is not None else q.dtype)
    if o is not None:
        _check(o, "o", out_dtype, 3)
        _shape(o, "o", R, H, dv)
    _devices(("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta), ("state_pool", state_pool),
             ("slot_idx", slot_idx), ("o", o), *extra)
    if o is None:
        o = torch.empty((R, H, dv), dtype=out_dtype, device=q.device)
    return R, H, dk, dv, out_dtype, o


def gla_decode_step(q, k, v, alpha, state_pool, slot_idx, *, out_dtype=None, o=None):
    """One GLA decode token per request, in place on state_pool[slot_idx]; returns o."""
    R, H, dk, dv, out_dtype, o = _decode_common(q, k, v, alpha, state_pool, slot_idx, out_dtype, o)
    _lib.call("gla_decode_step", q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(), R, H,
              dk, dv, _DT[q.dtype], _DT[out_dtype], state_pool.data_ptr(), state_pool.shape[0],
              slot_idx.data_ptr(), o.data_ptr(), _stream(q))
    return o


def gdn_decode_step(q, k, v, alpha, beta, state_pool, slot_idx, *, out_dtype=None, o=None):
    """One Gated DeltaNet decode token per request, in place; returns o."""
    R, H, dk, dv, out_dtype, o = _decode_common(q, k, v, alpha, state_pool, slot_idx, out_dtype, o,
                                                beta=beta)
    _lib.call("gdn_decode_step", q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(),
              beta.data_ptr(), R, H, dk, dv, _DT[q.dtype], _DT[out_dtype], state_pool.data_ptr(),
              state_pool.shape[0], slot_idx.data_ptr(), o.data_ptr(), _stream(q))
    return o


def _multi_common(q, k, v, alpha, state_pool, slot_idx, pos_slots, out_dtype, o, beta=None):
    """Checks of the multi-token decode: q, k [R, J, H, dk]; v, o
    [R, J, H, dv]; alpha (and beta) [R, J, H]; state_pool [n_slots, H, dk, dv];
    slot_idx [R]; pos_slots [R, J]; everything on one device."""
    for t, n, d, nd in [(q, "q", (torch.float32, torch.bfloat16), 4),
                        (k, "k", (torch.float32, torch.bfloat16), 4),
                        (v, "v", (torch.float32, torch.bfloat16), 4),
                        (alpha, "alpha", torch.float32, 3),
                        (state_pool, "state_pool", torch.float32, 4),
                        (slot_idx, "slot_idx", torch.int32, 1),
                        (pos_slots, "pos_slots", torch.int32, 2)]:
        _check(t, n, d, nd)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    R, J, H, dk = q.shape
    dv = v.shape[3]
    _shape(k, "k", R, J, H, dk)
    _shape(v, "v", R, J, H, dv)
    _shape(alpha, "alpha", R, J, H)
    if beta is not None:
        _check(beta, "beta", torch.float32, 3)
        _shape(beta, "beta", R, J, H)
    if tuple(pos_slots.shape) != (R, J) or slot_idx.shape[0] != R:
        raise ValueError("pos_slots must be [n_req, n_tok] and slot_idx [n_req]")
    _shape(state_pool, "state_pool", None, H, dk, dv)
    out_dtype = out_dtype or (o.dtype if o is not None else q.dtype)
    if o is not None:
        _check(o, "o", out_dtype, 4)
        _shape(o, "o", R, J, H, dv)
    _devices(("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta), ("state_pool", state_pool),
             ("slot_idx", slot_idx), ("pos_slots", pos_slots), ("o", o))
    if o is None:
        o = torch.empty((R, J, H, dv), dtype=out_dtype, device=q.device)
    return R, J, H, dk, dv, out_dtype, o


def gla_decode_multi(q, k, v, alpha, state_pool, slot_idx, pos_slots, *, out_dtype=None, o=None):
    """n_tok GLA tokens per request from state_pool[slot_idx]; the state after
    position j goes to state_pool[pos_slots[:, j]] (negative = not kept).
    q, k [R, n_tok, H, dk]; v [R, n_tok, H, dv]; alpha [R, n_tok, H]. Returns o."""
    R, J, H, dk, dv, out_dtype, o = _multi_common(q, k, v, alpha, state_pool, slot_idx, pos_slots,
                                                  out_dtype, o)
    _lib.call("gla_decode_multi", q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(), R, J,
              H, dk, dv, _DT[q.dtype], _DT[out_dtype], state_pool.data_ptr(), state_pool.shape[0],
              slot_idx.data_ptr(), pos_slots.data_ptr(), o.data_ptr(), _stream(q))
    return o


def gdn_decode_multi(q, k, v, alpha, beta, state_pool, slot_idx, pos_slots, *, out_dtype=None,
                     o=None):
    """Gated DeltaNet form of gla_decode_multi; beta [R, n_tok, H]."""
    R, J, H, dk, dv, out_dtype, o = _multi_common(q, k, v, alpha, state_pool, slot_idx, pos_slots,
                                                  out_dtype, o, beta=beta)
    _lib.call("gdn_decode_multi", q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(),
              beta.data_ptr(), R, J, H, dk, dv, _DT[q.dtype], _DT[out_dtype],
              state_pool.data_ptr(), state_pool.shape[0], slot_idx.data_ptr(), pos_slots.data_ptr(),
              o.data_ptr(), _stream(q))
    return o


def gla_state_copy(state_pool, src_slots, dst_slots):
    """state_pool[dst_slots[i]] <- state_pool[src_slots[i]] (all heads), in place."""
    _check(state_pool, "state_pool", torch.float32, 4)
    _check(src_slots, "src_slots", torch.int32, 1)
    _check(dst_slots, "dst_slots", torch.int32, 1)
    if src_slots.shape != dst_slots.shape:
        raise ValueError("src_slots and dst_slots must have the same length")
    _devices(("state_pool", state_pool), ("src_slots", src_slots), ("dst_slots", dst_slots))
    n, H, dk, dv = state_pool.shape
    _lib.call("gla_state_copy", state_pool.data_ptr(), n, H, dk, dv, src_slots.data_ptr(),
              dst_slots.data_ptr(), src_slots.shape[0], _stream(state_pool))
    return state_pool


def lin_attn_chunk_fwd(q, k, v, cu_seqlens, state_pool, norm_pool, slot_idx, *, chunk=64,
                       eps=1e-6, out_dtype=None, zero_init=False, o=None, workspace=None):
    """Normalised linear attention (phi = elu + 1), chunked; updates
    state_pool[slot_idx] and norm_pool[slot_idx] ([n_slots, H, dk] fp32) in
    place, returns o."""
    _check(norm_pool, "norm_pool", torch.float32, 3)
    _shape(norm_pool, "norm_pool", state_pool.shape[0] if state_pool.dim() == 4 else None,
           q.shape[1] if q.dim() == 3 else None, q.shape[2] if q.dim() == 3 else None)
    N, H, dk, dv, out_dtype, o = _chunk_common(q, k, v, None, cu_seqlens, state_pool, slot_idx,
                                               out_dtype, o, workspace=workspace,
                                               extra=(("norm_pool", norm_pool),))
    B = cu_seqlens.shape[0] - 1
    need = _lib.lib().lin_attn_chunk_workspace_bytes(B, N, H, dk, dv, chunk)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _lib.call("lin_attn_chunk_fwd", q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(),
              B, N, H, dk, dv, chunk, _DT[q.dtype], _DT[out_dtype],
              state_pool.data_ptr(), norm_pool.data_ptr(), state_pool.shape[0], slot_idx.data_ptr(),
              _lib.GLA_ZERO_INIT if zero_init else 0, float(eps), o.data_ptr(), _ptr(workspace),
              0 if workspace is None else workspace.numel() * workspace.element_size(),
              _stream(q))
    return o


def lin_attn_decode_step(q, k, v, state_pool, norm_pool, slot_idx, *, eps=1e-6, out_dtype=None,
                         o=None):
    """One normalised-linear-attention token per request, in place; returns o."""
    _check(norm_pool, "norm_pool", torch.float32, 3)
    _shape(norm_pool, "norm_pool", state_pool.shape[0] if state_pool.dim() == 4 else None,
           q.shape[1] if q.dim() == 3 else None, q.shape[2] if q.dim() == 3 else None)
    R, H, dk, dv, out_dtype, o = _decode_common(q, k, v, None, state_pool, slot_idx, out_dtype, o,
                                                extra=(("norm_pool", norm_pool),))
    _lib.call("lin_attn_decode_step", q.data_ptr(), k.data_ptr(), v.data_ptr(), R, H, dk, dv,
              _DT[q.dtype], _DT[out_dtype], state_pool.data_ptr(), norm_pool.data_ptr(),
              state_pool.shape[0], slot_idx.data_ptr(), float(eps), o.data_ptr(),
              _stream(q))
    return o


def gla_slot_copy(buf, src_slots, dst_slots):
    """buf[dst_slots[i]] <- buf[src_slots[i]] for a slot-major buffer (a
    normaliser pool, a conv cache), in place."""
    _check(buf, "buf")
    _check(src_slots, "src_slots", torch.int32, 1)
    _check(dst_slots, "dst_slots", torch.int32, 1)
    if src_slots.shape != dst_slots.shape:
        raise ValueError("src_slots and dst_slots must have the same length")
    _devices(("buf", buf), ("src_slots", src_slots), ("dst_slots", dst_slots))
    slot_bytes = buf[0].numel() * buf.element_size() if buf.shape[0] > 0 else 16
    _lib.call("gla_slot_copy", buf.data_ptr(), slot_bytes, buf.shape[0], src_slots.data_ptr(),
              dst_slots.data_ptr(), src_slots.shape[0], _stream(buf))
    return buf


def causal_conv1d_fwd(x, w, cu_seqlens, conv_cache, slot_idx, *, zero_init=False, y=None):
    """Depthwise causal conv with per-slot cache (updated in place); returns y."""
    _check(x, "x", (torch.float32, torch.bfloat16), 2)
    _check(w, "w", torch.float32, 2)
    _check(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _check(conv_cache, "conv_cache", x.dtype, 3)
    _check(slot_idx, "slot_idx", torch.int32, 1)
    N, C = x.shape
    W = w.shape[1]
    _shape(w, "w", C, W)
    if cu_seqlens.shape[0] < 1:
        raise ValueError("cu_seqlens must hold n_seqs + 1 entries")
    _shape(slot_idx, "slot_idx", cu_seqlens.shape[0] - 1)
    _shape(conv_cache, "conv_cache", None, W - 1, C)
    if y is not None:
        _check(y, "y", x.dtype, 2)
        _shape(y, "y", N, C)
    _devices(("x", x), ("w", w), ("cu_seqlens", cu_seqlens), ("conv_cache", conv_cache),
             ("slot_idx", slot_idx), ("y", y))
    if y is None:
        y = torch.empty_like(x)
    _lib.call("causal_conv1d_fwd", x.data_ptr(), w.data_ptr(), cu_seqlens.data_ptr(),
              cu_seqlens.shape[0] - 1, N, C, W, conv_cache.data_ptr(), conv_cache.shape[0],
              slot_idx.data_ptr(), _lib.GLA_ZERO_INIT if zero_init else 0, y.data_ptr(),
              _DT[x.dtype], _stream(x))
    return y


def gla_hbm_probe(mode, state_pool, slot_idx, sink=None):
    """Measurement helper: the decode step's HBM traffic on state_pool at
    slot_idx without its arithmetic (mode 0 read, 1 write zeros, 2 read and
    write back in place, 3 as 2 with two heads per workgroup)."""
    _check(state_pool, "state_pool", torch.float32, 4)
    _check(slot_idx, "slot_idx", torch.int32, 1)
    if sink is None:
        sink = torch.empty(4, dtype=torch.int32, device=state_pool.device)
    _devices(("state_pool", state_pool), ("slot_idx", slot_idx), ("sink", sink))
    n, H, dk, dv = state_pool.shape
    _lib.call("gla_hbm_probe", int(mode), state_pool.data_ptr(), slot_idx.shape[0], H, dk, dv, n,
              slot_idx.data_ptr(), sink.data_ptr(), _stream(state_pool))
