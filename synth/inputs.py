"""Seeded synthetic inputs shaped like the workloads of
"Inference for linear attention and hybrid architectures" (the worked example
in section "Two ways to write the same computation", and the 16-head 128x128
fp32-state layers of section "The real model's ledger").

Every generator returns plain numpy arrays.  bf16 tensors are stored as
``uint16`` bit patterns (``*_bits``) together with their exact fp32 values,
so the oracle (fp64) and the device path see identical numbers.

Draw order inside one generator is fixed: q, k, v, alpha, beta, S0, slots,
lengths (whatever subset the workload has), all from one
``numpy.random.Generator(PCG64(seed))``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "bf16_bits", "bf16_to_f32", "round_bf16", "sigmoid",
    "Workload", "page_toy_example", "prefill_gla", "prefill_gdn", "decode",
    "mixed_varlen", "random_varlen", "loguniform_lengths", "page_toy_workload", "decode_multi",
    "lin_attn_varlen",
]


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> exact fp32 value."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded (RNE) to the nearest bf16, returned as fp32."""
    return bf16_to_f32(bf16_bits(x))


def sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32)
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True)).astype(np.float32)
    return (x / n).astype(np.float32)


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------
@dataclass
class Workload:
    """One batch of inputs.

    Token-major packed layout: q, k [N, H, dk]; v [N, H, dv]; alpha, beta
    [N, H]; cu_seqlens [B+1] int32; state pool [n_slots, H, dk, dv] fp32;
    slot_idx [B] int32.  ``dtype`` is the storage format of q, k, v ("f32"
    or "bf16"); for "bf16" the fp32 arrays hold the exact bf16 values and the
    ``*_bits`` arrays their bit patterns.
    """
    name: str
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    cu_seqlens: np.ndarray
    pool: np.ndarray
    slot_idx: np.ndarray
    zero_init: bool
    chunk: int = 64
    beta: np.ndarray | None = None
    extra: dict = field(default_factory=dict)

    @property
    def n_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def n_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def dk(self) -> int:
        return int(self.q.shape[2])

    @property
    def dv(self) -> int:
        return int(self.v.shape[2])

    @property
    def n_seqs(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    def bits(self, name: str) -> np.ndarray:
        """bf16 bit pattern of q, k or v (bf16 workloads only)."""
        assert self.dtype == "bf16"
        return bf16_bits(getattr(self, name))


def _bf16(x: np.ndarray) -> np.ndarray:
    return round_bf16(x.astype(np.float32))


# --------------------------------------------------------------------------
# the pages' worked example
# --------------------------------------------------------------------------
def page_toy_example():
    """The GLA example of "Two ways to write the same computation":
    T=64, d_k=d_v=16, C=16, drawn with torch's CPU generator after
    ``manual_seed(0)`` in the page's call order: q, k, v, then the gate
    (q, k ~ N(0,1)/4, v ~ N(0,1), alpha = sigmoid(N(0,1) + 3)).
    Returns fp32 numpy arrays (T, d) and (T,).
    """
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(0)
    T, DK, DV = 64, 16, 16
    q = torch.randn(T, DK, generator=g) / 4
    k = torch.randn(T, DK, generator=g) / 4
    v = torch.randn(T, DV, generator=g)
    alpha = torch.sigmoid(torch.randn(T, generator=g) + 3)
    return q.numpy(), k.numpy(), v.numpy(), alpha.numpy()


def page_toy_workload() -> Workload:
    """The worked example as a one-sequence, one-head fp32 workload, C=16."""
    q, k, v, a = page_toy_example()
    return Workload(
        name="gla-toy-T64-d16-C16-f32", dtype="f32",
        q=q[:, None, :].copy(), k=k[:, None, :].copy(), v=v[:, None, :].copy(),
        alpha=a[:, None].copy(), cu_seqlens=np.array([0, 64], np.int32),
        pool=np.zeros((1, 1, 16, 16), np.float32), slot_idx=np.array([0], np.int32),
        zero_init=True, chunk=16)


# --------------------------------------------------------------------------
# generic generators
# --------------------------------------------------------------------------
def _qkv(rng, N, H, dk, dv, dtype, normalise_k):
    qs = 1.0 / math.sqrt(dk)
    if normalise_k:
        q = _l2_normalise(rng.standard_normal((N, H, dk), dtype=np.float32))
        k = _l2_normalise(rng.standard_normal((N, H, dk), dtype=np.float32))
    else:
        q = rng.standard_normal((N, H, dk), dtype=np.float32) * np.float32(qs)
        k = rng.standard_normal((N, H, dk), dtype=np.float32) * np.float32(qs)
    v = rng.standard_normal((N, H, dv), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = _bf16(q), _bf16(k), _bf16(v)
    return q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)


def _gates(rng, N, H, with_beta):
    alpha = sigmoid(rng.standard_normal((N, H), dtype=np.float32) + np.float32(3.0))
    beta = sigmoid(rng.standard_normal((N, H), dtype=np.float32)) if with_beta else None
    return alpha, beta


def random_varlen(seed: int, lengths, n_heads: int, dk: int, dv: int, *,
                  dtype: str = "bf16", gdn: bool = False, n_slots: int | None = None,
                  zero_init: bool = False, state_std: float = 0.05, chunk: int = 64,
                  name: str = "varlen") -> Workload:
    """Packed variable-length batch with the value recipe of the prefill
    workloads: q, k ~ N(0,1)/sqrt(dk) (GLA) or L2-normalised N(0,1) (GDN),
    v ~ N(0,1), alpha = sigmoid(N(0,1)+3), beta = sigmoid(N(0,1)), states
    ~ N(0, state_std) in a pool of ``n_slots`` slots (default: one per
    sequence plus 3 spare), slots a random distinct subset."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = [int(x) for x in lengths]
    N = int(sum(lengths))
    H = n_heads
    q, k, v = _qkv(rng, N, H, dk, dv, dtype, normalise_k=gdn)
    alpha, beta = _gates(rng, N, H, gdn)
    B = len(lengths)
    n_slots = n_slots if n_slots is not None else B + 3
    pool = (rng.standard_normal((n_slots, H, dk, dv), dtype=np.float32) * np.float32(state_std))
    slots = rng.permutation(n_slots)[:B].astype(np.int32)
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    return Workload(name=name, dtype=dtype, q=q, k=k, v=v, alpha=alpha, beta=beta,
                    cu_seqlens=cu, pool=pool, slot_idx=slots, zero_init=zero_init,
                    chunk=chunk)


# --------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------
def prefill_gla(seed: int = 2, batch: int = 4, T: int = 4096, H: int = 16, d: int = 128,
                chunk: int = 64) -> Workload:
    """GLA chunked prefill: batch x T tokens packed, H heads, d_k=d_v=d, C=chunk;
    q,k = bf16(N(0,1)/sqrt(d)), v = bf16(N(0,1)), alpha = sigmoid(N(0,1)+3) fp32;
    zero initial state in slots 0..batch-1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    N = batch * T
    q, k, v = _qkv(rng, N, H, d, d, "bf16", normalise_k=False)
    alpha, _ = _gates(rng, N, H, False)
    cu = (np.arange(batch + 1) * T).astype(np.int32)
    return Workload(name=f"gla-prefill-{batch}x{T}-H{H}-d{d}-C{chunk}-bf16", dtype="bf16",
                    q=q, k=k, v=v, alpha=alpha, cu_seqlens=cu,
                    pool=np.zeros((batch, H, d, d), np.float32),
                    slot_idx=np.arange(batch, dtype=np.int32), zero_init=True, chunk=chunk)


def prefill_gdn(seed: int = 4, batch: int = 2, T: int = 8192, H: int = 16, d: int = 128,
                chunk: int = 64) -> Workload:
    """Gated DeltaNet chunked prefill: batch x T tokens, q,k = bf16(L2-normalised
    N(0,1)) per (token, head), v = bf16(N(0,1)), alpha = sigmoid(N(0,1)+3),
    beta = sigmoid(N(0,1)); initial states ~ N(0, 0.05) in slots 0..batch-1.
    ``extra['segments']`` holds the three-call split 2000/3000/rest."""
    rng = np.random.Generator(np.random.PCG64(seed))
    N = batch * T
    q, k, v = _qkv(rng, N, H, d, d, "bf16", normalise_k=True)
    alpha, beta = _gates(rng, N, H, True)
    pool = rng.standard_normal((batch, H, d, d), dtype=np.float32) * np.float32(0.05)
    cu = (np.arange(batch + 1) * T).astype(np.int32)
    segs = [0, min(2000, T), min(5000, T), T]
    return Workload(name=f"gdn-prefill-{batch}x{T}-H{H}-d{d}-C{chunk}-bf16", dtype="bf16",
                    q=q, k=k, v=v, alpha=alpha, beta=beta, cu_seqlens=cu, pool=pool,
                    slot_idx=np.arange(batch, dtype=np.int32), zero_init=False, chunk=chunk,
                    extra={"segments": segs})


def decode(seed: int = 3, n_req: int = 256, H: int = 16, d: int = 128, n_slots: int = 1024,
           gdn: bool = False, pool: np.ndarray | None = None) -> Workload:
    """One decode token per request: pool [n_slots,H,d,d] ~ N(0,0.05) fp32,
    slot ids = the first n_req of a random permutation of n_slots;
    q = bf16(N(0,1)/sqrt(d)), v = bf16(N(0,1)), k as q (GLA) or L2-normalised
    (GDN); alpha = sigmoid(N(0,1)+3), beta = sigmoid(N(0,1)).
    ``extra['perm']`` is the full permutation (its disjoint quarters are
    used to rotate slot sets between timed iterations)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if pool is None:
        pool = rng.standard_normal((n_slots, H, d, d), dtype=np.float32) * np.float32(0.05)
    perm = rng.permutation(n_slots).astype(np.int32)
    slots = perm[:n_req].copy()
    q = _bf16(rng.standard_normal((n_req, H, d), dtype=np.float32) * np.float32(1 / math.sqrt(d)))
    if gdn:
        k = _bf16(_l2_normalise(rng.standard_normal((n_req, H, d), dtype=np.float32)))
    else:
        k = _bf16(rng.standard_normal((n_req, H, d), dtype=np.float32) * np.float32(1 / math.sqrt(d)))
    v = _bf16(rng.standard_normal((n_req, H, d), dtype=np.float32))
    alpha = sigmoid(rng.standard_normal((n_req, H), dtype=np.float32) + np.float32(3.0))
    beta = sigmoid(rng.standard_normal((n_req, H), dtype=np.float32))
    cu = np.arange(n_req + 1, dtype=np.int32)
    return Workload(name=f"{'gdn' if gdn else 'gla'}-decode-{n_req}req-H{H}-d{d}-pool{n_slots}",
                    dtype="bf16", q=q, k=k, v=v, alpha=alpha, beta=beta if gdn else None,
                    cu_seqlens=cu, pool=pool, slot_idx=slots, zero_init=False, chunk=1,
                    extra={"perm": perm})


def loguniform_lengths(rng, n: int, lo: int = 16, hi: int = 32768) -> np.ndarray:
    """n lengths round(exp(U(ln lo, ln hi))) clipped to [lo, hi]."""
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))
    return np.clip(np.round(x), lo, hi).astype(np.int64)


def mixed_varlen(seed: int = 5, n_prefill: int = 48, n_decode: int = 512, H: int = 16,
                 d: int = 128, n_slots: int = 1024, conv_width: int = 4,
                 max_len: int = 32768, min_len: int = 16) -> Workload:
    """Mixed varlen GDN step: n_prefill prompts of log-uniform length in
    [min_len, max_len] followed by n_decode one-token requests, packed in that
    order.  Channels = H*d.  x = bf16(N(0,1)) [N, H*d]; conv weights
    w = N(0,1)/2 fp32 [H*d, width]; conv caches bf16(N(0,1)) [n_slots,
    width-1, H*d]; pool ~ N(0,0.05); q,k L2-normalised bf16; alpha, beta as
    the GDN prefill; v is the conv output (computed by whoever runs the step).
    Slots: the first n_prefill+n_decode of a permutation of n_slots."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = loguniform_lengths(rng, n_prefill, min_len, max_len)
    lens = np.concatenate([lengths, np.ones(n_decode, np.int64)])
    N = int(lens.sum())
    B = int(lens.shape[0])
    Cch = H * d
    q = _bf16(_l2_normalise(rng.standard_normal((N, H, d), dtype=np.float32)))
    k = _bf16(_l2_normalise(rng.standard_normal((N, H, d), dtype=np.float32)))
    alpha, beta = _gates(rng, N, H, True)
    pool = rng.standard_normal((n_slots, H, d, d), dtype=np.float32) * np.float32(0.05)
    perm = rng.permutation(n_slots).astype(np.int32)
    slots = perm[:B].copy()
    x = _bf16(rng.standard_normal((N, Cch), dtype=np.float32))
    w = (rng.standard_normal((Cch, conv_width), dtype=np.float32) * np.float32(0.5)).astype(np.float32)
    conv_cache = _bf16(rng.standard_normal((n_slots, conv_width - 1, Cch), dtype=np.float32))
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    return Workload(name=f"gdn-mixed-{n_prefill}p+{n_decode}d-H{H}-d{d}-conv{conv_width}",
                    dtype="bf16", q=q, k=k, v=np.zeros((N, H, d), np.float32), alpha=alpha,
                    beta=beta, cu_seqlens=cu, pool=pool, slot_idx=slots, zero_init=False,
                    chunk=64, extra={"x": x, "w": w, "conv_cache": conv_cache,
                                     "n_prefill": n_prefill, "n_decode": n_decode,
                                     "lengths": lens})


def decode_multi(seed: int = 6, n_req: int = 256, n_tok: int = 4, H: int = 16, dk: int = 128,
                 dv: int = 128, n_slots: int = 2048, gdn: bool = False,
                 dtype: str = "bf16") -> Workload:
    """n_tok draft tokens per request (speculative-decoding verification)
    with a slot for every position's state.  q, k, v [n_req, n_tok, H, d]
    with the decode value recipe (q = N(0,1)/sqrt(dk), k as q or
    L2-normalised for GDN, v = N(0,1)); alpha, beta [n_req, n_tok, H] as
    decode; pool [n_slots, H, dk, dv] ~ N(0, 0.05).  From one permutation
    of the slots: slot_idx = its first n_req entries, and
    ``extra['pos_slots']`` [n_req, n_tok] the next n_req * n_tok."""
    assert n_slots >= n_req * (n_tok + 1)
    rng = np.random.Generator(np.random.PCG64(seed))
    M = n_req * n_tok
    q, k, v = _qkv(rng, M, H, dk, dv, dtype, normalise_k=False)
    if gdn:
        k = _l2_normalise(rng.standard_normal((M, H, dk), dtype=np.float32))
        if dtype == "bf16":
            k = _bf16(k)
    alpha, beta = _gates(rng, M, H, True)
    pool = rng.standard_normal((n_slots, H, dk, dv), dtype=np.float32) * np.float32(0.05)
    perm = rng.permutation(n_slots).astype(np.int32)
    slots = perm[:n_req].copy()
    pos = perm[n_req:n_req + M].reshape(n_req, n_tok).copy()
    r4 = lambda x: x.reshape(n_req, n_tok, *x.shape[1:]).copy()  # noqa: E731
    cu = (np.arange(n_req + 1) * n_tok).astype(np.int32)
    return Workload(name=f"{'gdn' if gdn else 'gla'}-decode-multi-{n_req}req-x{n_tok}-H{H}-"
                         f"d{dk}x{dv}-pool{n_slots}",
                    dtype=dtype, q=r4(q), k=r4(k), v=r4(v), alpha=r4(alpha),
                    beta=r4(beta) if gdn else None, cu_seqlens=cu, pool=pool, slot_idx=slots,
                    zero_init=False, chunk=1, extra={"pos_slots": pos, "perm": perm})


def lin_attn_varlen(seed: int, lengths, n_heads: int = 16, dk: int = 128, dv: int = 128, *,
                    dtype: str = "bf16", n_slots: int | None = None, zero_init: bool = False,
                    chunk: int = 64, name: str = "lin-attn") -> Workload:
    """Inputs for normalised kernelised linear attention: q, k, v ~ N(0,1)
    (unit scale, so the feature map sees both signs over a wide range);
    states ~ N(0,1) * 4 and normalisers ~ U(16, 48) (positive, like a sum of
    positive features over an earlier prefix) in a pool of ``n_slots``;
    slots a random distinct subset.  ``extra['zpool']`` [n_slots, H, dk]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = [int(x) for x in lengths]
    N, H, B = int(sum(lengths)), n_heads, len(lengths)
    q = rng.standard_normal((N, H, dk), dtype=np.float32)
    k = rng.standard_normal((N, H, dk), dtype=np.float32)
    v = rng.standard_normal((N, H, dv), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = _bf16(q), _bf16(k), _bf16(v)
    n_slots = n_slots if n_slots is not None else B + 3
    pool = rng.standard_normal((n_slots, H, dk, dv), dtype=np.float32) * np.float32(4.0)
    zpool = rng.uniform(16.0, 48.0, size=(n_slots, H, dk)).astype(np.float32)
    slots = rng.permutation(n_slots)[:B].astype(np.int32)
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    return Workload(name=name, dtype=dtype, q=q.astype(np.float32), k=k.astype(np.float32),
                    v=v.astype(np.float32), alpha=np.ones((N, H), np.float32), cu_seqlens=cu,
                    pool=pool, slot_idx=slots, zero_init=zero_init, chunk=chunk,
                    extra={"zpool": zpool})
