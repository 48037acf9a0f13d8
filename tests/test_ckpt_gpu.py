"""GPU parity of the chunked prefills that save state checkpoints at block
boundaries, against the fp64 oracle (section "Prefix caching has to be
redone": a prefix is reusable only where a whole state was saved, so
engines save states at block boundaries during prefill)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import check, dev, host, note

pytestmark = pytest.mark.gpu


def _ckpt_table(w, interval, stride, n_extra, seed):
    """Pool with n_extra spare slots appended; a checkpoint slot table drawn
    from the spare slots (a few entries left negative)."""
    rng = np.random.default_rng(seed)
    B = w.n_seqs
    n0 = w.pool.shape[0]
    pool = np.concatenate([w.pool, (rng.standard_normal((n_extra,) + w.pool.shape[1:]) * 0.05)
                           .astype(np.float32)])
    spare = rng.permutation(np.arange(n0, n0 + n_extra))[:B * stride]
    ck = spare.reshape(B, stride).astype(np.int32)
    if B * stride > 3:
        ck.flat[1] = -1
    return pool, ck


def _run(kind, w, pool_h, ck, interval, out_dtype="f32"):
    import gated_deltanet_gla_amd as G
    tin = w.dtype
    q, k, v, a = dev(w.q, tin), dev(w.k, tin), dev(w.v, tin), dev(w.alpha)
    pool = dev(pool_h)
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    args = (dev(w.cu_seqlens), pool, dev(w.slot_idx), dev(ck), interval)
    if kind == "gla":
        o = G.gla_chunk_fwd_ckpt(q, k, v, a, *args, chunk=w.chunk, out_dtype=od,
                                 zero_init=w.zero_init)
    else:
        o = G.gdn_chunk_fwd_ckpt(q, k, v, a, dev(w.beta), *args, chunk=w.chunk, out_dtype=od,
                                 zero_init=w.zero_init)
    torch.cuda.synchronize()
    return o, pool


def _oracle(kind, w, pool_h, ck, interval):
    if kind == "gla":
        return oracle.gla_varlen_ckpt(w.q, w.k, w.v, w.alpha, w.cu_seqlens, pool_h, w.slot_idx, ck,
                                      interval, w.zero_init)
    return oracle.gdn_varlen_ckpt(w.q, w.k, w.v, w.alpha, w.beta, w.cu_seqlens, pool_h, w.slot_idx,
                                  ck, interval, w.zero_init)


CASES = [
    # (dtype, d_k, d_v, chunk, H, lengths, interval, stride): bf16 d=128 C=64 runs the
    # segmented GLA path (segments of 256 tokens here) and the bf16 GDN serial kernel
    ("bf16", 128, 128, 64, 2, [1000, 77, 0, 640, 300], 64, 16),
    ("bf16", 128, 128, 64, 2, [1000, 513, 129], 192, 4),
    ("bf16", 128, 128, 64, 3, [2050, 256], 256, 9),
    # 11 and 7 segments a sequence: the GLA entry states are scanned, not folded
    ("bf16", 128, 128, 64, 2, [2600, 1700], 128, 21),
    ("bf16", 64, 64, 32, 2, [300, 31, 160], 96, 3),
    ("f32", 32, 32, 16, 2, [100, 16, 47], 16, 7),
    ("f32", 16, 64, 16, 1, [64, 63], 32, 2),
]


@pytest.mark.parametrize("kind", ["gla", "gdn"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-d{c[1]}x{c[2]}-C{c[3]}-iv{c[6]}" for c in CASES])
def test_chunk_ckpt_parity(kind, case):
    dtype, dk, dv, C, H, lengths, iv, stride = case
    note(f"ckpt {kind} {dtype} dk={dk} dv={dv} C={C} lengths={lengths} interval={iv}")
    w = synth.random_varlen(500 + dk + iv, lengths, H, dk, dv, dtype=dtype, gdn=(kind == "gdn"),
                            chunk=C, zero_init=(kind == "gla"))
    pool_h, ck = _ckpt_table(w, iv, stride, len(lengths) * stride + 3, seed=iv)
    o, pool = _run(kind, w, pool_h, ck, iv)
    o_ref, pool_ref = _oracle(kind, w, pool_h, ck, iv)
    check(host(o), o_ref, dtype, f"{kind} o")
    p = host(pool)
    saved = sorted(set(int(x) for x in ck.ravel() if x >= 0) | set(w.slot_idx.tolist()))
    check(p[saved], pool_ref[saved], dtype, f"{kind} checkpoints and final states")
    # checkpoints past a sequence's end and every other slot keep their bytes
    same = np.all(pool_ref == pool_h.astype(np.float64), axis=(1, 2, 3))
    assert np.array_equal(pool.cpu().numpy()[same], pool_h[same])


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_ckpt_reuse_equals_uncut_prompt(kind):
    """Continue a second request from a copy of the first request's
    checkpoint (copy-on-write prefix sharing): its outputs match the uncut
    prompt's outputs after the shared prefix."""
    import gated_deltanet_gla_amd as G
    note(f"ckpt reuse {kind}")
    w = synth.random_varlen(77, [1536], 2, 128, 128, dtype="bf16", gdn=(kind == "gdn"), n_slots=4,
                            zero_init=False)
    pool_h = w.pool.copy()
    slot, spare, fresh = int(w.slot_idx[0]), *[s for s in range(4) if s != w.slot_idx[0]][:2]
    ck = np.array([[spare]], np.int32)
    _, pool = _run(kind, w, pool_h, ck, 512)          # saves the state after 512 tokens
    G.gla_state_copy(pool, dev(np.array([spare], np.int32)), dev(np.array([fresh], np.int32)))
    cut = 512
    cu2 = dev(np.array([0, 1536 - cut], np.int32))
    tail = lambda x: dev(x[cut:], w.dtype)  # noqa: E731
    if kind == "gla":
        o2 = G.gla_chunk_fwd(tail(w.q), tail(w.k), tail(w.v), dev(w.alpha[cut:]), cu2, pool,
                             dev(np.array([fresh], np.int32)), out_dtype=torch.float32)
        o_ref, _ = oracle.gla_sequence(w.q, w.k, w.v, w.alpha, S0=w.pool[slot])
    else:
        o2 = G.gdn_chunk_fwd(tail(w.q), tail(w.k), tail(w.v), dev(w.alpha[cut:]), dev(w.beta[cut:]),
                             cu2, pool, dev(np.array([fresh], np.int32)), out_dtype=torch.float32)
        o_ref, _ = oracle.gdn_sequence(w.q, w.k, w.v, w.alpha, w.beta, S0=w.pool[slot])
    torch.cuda.synchronize()
    check(host(o2), o_ref[cut:], "bf16", "o continued from the checkpoint copy")


@pytest.mark.parametrize("kind", ["gla", "gdn"])
def test_ckpt_full_size_every_block(kind):
    """Benchmark shapes with a checkpoint every 1024 tokens (GLA 4 x 4096, GDN
    2 x 8192, 16 heads): outputs and final states as without checkpoints
    (bitwise: the checkpoint stores do not change the arithmetic), and each
    saved state equals the final state of a prefill stopped there."""
    import gated_deltanet_gla_amd as G
    note(f"ckpt full size {kind}")
    w = synth.prefill_gla() if kind == "gla" else synth.prefill_gdn()
    B, iv = w.n_seqs, 1024
    stride = int(w.cu_seqlens[1]) // iv
    n0 = w.pool.shape[0]
    pool_h = np.concatenate([w.pool, np.zeros((B * stride,) + w.pool.shape[1:], np.float32)])
    ck = (n0 + np.arange(B * stride)).reshape(B, stride).astype(np.int32)
    o1, pool1 = _run(kind, w, pool_h, ck, iv, out_dtype="bf16")
    import gated_deltanet_gla_amd as G2  # noqa: F401
    q, k, v, a = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), dev(w.alpha)
    pool0 = dev(pool_h)
    if kind == "gla":
        o0 = G.gla_chunk_fwd(q, k, v, a, dev(w.cu_seqlens), pool0, dev(w.slot_idx), zero_init=True)
    else:
        o0 = G.gdn_chunk_fwd(q, k, v, a, dev(w.beta), dev(w.cu_seqlens), pool0, dev(w.slot_idx))
    torch.cuda.synchronize()
    assert torch.equal(o0, o1)
    assert torch.equal(pool0[:n0], pool1[:n0])
    # saved state j of sequence b == final state of the same prefill cut after (j+1)*iv tokens
    T = int(w.cu_seqlens[1])
    for j in (0, stride // 2, stride - 2):
        p = (j + 1) * iv
        idx = np.concatenate([np.arange(b * T, b * T + p) for b in range(B)])
        cu = dev((np.arange(B + 1) * p).astype(np.int32))
        pool2 = dev(w.pool)
        sub = lambda x, dt="f32": dev(x[idx], dt)  # noqa: E731
        if kind == "gla":
            G.gla_chunk_fwd(sub(w.q, "bf16"), sub(w.k, "bf16"), sub(w.v, "bf16"), sub(w.alpha), cu,
                            pool2, dev(w.slot_idx), zero_init=True)
        else:
            G.gdn_chunk_fwd(sub(w.q, "bf16"), sub(w.k, "bf16"), sub(w.v, "bf16"), sub(w.alpha),
                            sub(w.beta), cu, pool2, dev(w.slot_idx))
        torch.cuda.synchronize()
        for b in range(B):
            check(host(pool1[int(ck[b, j])]), host(pool2[int(w.slot_idx[b])]), "bf16",
                  f"checkpoint {j} of sequence {b}")


def test_gdn_ckpt_wide_columns():
    """Checkpoints from the 32-column serial workgroups (a batch with enough
    (sequence, head) pairs to select them)."""
    H, d, iv = 2, 128, 128
    rng = np.random.default_rng(140)
    lengths = rng.integers(100, 400, size=70).tolist()      # 70 x 2 heads x 8 tiles > 1024
    note("ckpt gdn wide columns")
    w = synth.random_varlen(141, lengths, H, d, d, dtype="bf16", gdn=True, chunk=64)
    stride = 3
    pool_h, ck = _ckpt_table(w, iv, stride, len(lengths) * stride + 3, seed=142)
    o, pool = _run("gdn", w, pool_h, ck, iv)
    o_ref, pool_ref = _oracle("gdn", w, pool_h, ck, iv)
    check(host(o), o_ref, "bf16", "o")
    p = host(pool)
    saved = sorted(set(int(x) for x in ck.ravel() if x >= 0) | set(w.slot_idx.tolist()))
    check(p[saved], pool_ref[saved], "bf16", "checkpoints and final states")
