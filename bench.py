#!/usr/bin/env python3
"""Benchmark of the gated linear-attention state recurrence on one MI355X.

Headline (``value``): chunked GLA prefill tokens/s on 4 sequences x 4096
tokens, 16 heads, d_k = d_v = 128, chunk 64, bf16 q/k/v/o, fp32 gates and
states, zero initial state (a token = one sequence position with all 16
heads).  One step = one ``gla_chunk_fwd`` over the whole batch with the
inputs resident in HBM.  The same JSON line also carries the decode-step
HBM GB/s (256 requests x 16 heads of 128x128 fp32 states in a 1024-slot
pool, GLA and Gated DeltaNet), the Gated DeltaNet prefill (2 x 8192 tokens)
and the mixed varlen Gated DeltaNet step (conv prelude + 48 prompts + 512
decodes), each timed the same way.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME]
Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "chunked prefill tokens/s + decode-step HBM GB/s, 128×128 fp32 state heads"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--only", default="all",
                   choices=["all", "gla_prefill", "gdn_prefill", "decode", "mixed", "lin_attn"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (HBM counter calibration)")
    p.add_argument("--cpu-baseline-child", action="store_true", help=argparse.SUPPRESS)
    p.add_argument("--sweep", action="store_true",
                   help="instead of the benchmark line: GLA / GDN prefill over batch x length mixes "
                        "and decode over batch sizes, one JSON line per shape")
    p.add_argument("--sweep-kind", default="all", choices=["all", "gla", "gdn", "decode"],
                   help="with --sweep: only the GLA prefills, the GDN prefills or the decodes")
    return p.parse_args()


# ---------------------------------------------------------------- CPU baseline
def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline_child():
    """The fp64 oracle, single-threaded on one pinned core, timed on each
    workload: the toy example, the GLA prefill (all 4 x 4096 tokens x 16
    heads), one GLA and one Gated DeltaNet decode step (256 requests x 16
    heads; the pool passed holds just the 256 slots the step touches, so
    the oracle does not copy the 768 others), the Gated DeltaNet prefill
    (all 2 x 8192 tokens x 16 heads) and the mixed step on heads 0 and 7 of
    every request (conv over those heads' channels, then the recurrence),
    scaled by 16 / 2 since heads are independent."""
    host = {"os_cpu_count": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
            "cpu_model": _cpu_model()}
    os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    import numpy as np
    import oracle
    import synth

    def clock(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    cfg = {}
    w = synth.page_toy_workload()
    dt = clock(lambda: oracle.gla_varlen(w.q, w.k, w.v, w.alpha, w.cu_seqlens, w.pool, w.slot_idx, True))
    cfg["toy"] = {"tokens_per_s": 64 / dt, "seconds": dt, "sample": "whole workload (T=64, d=16, 1 head)"}
    w = synth.prefill_gla()
    N = w.n_tokens
    dt = clock(lambda: oracle.gla_varlen(w.q, w.k, w.v, w.alpha, w.cu_seqlens, w.pool, w.slot_idx, True))
    cfg["gla_prefill"] = {"tokens_per_s": N / dt, "seconds": dt,
                          "sample": "whole workload (4 x 4096 tokens x 16 heads)"}
    for gdn in (False, True):
        w = synth.decode(seed=3, gdn=gdn)
        R = w.q.shape[0]
        sub = w.pool[w.slot_idx]
        ident = np.arange(R, dtype=np.int32)
        if gdn:
            f = lambda: oracle.gdn_decode(w.q, w.k, w.v, w.alpha, w.beta, sub, ident)  # noqa: E731
        else:
            f = lambda: oracle.gla_decode(w.q, w.k, w.v, w.alpha, sub, ident)  # noqa: E731
        dt = clock(f)
        nbytes = R * w.q.shape[1] * (2 * 128 * 128 * 4 + 4 * 128 * 2 + (8 if gdn else 4))
        cfg["gdn_decode" if gdn else "gla_decode"] = {
            "ms_per_step": dt * 1e3, "GBps": nbytes / dt / 1e9, "seconds": dt,
            "sample": "whole step (256 requests x 16 heads)"}
    w = synth.prefill_gdn()
    N = w.n_tokens
    dt = clock(lambda: oracle.gdn_varlen(w.q, w.k, w.v, w.alpha, w.beta, w.cu_seqlens, w.pool,
                                         w.slot_idx))
    cfg["gdn_prefill"] = {"tokens_per_s": N / dt, "seconds": dt,
                          "sample": "whole workload (2 x 8192 tokens x 16 heads)"}
    w = synth.mixed_varlen()
    heads, d = [0, 7], 128
    ch = np.concatenate([np.arange(h * d, (h + 1) * d) for h in heads])
    N = w.n_tokens

    def mixed():
        y, _ = oracle.causal_conv1d(w.extra["x"][:, ch], w.extra["w"][ch], w.cu_seqlens,
                                    w.extra["conv_cache"][:, :, ch], w.slot_idx)
        v = synth.round_bf16(y.astype(np.float32)).reshape(-1, len(heads), d)
        sl = w.slot_idx
        oracle.gdn_varlen(w.q[:, heads], w.k[:, heads], v, w.alpha[:, heads], w.beta[:, heads],
                          w.cu_seqlens, w.pool[sl][:, heads], np.arange(len(sl), dtype=np.int32))
    dt = clock(mixed)
    cfg["mixed_gdn_step"] = {"tokens_per_s": N / (dt * 16 / len(heads)), "seconds": dt,
                             "sample": f"heads 0 and 7 of all {N} tokens (conv over their 256 "
                                       f"channels, then the recurrence), time scaled by 8"}
    head = cfg["gla_prefill"]
    print(json.dumps({"value": head["tokens_per_s"], "unit": "tokens/s", "cores": 1, "kind": "oracle",
                      "sample": "GLA prefill, whole workload (4 x 4096 tokens x 16 heads), fp64 "
                                "token-by-token recurrence in numpy on 1 pinned core",
                      "seconds": sum(c["seconds"] for c in cfg.values()),
                      "host": host, "configs": cfg}))


def run_cpu_baseline():
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1",
               NUMEXPR_NUM_THREADS="1", HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    res = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-child"],
                         env=env, capture_output=True, text=True, timeout=900)
    if res.returncode != 0:
        raise RuntimeError(f"cpu baseline failed: {res.stderr[-2000:]}")
    return json.loads(res.stdout.strip().splitlines()[-1])


# ---------------------------------------------------------------- GPU timing
def timed(torch, fn, steps, warmup):
    """Run fn(i) warmup times, then time exactly `steps` calls between two
    HIP events on the current stream (synchronised on both sides)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(steps):
        fn(warmup + i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps   # ms per call


def per_call_ms(torch, fn, n, offset=0):
    """Each of n calls between its own pair of HIP events on the current
    stream (after the timed region): median, p10 and p90 in ms."""
    import numpy as np
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(offset + i)
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return {"p10": float(np.percentile(t, 10)), "median": float(np.median(t)),
            "p90": float(np.percentile(t, 90)), "calls": n}


def bench_gla_prefill(torch, G, synth, dev, steps, warmup):
    w = synth.prefill_gla()
    N, H, d = w.n_tokens, w.n_heads, w.dk
    sets = []
    for r in range(2):   # two resident copies, alternated: the working set exceeds the MALL
        sets.append((dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), dev(w.alpha)))
    cu, slots = dev(w.cu_seqlens), dev(w.slot_idx)
    pool = dev(w.pool)
    o = torch.empty((N, H, d), dtype=torch.bfloat16, device="cuda:0")
    ws = torch.empty(max(1, G.workspace_bytes("gla", w.n_seqs, N, H, d, d, w.chunk)),
                     dtype=torch.uint8, device="cuda:0")

    def step(i):
        q, k, v, a = sets[i % 2]
        G.gla_chunk_fwd(q, k, v, a, cu, pool, slots, chunk=w.chunk, zero_init=True, o=o,
                        workspace=ws)
    ms = timed(torch, step, steps, warmup)
    dist = per_call_ms(torch, step, max(steps, 20), warmup + steps)
    nbytes = (3 * N * H * d * 2) + N * H * 4 + N * H * d * 2 + w.n_seqs * H * d * d * 4
    flops = N * H * (2 * w.chunk * (2 * d) + 4 * d * d)
    return {"workload": w.name, "ms": ms, "tokens_per_s": N / (ms * 1e-3), "bytes": nbytes,
            "flops": flops, "n_tokens": N, "batch": w.n_seqs, "seq_len": N // w.n_seqs, "heads": H,
            "d": d, "chunk": w.chunk, "per_call_ms": dist}


def bench_gdn_prefill(torch, G, synth, dev, steps, warmup):
    w = synth.prefill_gdn()
    N, H, d = w.n_tokens, w.n_heads, w.dk
    sets = [(dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), dev(w.alpha), dev(w.beta))
            for _ in range(2)]
    cu, slots = dev(w.cu_seqlens), dev(w.slot_idx)
    pool = dev(w.pool)
    o = torch.empty((N, H, d), dtype=torch.bfloat16, device="cuda:0")
    ws = torch.empty(G.workspace_bytes("gdn", w.n_seqs, N, H, d, d, w.chunk), dtype=torch.uint8,
                     device="cuda:0")

    def step(i):
        q, k, v, a, b = sets[i % 2]
        G.gdn_chunk_fwd(q, k, v, a, b, cu, pool, slots, chunk=w.chunk, o=o, workspace=ws)
    ms = timed(torch, step, steps, warmup)
    dist = per_call_ms(torch, step, max(steps, 20), warmup + steps)
    nbytes = 3 * N * H * d * 2 + 2 * N * H * 4 + N * H * d * 2 + 2 * w.n_seqs * H * d * d * 4
    C = w.chunk
    flops = N * H * (2 * C * (3 * d + 2 * d) + C * C // 3 + 6 * d * d)
    return {"workload": w.name, "ms": ms, "tokens_per_s": N / (ms * 1e-3), "bytes": nbytes,
            "flops": flops, "per_call_ms": dist}


def bench_decode(torch, G, synth, dev, steps, warmup, gdn):
    w = synth.decode(seed=3, gdn=gdn)
    R, H, d = w.q.shape
    q, k, v, a = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), dev(w.alpha)
    b = dev(w.beta) if gdn else None
    pool = dev(w.pool)
    perm = w.extra["perm"]
    quarters = [dev(perm[i * R:(i + 1) * R].copy()) for i in range(len(perm) // R)]
    o = torch.empty((R, H, d), dtype=torch.bfloat16, device="cuda:0")

    def step(i):
        sl = quarters[i % len(quarters)]   # disjoint slot sets: no MALL reuse between steps
        if gdn:
            G.gdn_decode_step(q, k, v, a, b, pool, sl, o=o)
        else:
            G.gla_decode_step(q, k, v, a, pool, sl, o=o)
    ms = timed(torch, step, steps, warmup)
    dist = per_call_ms(torch, step, max(steps, 20), warmup + steps)
    nbytes = R * H * (2 * d * d * 4 + 4 * d * 2 + (8 if gdn else 4))
    return {"workload": w.name, "ms": ms, "GBps": nbytes / (ms * 1e-3) / 1e9, "bytes": nbytes,
            "per_call_ms": dist}


def bench_decode_multi(torch, G, synth, dev, steps, warmup, gdn):
    """Speculative-decoding verification: 256 requests x 4 draft tokens x 16
    heads, the state after every position kept in its own slot (1280-slot
    pool); one read and four writes of each 64 KiB head state per call."""
    w = synth.decode_multi(seed=6, n_req=256, n_tok=4, n_slots=1280, gdn=gdn)
    R, J, H, d = w.q.shape
    q, k, v, a = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), dev(w.alpha)
    b = dev(w.beta) if gdn else None
    pool = dev(w.pool)
    slots, pos = dev(w.slot_idx), dev(w.extra["pos_slots"])
    o = torch.empty((R, J, H, d), dtype=torch.bfloat16, device="cuda:0")

    def step(i):
        if gdn:
            G.gdn_decode_multi(q, k, v, a, b, pool, slots, pos, o=o)
        else:
            G.gla_decode_multi(q, k, v, a, pool, slots, pos, o=o)
    ms = timed(torch, step, steps, warmup)
    dist = per_call_ms(torch, step, max(steps, 20), warmup + steps)
    nbytes = R * H * ((1 + J) * d * d * 4 + J * (4 * d * 2 + (8 if gdn else 4)))
    # replay strategy: verify with no state kept, then commit a random
    # accepted prefix (0..4 tokens) in place by running the draft again
    import numpy as np
    none = dev(np.full((R, J), -1, np.int32))
    acc = np.random.default_rng(7).integers(0, J + 1, size=R)
    cpos = np.full((R, J), -1, np.int32)
    for r in range(R):
        if acc[r] > 0:
            cpos[r, acc[r] - 1] = w.slot_idx[r]
    cpos = dev(cpos)

    def replay(i):
        for pos_ in (none, cpos):
            if gdn:
                G.gdn_decode_multi(q, k, v, a, b, pool, slots, pos_, o=o)
            else:
                G.gla_decode_multi(q, k, v, a, pool, slots, pos_, o=o)
    ms_r = timed(torch, replay, steps, warmup)
    return {"workload": w.name, "ms": ms, "GBps": nbytes / (ms * 1e-3) / 1e9, "bytes": nbytes,
            "replay_ms": ms_r, "per_call_ms": dist}


def bench_gdn_prefill_ckpt(torch, G, synth, dev, steps, warmup):
    """The Gated DeltaNet prefill saving a state checkpoint every 1024 tokens
    (8 per sequence, 16 MiB of extra state writes per call)."""
    import numpy as np
    w = synth.prefill_gdn()
    N, H, d = w.n_tokens, w.n_heads, w.dk
    B, iv = w.n_seqs, 1024
    stride = int(w.cu_seqlens[1]) // iv
    n0 = w.pool.shape[0]
    pool = dev(np.concatenate([w.pool, np.zeros((B * stride,) + w.pool.shape[1:], np.float32)]))
    ck = dev((n0 + np.arange(B * stride)).reshape(B, stride).astype(np.int32))
    q, k, v, a, b = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), dev(w.alpha), dev(w.beta)
    cu, slots = dev(w.cu_seqlens), dev(w.slot_idx)
    o = torch.empty((N, H, d), dtype=torch.bfloat16, device="cuda:0")
    ws = torch.empty(G.workspace_bytes("gdn", B, N, H, d, d, w.chunk), dtype=torch.uint8,
                     device="cuda:0")
    def step(i):
        G.gdn_chunk_fwd_ckpt(q, k, v, a, b, cu, pool, slots, ck, iv, chunk=w.chunk, o=o, workspace=ws)
    ms = timed(torch, step, steps, warmup)
    dist = per_call_ms(torch, step, max(steps, 20), warmup + steps)
    return {"workload": w.name + f"-ckpt{iv}", "ms": ms, "tokens_per_s": N / (ms * 1e-3),
            "per_call_ms": dist}


def bench_lin_attn(torch, G, synth, dev, steps, warmup):
    """Normalised linear attention (phi = elu + 1): prefill of 4 x 4096
    tokens x 16 heads (d = 128, chunk 64, bf16, from pool states), and one
    decode step of 256 requests x 16 heads."""
    w = synth.lin_attn_varlen(640, [4096] * 4, 16, 128, 128, dtype="bf16", chunk=64)
    N, H, d = w.n_tokens, w.n_heads, w.dk
    q, k, v = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16")
    pool, zpool = dev(w.pool), dev(w.extra["zpool"])
    cu, slots = dev(w.cu_seqlens), dev(w.slot_idx)
    o = torch.empty((N, H, d), dtype=torch.bfloat16, device="cuda:0")
    ws = torch.empty(G.workspace_bytes("lin", w.n_seqs, N, H, d, d, 64), dtype=torch.uint8,
                     device="cuda:0")
    def pstep(i):
        G.lin_attn_chunk_fwd(q, k, v, cu, pool, zpool, slots, chunk=64, o=o, workspace=ws)
    ms = timed(torch, pstep, steps, warmup)
    pdist = per_call_ms(torch, pstep, max(steps, 20), warmup + steps)
    nbytes = 4 * N * H * d * 2 + 4 * H * (2 * d * d * 4 + 2 * d * 4)
    R = 256
    wd = synth.lin_attn_varlen(641, [1] * R, 16, 128, 128, dtype="bf16", n_slots=1024)
    qd, kd, vd = dev(wd.q, "bf16"), dev(wd.k, "bf16"), dev(wd.v, "bf16")
    pd, zd, sd = dev(wd.pool), dev(wd.extra["zpool"]), dev(wd.slot_idx)
    od = torch.empty((R, H, d), dtype=torch.bfloat16, device="cuda:0")
    def dstep(i):
        G.lin_attn_decode_step(qd, kd, vd, pd, zd, sd, o=od)
    msd = timed(torch, dstep, steps, warmup)
    ddist = per_call_ms(torch, dstep, max(steps, 20), warmup + steps)
    dbytes = R * H * (2 * d * d * 4 + 2 * d * 4 + 4 * d * 2)
    return {"prefill": {"workload": "lin-attn-prefill-4x4096-H16-d128-C64-bf16", "ms": ms,
                        "tokens_per_s": N / (ms * 1e-3),
                        "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, "per_call_ms": pdist},
            "decode": {"workload": "lin-attn-decode-256req-H16-d128-pool1024", "ms": msd,
                       "GBps": dbytes / (msd * 1e-3) / 1e9,
                       "hbm_frac": dbytes / (msd * 1e-3) / 1e9 / HBM_PEAK_GBPS, "per_call_ms": ddist}}


def bench_slot_copy(torch, G, synth, dev, steps, warmup):
    """Whole-slot copies (prefix-cache copy-on-write, committing a draft
    position): 256 pairs of 1 MiB state slots (16 heads x 128 x 128 fp32)
    in a 1024-slot pool; one read and one write of each slot."""
    import numpy as np
    pool = torch.randn((1024, 16, 128, 128), device="cuda:0") * 0.05
    perm = np.random.default_rng(9).permutation(1024).astype(np.int32)
    pairs = [(dev(perm[512 * r:512 * r + 256].copy()), dev(perm[512 * r + 256:512 * r + 512].copy()))
             for r in range(2)]
    def step(i):
        G.gla_state_copy(pool, *pairs[i % 2])
    ms = timed(torch, step, steps, warmup)
    dist = per_call_ms(torch, step, max(steps, 20), warmup + steps)
    nbytes = 2 * 256 * 16 * 128 * 128 * 4
    return {"workload": "256 slot pairs x 1 MiB, 1024-slot pool", "ms": ms,
            "GBps": nbytes / (ms * 1e-3) / 1e9, "per_call_ms": dist}


def bench_hbm_ceiling(torch, G, synth, dev, steps, warmup):
    """The decode step's HBM footprint without its arithmetic
    (gla_hbm_probe): 256 requests x 16 heads of 64 KiB state blocks in a
    1024-slot pool, the 4 disjoint slot quarters rotated as in the decode
    leg.  Read only, write only, read + write back in place, and read +
    write with two heads per workgroup, each with nontemporal ("nt") or
    default-policy ("def") loads and stores; the best of each is the
    ceiling."""
    w = synth.decode(seed=3, gdn=False)
    R, H, d = w.q.shape
    pool = dev(w.pool)
    perm = w.extra["perm"]
    quarters = [dev(perm[i * R:(i + 1) * R].copy()) for i in range(len(perm) // R)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    block = R * H * d * d * 4
    out = {"workload": "256 requests x 16 heads x 64 KiB, 1024-slot pool, slot quarters rotated",
           "variants": {}}
    ops = ((0, "read", block), (1, "write", block), (2, "read_write", 2 * block),
           (3, "read_write_2heads_per_wg", 2 * block))
    for op, name, nb in ops:
        pols = [(0, "nt")] if op == 1 else [(0, "nt"), (4, "def")]
        if op != 0:
            pols = [(p | s, f"{ln}_load/{sn}_store" if op >= 2 else f"{sn}_store")
                    for p, ln in pols for s, sn in ((0, "nt"), (8, "def"))]
        else:
            pols = [(p, f"{ln}_load") for p, ln in pols]
        best = None
        for pol, pname in pols:
            def step(i, mode=op | pol):
                G.gla_hbm_probe(mode, pool, quarters[i % len(quarters)], sink)
            ms = timed(torch, step, steps, warmup)
            rec = {"GBps": nb / (ms * 1e-3) / 1e9, "ms": ms,
                   "per_call_ms": per_call_ms(torch, step, max(steps, 20), warmup + steps)}
            out["variants"][f"{name} {pname}"] = rec
            if best is None or rec["GBps"] > best["GBps"]:
                best = dict(rec, policy=pname)
        out[name] = best
    return out


def bench_mixed(torch, G, synth, dev, steps, warmup):
    import numpy as np
    from gated_deltanet_gla_amd.step import MixedStep
    w = synth.mixed_varlen()
    x = w.extra["x"]
    P, D = w.extra["n_prefill"], w.extra["n_decode"]
    lens = w.extra["lengths"]
    NP = int(lens[:P].sum())
    N, H, d = w.q.shape
    cu_p = np.concatenate([[0], np.cumsum(lens[:P])]).astype(np.int32)
    step_obj = MixedStep(dev(x, "bf16"), dev(w.extra["w"]), dev(w.extra["conv_cache"], "bf16"),
                         dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.alpha), dev(w.beta),
                         dev(w.cu_seqlens), dev(cu_p), dev(w.pool), dev(w.slot_idx), P, NP)
    ms = timed(torch, lambda i: step_obj(), steps, warmup)
    dist = per_call_ms(torch, lambda i: step_obj(), max(steps, 5), warmup + steps)
    nbytes = (N * H * d * 2 * 3 + N * H * 8            # q, k, o; alpha, beta
              + N * H * d * 2 * 2                       # conv x in, y out (= v)
              + N * H * d * 2                           # v read by the recurrence
              + len(lens) * H * d * d * 4 * 2           # state read + write
              + len(lens) * 3 * H * d * 2 * 2)          # conv cache read + write
    return {"workload": w.name, "ms": ms, "tokens_per_s": N / (ms * 1e-3), "n_tokens": N,
            "prefill_tokens": NP, "longest_prompt": int(lens[:P].max()), "bytes": nbytes,
            "GBps": nbytes / (ms * 1e-3) / 1e9, "per_call_ms": dist}


def _profile_entry(kernel: str):
    """The rocprofv3 counter entry of a call (profiles/traffic.json), or None
    when the kernel's sources changed since the counters were taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            tab = json.load(f)
        ent = tab[kernel]
        m = hashlib.sha256()
        for src in ent["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                m.update(f.read())
        return ent if m.hexdigest() == ent["sha256"] else None
    except (OSError, KeyError, ValueError):
        return None


def measured_traffic(kernel: str):
    """HBM bytes per call measured with rocprofv3 (FETCH_SIZE + WRITE_SIZE)."""
    ent = _profile_entry(kernel)
    return None if ent is None else ent["fetch_bytes"] + ent["write_bytes"]


def measured_mfma(kernel: str):
    """rocprofv3 MfmaUtil per kernel (% of SIMD cycles with the MFMA unit
    busy) and the MFMA flops the call executes (SQ_INSTS_VALU_MFMA_MOPS_*)."""
    ent = _profile_entry(kernel)
    return None if ent is None else ent.get("mfma")


def run_sweep(torch, G, steps, warmup, kind="all"):
    """Prefill over batch x length mixes of about the same token count (and
    two larger ones), decode over batch sizes.  Inputs are drawn on the
    device with the benchmark's distributions (GLA q, k ~ N(0,1)/sqrt(d);
    GDN q, k L2-normalised; v ~ N(0,1); alpha = sigmoid(N(0,1)+3); beta =
    sigmoid(N(0,1))); prefills start from zero states; decode rotates over
    disjoint slot sets of a 2048-slot pool."""
    import math
    H, d, C = 16, 128, 64
    gen = torch.Generator(device="cuda:0").manual_seed(5)

    def rn(*shape):
        return torch.randn(*shape, device="cuda:0", generator=gen)

    def qk(n, gdn):
        if gdn:
            return torch.nn.functional.normalize(rn(n, H, d), dim=-1).bfloat16()
        return (rn(n, H, d) / math.sqrt(d)).bfloat16()

    for gdn in [g for g, name in ((False, "gla"), (True, "gdn")) if kind in ("all", name)]:
        for B, T in ((1, 16384), (2, 8192), (4, 4096), (16, 1024), (64, 256), (256, 64), (8, 8192),
                     (1, 65536)):
            N = B * T
            sets = [(qk(N, gdn), qk(N, gdn), rn(N, H, d).bfloat16(), torch.sigmoid(rn(N, H) + 3),
                     torch.sigmoid(rn(N, H))) for _ in range(2)]
            cu = torch.arange(0, N + 1, T, dtype=torch.int32, device="cuda:0")
            slots = torch.arange(B, dtype=torch.int32, device="cuda:0")
            pool = torch.zeros((B, H, d, d), device="cuda:0")
            o = torch.empty((N, H, d), dtype=torch.bfloat16, device="cuda:0")
            ws = torch.empty(max(1, G.workspace_bytes("gdn" if gdn else "gla", B, N, H, d, d, C)),
                             dtype=torch.uint8, device="cuda:0")

            def step(i):
                q, k, v, a, b = sets[i % 2]
                if gdn:
                    G.gdn_chunk_fwd(q, k, v, a, b, cu, pool, slots, chunk=C, zero_init=True, o=o,
                                    workspace=ws)
                else:
                    G.gla_chunk_fwd(q, k, v, a, cu, pool, slots, chunk=C, zero_init=True, o=o,
                                    workspace=ws)
            ms = timed(torch, step, steps, warmup)
            print(json.dumps({"sweep": "gdn_prefill" if gdn else "gla_prefill", "batch": B, "seq_len": T,
                              "ms": ms, "tokens_per_s": N / (ms * 1e-3)}), flush=True)
            del sets, o, ws, pool
    if kind not in ("all", "decode"):
        return
    n_slots = 2048
    pool = rn(n_slots, H, d, d) * 0.05
    perm = torch.randperm(n_slots, device="cuda:0", generator=gen).to(torch.int32)
    for gdn in (False, True):
        for R in (1, 8, 32, 64, 128, 256, 512, 1024):
            q, k, v = (rn(R, H, d) / math.sqrt(d)).bfloat16(), qk(R, gdn), rn(R, H, d).bfloat16()
            a, b = torch.sigmoid(rn(R, H) + 3), torch.sigmoid(rn(R, H))
            nsets = min(8, n_slots // R)
            sl = [perm[i * R:(i + 1) * R].contiguous() for i in range(nsets)]
            o = torch.empty((R, H, d), dtype=torch.bfloat16, device="cuda:0")

            def step(i):
                if gdn:
                    G.gdn_decode_step(q, k, v, a, b, pool, sl[i % nsets], o=o)
                else:
                    G.gla_decode_step(q, k, v, a, pool, sl[i % nsets], o=o)
            ms = timed(torch, step, steps, warmup)
            nbytes = R * H * (2 * d * d * 4 + 4 * d * 2 + (8 if gdn else 4))
            rec = {"sweep": "gdn_decode" if gdn else "gla_decode", "requests": R, "ms": ms,
                   "GBps": nbytes / (ms * 1e-3) / 1e9}
            if R <= 32:
                # the same calls replayed from a HIP graph: no host work per call
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(20):
                        step(i)
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                for _ in range(10):
                    g.replay()
                e.record()
                torch.cuda.synchronize()
                rec["graph_ms"] = s.elapsed_time(e) / 200
            print(json.dumps(rec), flush=True)


def calib_copy(torch):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    a.fill_(1)
    torch.cuda.synchronize()
    ms = timed(torch, lambda i: b.copy_(a), 5, 2)
    return {"bytes_each_way": n, "ms": ms, "GBps": 2 * n / (ms * 1e-3) / 1e9}


def main():
    args = parse()
    if args.cpu_baseline_child:
        cpu_baseline_child()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(every (sequence, head) is independent, so N GPUs would each run this workload "
              f"on their own share)", file=sys.stderr)
        sys.exit(2)

    cpu = None
    if not args.no_cpu_baseline and not args.sweep and args.only in ("all", "gla_prefill"):
        cpu = run_cpu_baseline()      # before this process touches the GPU

    import torch
    import gated_deltanet_gla_amd as G
    import synth
    from gated_deltanet_gla_amd import _lib
    _lib.lib()   # fail loudly if the HIP library is missing
    if args.sweep:
        run_sweep(torch, G, max(args.steps, 30), args.warmup, args.sweep_kind)
        return

    def dev(x, dtype="f32"):
        import numpy as np
        if dtype == "bf16":
            bits = synth.bf16_bits(np.asarray(x, np.float32)).view(np.int16)
            return torch.from_numpy(bits.copy()).to("cuda:0").view(torch.bfloat16)
        if x.dtype in (np.int32, np.int64):
            return torch.from_numpy(np.ascontiguousarray(x.astype(np.int32))).to("cuda:0")
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")

    res = {}
    K, W = args.steps, args.warmup
    if args.only in ("all", "gla_prefill"):
        res["gla_prefill"] = bench_gla_prefill(torch, G, synth, dev, K, W)
        print(f"# gla prefill {res['gla_prefill']['ms']:.3f} ms", file=sys.stderr, flush=True)
    if args.only in ("all", "decode"):
        res["gla_decode"] = bench_decode(torch, G, synth, dev, K, W, gdn=False)
        res["gdn_decode"] = bench_decode(torch, G, synth, dev, K, W, gdn=True)
        print(f"# decode {res['gla_decode']['ms']:.3f} / {res['gdn_decode']['ms']:.3f} ms",
              file=sys.stderr, flush=True)
        res["slot_copy"] = bench_slot_copy(torch, G, synth, dev, K, W)
        res["hbm_ceiling"] = bench_hbm_ceiling(torch, G, synth, dev, K, W)
        print(f"# ceiling read {res['hbm_ceiling']['read']['GBps']:.0f} write "
              f"{res['hbm_ceiling']['write']['GBps']:.0f} read+write "
              f"{res['hbm_ceiling']['read_write']['GBps']:.0f} GB/s", file=sys.stderr, flush=True)
        res["gla_decode_multi"] = bench_decode_multi(torch, G, synth, dev, K, W, gdn=False)
        res["gdn_decode_multi"] = bench_decode_multi(torch, G, synth, dev, K, W, gdn=True)
        print(f"# decode multi {res['gla_decode_multi']['ms']:.3f} / "
              f"{res['gdn_decode_multi']['ms']:.3f} ms", file=sys.stderr, flush=True)
    if args.only in ("all", "gdn_prefill"):
        res["gdn_prefill"] = bench_gdn_prefill(torch, G, synth, dev, K, W)
        print(f"# gdn prefill {res['gdn_prefill']['ms']:.3f} ms", file=sys.stderr, flush=True)
        res["gdn_prefill_ckpt"] = bench_gdn_prefill_ckpt(torch, G, synth, dev, K, W)
        print(f"# gdn prefill + checkpoints {res['gdn_prefill_ckpt']['ms']:.3f} ms", file=sys.stderr,
              flush=True)
    if args.only in ("all", "lin_attn"):
        res["lin_attn"] = bench_lin_attn(torch, G, synth, dev, K, W)
        print(f"# lin attn prefill {res['lin_attn']['prefill']['ms']:.3f} ms, decode "
              f"{res['lin_attn']['decode']['ms']:.3f} ms", file=sys.stderr, flush=True)
    if args.only in ("all", "mixed"):
        res["mixed"] = bench_mixed(torch, G, synth, dev, max(3, K // 4), max(1, W // 2))
        print(f"# mixed {res['mixed']['ms']:.3f} ms", file=sys.stderr, flush=True)
    if args.calib_copy:
        res["copy"] = calib_copy(torch)

    head = res.get("gla_prefill")
    out = {"metric": METRIC, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic"}
    if head:
        ach = head["bytes"] / (head["ms"] * 1e-3) / 1e9
        out.update({
            "value": head["tokens_per_s"], "ms_per_step": head["ms"],
            "config": {"workload": head["workload"], "global_batch": head["batch"],
                       "seq_len": head["seq_len"], "heads": head["heads"], "dk": head["d"],
                       "dv": head["d"], "chunk": head["chunk"], "state": "fp32",
                       "io": "bf16 q/k/v/o, fp32 alpha"},
            # one gla_chunk_fwd call = two dependent launches (gla_seg_state,
            # then gla_seg_out); both are timed together by the events around
            # the call, and the traffic is the sum of their counters
            "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": ach / HBM_PEAK_GBPS, "traffic": measured_traffic("gla_chunk_fwd"),
                         "kernel": "gla_chunk_fwd (gla_seg_state + gla_seg_out)",
                         "algorithmic_bytes": head["bytes"],
                         "mfma_frac": head["flops"] / (head["ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                         "mfma_counters": measured_mfma("gla_chunk_fwd")},
            "per_call_ms": head["per_call_ms"],
        })
    else:
        out.update({"value": None, "ms_per_step": None, "config": {"workload": args.only}})
    if "gla_decode" in res:
        r = res["gla_decode"]
        out["roofline_decode"] = {"bound": "hbm", "achieved": r["GBps"], "peak": HBM_PEAK_GBPS,
                                  "unit": "GB/s", "frac": r["GBps"] / HBM_PEAK_GBPS,
                                  "traffic": measured_traffic("decode_kernel_gla"),
                                  "kernel": "decode_kernel (GLA)", "algorithmic_bytes": r["bytes"]}
        if "hbm_ceiling" in res:
            c = res["hbm_ceiling"]
            best = max(c["read_write"]["GBps"], c["read_write_2heads_per_wg"]["GBps"])
            out["roofline_decode"]["measured_ceiling"] = {
                "read_GBps": c["read"]["GBps"], "write_GBps": c["write"]["GBps"],
                "read_write_GBps": c["read_write"]["GBps"],
                "read_write_2heads_per_wg_GBps": c["read_write_2heads_per_wg"]["GBps"],
                "frac_of_read_write": r["GBps"] / best,
                "variants_GBps": {k: v["GBps"] for k, v in c["variants"].items()},
                "workload": c["workload"], "per_call_ms": {k: c[k]["per_call_ms"] for k in
                                                           ("read", "write", "read_write",
                                                            "read_write_2heads_per_wg")}}
        out["decode_hbm_GBps"] = {
            "gla": res["gla_decode"]["GBps"], "gdn": res["gdn_decode"]["GBps"],
            "frac_of_peak": {"gla": res["gla_decode"]["GBps"] / HBM_PEAK_GBPS,
                             "gdn": res["gdn_decode"]["GBps"] / HBM_PEAK_GBPS},
            "ms": {"gla": res["gla_decode"]["ms"], "gdn": res["gdn_decode"]["ms"]},
            "per_call_ms": {"gla": res["gla_decode"]["per_call_ms"],
                            "gdn": res["gdn_decode"]["per_call_ms"]},
            "workload": "256 requests x 16 heads, 128x128 fp32 states, 1024-slot pool, in place"}
    if "slot_copy" in res:
        r = res["slot_copy"]
        out["slot_copy_hbm_GBps"] = {"GBps": r["GBps"], "ms": r["ms"],
                                     "frac_of_peak": r["GBps"] / HBM_PEAK_GBPS,
                                     "workload": r["workload"], "per_call_ms": r["per_call_ms"]}
    if "gla_decode_multi" in res:
        out["decode_multi_hbm_GBps"] = {
            k: res[f"{k}_decode_multi"]["GBps"] for k in ("gla", "gdn")}
        out["decode_multi_hbm_GBps"].update({
            "frac_of_peak": {k: res[f"{k}_decode_multi"]["GBps"] / HBM_PEAK_GBPS
                             for k in ("gla", "gdn")},
            "ms": {k: res[f"{k}_decode_multi"]["ms"] for k in ("gla", "gdn")},
            "replay_strategy_ms": {k: res[f"{k}_decode_multi"]["replay_ms"] for k in ("gla", "gdn")},
            "per_call_ms": {k: res[f"{k}_decode_multi"]["per_call_ms"] for k in ("gla", "gdn")},
            "workload": "256 requests x 4 draft tokens x 16 heads, 128x128 fp32 states, state "
                        "after every position kept (1280-slot pool)"})
    other = {}
    if "gdn_prefill" in res:
        r = res["gdn_prefill"]
        ach = r["bytes"] / (r["ms"] * 1e-3) / 1e9
        other["gdn_prefill"] = {"workload": r["workload"], "tokens_per_s": r["tokens_per_s"],
                                "ms": r["ms"], "hbm_frac": ach / HBM_PEAK_GBPS,
                                "mfma_frac": r["flops"] / (r["ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                                "traffic": measured_traffic("gdn_chunk_fwd"),
                                "mfma_counters": measured_mfma("gdn_chunk_fwd"),
                                "per_call_ms": r["per_call_ms"]}
    if "gdn_prefill_ckpt" in res:
        r = res["gdn_prefill_ckpt"]
        other["gdn_prefill_ckpt"] = {k: r[k] for k in ("workload", "ms", "tokens_per_s", "per_call_ms")}
    if "lin_attn" in res:
        other["lin_attn_prefill"] = res["lin_attn"]["prefill"]
        other["lin_attn_decode"] = res["lin_attn"]["decode"]
    if "mixed" in res:
        r = res["mixed"]
        other["mixed_gdn_step"] = {k: r[k] for k in ("workload", "ms", "tokens_per_s", "n_tokens",
                                                     "prefill_tokens", "longest_prompt", "GBps",
                                                     "per_call_ms")}
        other["mixed_gdn_step"]["hbm_frac"] = r["GBps"] / HBM_PEAK_GBPS
        other["mixed_gdn_step"]["traffic"] = measured_traffic("mixed_gdn_step")
    if other:
        out["other_workloads"] = other
    if "copy" in res:
        out["copy_calibration"] = res["copy"]
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out))


if __name__ == "__main__":
    main()
