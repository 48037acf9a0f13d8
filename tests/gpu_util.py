"""Helpers for the GPU parity tests: move synthetic workloads to the device
and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth

DEV = "cuda:0"


def note(msg: str):
    """Name the case on stdout before a GPU step (flushed)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(x: np.ndarray) -> torch.Tensor:
    """fp32 array holding exact bf16 values -> bf16 device tensor (same values)."""
    bits = synth.bf16_bits(x).view(np.int16)
    return torch.from_numpy(bits.copy()).to(DEV).view(torch.bfloat16)


def dev(x: np.ndarray, dtype: str = "f32") -> torch.Tensor:
    if dtype == "bf16":
        return dev_bf16(np.asarray(x, np.float32))
    if x.dtype == np.int32 or x.dtype == np.int64:
        return torch.from_numpy(np.ascontiguousarray(x.astype(np.int32))).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(x, ref) -> float:
    """max_i |x_i - r_i| / max_i |r_i| over one tensor."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(x - ref).max() / (den if den > 0 else 1.0))


def abs_err(x, ref) -> float:
    return float(np.abs(np.asarray(x, np.float64) - np.asarray(ref, np.float64)).max())


def rne_bf16(t: torch.Tensor) -> torch.Tensor:
    """torch's fp32 -> bf16 cast (round to nearest even), as an independent check."""
    return t.float().cpu().to(torch.bfloat16)


# tolerances: fp32 inputs -> 1e-5 absolute; bf16 inputs (fp32 accumulate) ->
# 3e-3 max relative error, gated on fp32 outputs and fp32 final states.
TOL_F32_ABS = 1e-5
TOL_BF16_REL = 3e-3


def check(x, ref, dtype, what):
    if dtype == "f32":
        e = abs_err(x, ref)
        assert e <= TOL_F32_ABS, f"{what}: abs err {e:.3e} > {TOL_F32_ABS}"
    else:
        e = rel_err(x, ref)
        assert e <= TOL_BF16_REL, f"{what}: rel err {e:.3e} > {TOL_BF16_REL}"
    return e


def check_bf16_storage(x, ref, what, slack=1e-5):
    """A bf16-stored result must be within one bf16 rounding of the exact
    value: |x - r| <= 2^-8 |r| elementwise (bf16 keeps 8 significant bits, so
    round-to-nearest moves a value by at most half an ulp = 2^-8 relative to
    the bottom of its binade), plus a small slack for fp32 arithmetic."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    excess = np.abs(x - ref) - 2.0 ** -8 * np.abs(ref)
    worst = float(excess.max() / max(np.abs(ref).max(), 1e-30))
    assert worst <= slack, f"{what}: exceeds one bf16 rounding by {worst:.3e} (relative to max)"
    return worst
