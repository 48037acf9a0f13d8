"""ctypes view of the C ABI in include/gla.h.

Loads ``libgla_mi355x.so`` from this package directory.  There is no
fallback: if the library is missing or cannot be loaded, importing the
functions raises.
"""
from __future__ import annotations

import ctypes as ct
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgla_mi355x.so")

GLA_F32, GLA_BF16 = 0, 1
GLA_OK, GLA_EPTR, GLA_ESHAPE, GLA_EDTYPE, GLA_ECHUNK, GLA_EWORKSPACE, GLA_EHIP = 0, -1, -2, -3, -4, -5, -6
GLA_ESCRATCH = -7
GLA_NOALLOC_SCRATCH_BYTES = 64 << 20
GLA_ZERO_INIT = 1

# name -> (restype, argtypes); mirrors include/gla.h
_P, _F, _I32, _U32, _SZ = ct.c_void_p, ct.c_void_p, ct.c_int32, ct.c_uint32, ct.c_size_t
SIGNATURES = {
    "gla_chunk_fwd": (ct.c_int, [_P, _P, _P, _F, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                 ct.c_int, ct.c_int, _F, _I32, _P, _U32, _P, _P, _SZ, _P]),
    "gla_chunk_fwd_noalloc": (ct.c_int, [_P, _P, _P, _F, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                         ct.c_int, ct.c_int, _F, _I32, _P, _U32, _P, _P]),
    "gdn_chunk_fwd": (ct.c_int, [_P, _P, _P, _F, _F, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                 ct.c_int, ct.c_int, _F, _I32, _P, _U32, _P, _P, _SZ, _P]),
    "gla_chunk_fwd_ckpt": (ct.c_int, [_P, _P, _P, _F, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                      ct.c_int, ct.c_int, _F, _I32, _P, _U32, _I32, _P, _I32, _P,
                                      _P, _SZ, _P]),
    "gdn_chunk_fwd_ckpt": (ct.c_int, [_P, _P, _P, _F, _F, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                      ct.c_int, ct.c_int, _F, _I32, _P, _U32, _I32, _P, _I32, _P,
                                      _P, _SZ, _P]),
    "gdn_chunk_prep": (ct.c_int, [_P, _P, _F, _F, _P, _I32, _I32, _I32, _I32, _I32, _I32, ct.c_int,
                                  _P, _SZ, _P]),
    "gdn_chunk_run": (ct.c_int, [_P, _P, _P, _F, _F, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                 ct.c_int, ct.c_int, _F, _I32, _P, _U32, _P, _P, _SZ, _P]),
    "gla_chunk_workspace_bytes": (ct.c_size_t, [_I32] * 6),
    "gdn_chunk_workspace_bytes": (ct.c_size_t, [_I32] * 6),
    "gla_decode_step": (ct.c_int, [_P, _P, _P, _F, _I32, _I32, _I32, _I32, ct.c_int, ct.c_int,
                                   _F, _I32, _P, _P, _P]),
    "gdn_decode_step": (ct.c_int, [_P, _P, _P, _F, _F, _I32, _I32, _I32, _I32, ct.c_int,
                                   ct.c_int, _F, _I32, _P, _P, _P]),
    "gla_decode_multi": (ct.c_int, [_P, _P, _P, _F, _I32, _I32, _I32, _I32, _I32, ct.c_int,
                                    ct.c_int, _F, _I32, _P, _P, _P, _P]),
    "gdn_decode_multi": (ct.c_int, [_P, _P, _P, _F, _F, _I32, _I32, _I32, _I32, _I32, ct.c_int,
                                    ct.c_int, _F, _I32, _P, _P, _P, _P]),
    "gla_state_copy": (ct.c_int, [_F, _I32, _I32, _I32, _I32, _P, _P, _I32, _P]),
    "gla_slot_copy": (ct.c_int, [_P, _SZ, _I32, _P, _P, _I32, _P]),
    "gla_hbm_probe": (ct.c_int, [ct.c_int32, _F, _I32, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "lin_attn_chunk_fwd": (ct.c_int, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                      ct.c_int, ct.c_int, _F, _F, _I32, _P, _U32, ct.c_float, _P,
                                      _P, _SZ, _P]),
    "lin_attn_chunk_workspace_bytes": (ct.c_size_t, [_I32] * 6),
    "lin_attn_decode_step": (ct.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, ct.c_int, ct.c_int,
                                        _F, _F, _I32, _P, ct.c_float, _P, _P]),
    "causal_conv1d_fwd": (ct.c_int, [_P, _F, _P, _I32, _I32, _I32, _I32, _P, _I32, _P, _U32, _P,
                                     ct.c_int, _P]),
    "gla_status_string": (ct.c_char_p, [ct.c_int]),
    "gla_version": (ct.c_char_p, []),
}

_lib = None


class GlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status}: {status_string(status)}")
        self.status = status


def lib() -> ct.CDLL:
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m gated_deltanet_gla_amd.build")
        handle = ct.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().gla_status_string(int(status)).decode()


_fns: dict = {}


def call(name: str, *args) -> int:
    """Call an entry point; raise GlaError on a negative status."""
    f = _fns.get(name)
    if f is None:
        f = _fns[name] = getattr(lib(), name)
    st = f(*args)
    if st != GLA_OK:
        raise GlaError(name, st)
    return st
