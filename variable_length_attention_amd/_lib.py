"""ctypes binding of libhdpattn.so (argument marshalling only; every step runs in the library).

There is no fallback: if the library is missing or fails to load, importing the ops raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# HDP_LIB_PATH selects another build of the same library (the sanitizer build of the host layer)
LIB_PATH = os.environ.get("HDP_LIB_PATH") or os.path.join(_PKG, "libhdpattn.so")

HDP_OK = 0
HDP_ERR_INVALID_ARG = 1
HDP_ERR_UNSUPPORTED = 2
HDP_ERR_HIP = 3
HDP_ERR_OVERFLOW = 4
HDP_ERR_SCRATCH_LIMIT = 5
NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024

# (name, restype, argtypes) for every symbol include/hdp_attn.h declares.
P, I32, I64, F32, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_uint64
SIGNATURES = {
    "hdp_attn_varlen_fwd": (I32, [P, P, P, P, I32, I32, I32, I32, F32, P, P, P]),
    "hdp_attn_varlen_fwd_f32": (I32, [P, P, P, P, I32, I32, I32, I32, F32, P, P, P]),
    "hdp_attn_chunk_partial": (I32, [P, I32, P, P, I32, I64, I64, I32, I32, I32, I32, F32, P, P, P]),
    "hdp_attn_chunk_merge": (I32, [P, I32, P, P, I32, I64, I64, I32, I32, I32, I32, F32, P, P, P, P]),
    "hdp_lse_merge": (I32, [P, P, P, P, I32, I32, I32, P, P]),
    "hdp_attn_varlen_bwd": (I32, [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, F32, P, P, P, P]),
    "hdp_attn_varlen_bwd_noalloc": (I32, [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, F32, P, P, P, P]),
    "hdp_attn_chunk_bwd": (I32, [P, I32, P, P, I32, I64, I64, I32, I32, I32, I32, F32, P, P, P, P, P,
                                 P, P]),
    "hdp_seq_flops": (U64, [I64, I32, I32, I32, I32]),
    "hdp_chunk_flops": (U64, [I32, I32, I64, I64, I32, I32, I32, I32]),
    "hdp_pair_chunks": (I32, [I64, I32, I32, P, P]),
    "hdp_plan_shard": (I32, [P, I32, I64, I32, I32, I32, P, P, P, P, P, P, P]),
    "hdp_plan_unit_flops": (I32, [P, I32, I32, P, P, P, P, P, I32, I32, I32, P]),
    "hdp_plan_balance": (I32, [P, P, I32, I32, U64, P, P]),
    "hdp_probe_clock": (I32, [I32, P, P]),
    "hdp_set_trace": (I32, [P, I32]),
    "hdp_set_item_trace": (I32, [P, I32, I32]),
    "hdp_status_string": (ctypes.c_char_p, [I32]),
    "hdp_release_workspace": (I32, []),
}

_lib = None


class HdpError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s" % (fn, lib().hdp_status_string(status).decode()))


def lib():
    """Loads the library once; raises ImportError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libhdpattn.so is not built (expected at %s); run "
                          "`python -c 'import __graft_entry__ as g; g.build()'`" % LIB_PATH)
    l = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(l, name)
        fn.restype = res
        fn.argtypes = args
    _lib = l
    return l


def check(fn: str, status: int) -> None:
    if status != HDP_OK:
        raise HdpError(fn, status)
