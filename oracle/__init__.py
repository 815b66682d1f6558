"""fp64 CPU oracle for per-rank variable-length causal attention (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  It shares no code with the HIP library and never imports it.

The arithmetic lives in ``hdp_oracle.c`` (plain C, fp64, OpenMP over rows); this module only
marshals numpy arrays into it.  Inputs are widened to fp64 exactly (bf16 and fp32 both embed in
fp64), so the oracle sees the very values the GPU receives.

Sources ("Digest" = the research-digest page "ByteScale: Communication-Efficient Scaling of LLM
Training with a 2048K Context Length on 16384 GPUs"): packed short sequences that each attend
only to themselves (Digest §3.1, Figure 2; §3.2), ring steps over K/V chunks combined per step
(Digest §3.2), the causal mask (Digest §4), O(s^2) attention work (Digest §2).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hdp_oracle.c")
_LIB = os.path.join(_HERE, "libhdp_oracle.so")

_lib = None

ORC_OK = 0


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("HDP_ORACLE_LIB_PATH")   # another build of this file (sanitizers)
    if not path:
        build()
        path = _LIB
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.orc_varlen_fwd.argtypes = [P, P, P, P, i64, i32, i32, i32, f64, P, i64, P, P, i32]
    lib.orc_varlen_fwd.restype = i32
    lib.orc_chunk_partial.argtypes = [P, i64, P, P, i64, i64, i64, i32, i32, i32, i32, f64, P,
                                      i64, P, P, i32]
    lib.orc_chunk_partial.restype = i32
    lib.orc_lse_merge.argtypes = [P, P, P, P, i64, i32, i32]
    lib.orc_lse_merge.restype = i32
    lib.orc_varlen_bwd.argtypes = [P, P, P, P, P, i64, i32, i32, i32, f64, P, i64, P, i64, P, P,
                                   P, i32]
    lib.orc_varlen_bwd.restype = i32
    lib.orc_chunk_bwd.argtypes = [P, i64, P, P, i64, i64, i64, i32, i32, i32, i32, f64, P, P, P, P,
                                  i64, P, i64, P, P, P, i32]
    lib.orc_chunk_bwd.restype = i32
    lib.orc_count_pairs.argtypes = [i64, i64, i64, i64, i32]
    lib.orc_count_pairs.restype = ctypes.c_uint64
    lib.orc_attn_flops.argtypes = [i64, i64, i64, i64, i32, i32, i32, i32]
    lib.orc_attn_flops.restype = ctypes.c_uint64
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = i32
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    """Exact widening to a C-contiguous fp64 array (accepts numpy arrays or CPU torch tensors)."""
    if hasattr(a, "detach"):  # torch tensor: widen on the CPU, exactly
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _rows(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, int(r.shape[0])


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().orc_max_threads())


def varlen_fwd(q, k, v, cu_seqlens, scale, rows=None, nthreads=0):
    """Packed causal attention, forward.  q [T,H,D], k/v [T,Hkv,D]; returns (out, lse) in fp64.

    ``rows`` optionally selects packed token indices; outputs then follow that order.
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    n_seq = int(cu.shape[0]) - 1
    T, H, D = q.shape
    Hkv = k.shape[1]
    r, n_rows = _rows(rows)
    if r is None:
        n_rows = int(cu[-1]) if n_seq > 0 else 0
    out = np.zeros((n_rows, H, D), np.float64)
    lse = np.zeros((n_rows, H), np.float64)
    st = lib.orc_varlen_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu), n_seq, H, Hkv, D, float(scale),
                            _ptr(r), n_rows, _ptr(out), _ptr(lse), int(nthreads))
    if st != ORC_OK:
        raise ValueError("orc_varlen_fwd failed with status %d" % st)
    return out, lse


def chunk_partial(q_slice, k_chunk, v_chunk, q_offset, kv_offset, causal, scale, rows=None,
                  nthreads=0):
    """One ring step: slice [Lq,H,D] vs chunk [Lk,Hkv,D] at global offsets; (o, lse) fp64."""
    lib = _load()
    q, k, v = _f64(q_slice), _f64(k_chunk), _f64(v_chunk)
    Lq, H, D = q.shape
    Lk, Hkv = k.shape[0], k.shape[1]
    r, n_rows = _rows(rows)
    if r is None:
        n_rows = Lq
    o = np.zeros((n_rows, H, D), np.float64)
    lse = np.zeros((n_rows, H), np.float64)
    st = lib.orc_chunk_partial(_ptr(q), Lq, _ptr(k), _ptr(v), Lk, int(q_offset), int(kv_offset),
                               int(bool(causal)), H, Hkv, D, float(scale), _ptr(r), n_rows,
                               _ptr(o), _ptr(lse), int(nthreads))
    if st != ORC_OK:
        raise ValueError("orc_chunk_partial failed with status %d" % st)
    return o, lse


def lse_merge(o_acc, lse_acc, o_part, lse_part):
    """Returns the log-sum-exp merge of two partials (inputs are not modified)."""
    lib = _load()
    o = _f64(o_acc).copy()
    l = _f64(lse_acc).copy()
    op, lp = _f64(o_part), _f64(lse_part)
    n, H, D = o.shape
    st = lib.orc_lse_merge(_ptr(o), _ptr(l), _ptr(op), _ptr(lp), n, H, D)
    if st != ORC_OK:
        raise ValueError("orc_lse_merge failed with status %d" % st)
    return o, l


def varlen_bwd(q, k, v, dout, cu_seqlens, scale, qrows=None, krows=None, nthreads=0):
    """Backward by the chain rule; returns (dq [nq,H,D], dk [nk,Hkv,D], dv [nk,Hkv,D]) fp64."""
    lib = _load()
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    n_seq = int(cu.shape[0]) - 1
    T, H, D = q.shape
    Hkv = k.shape[1]
    qr, n_q = _rows(qrows)
    kr, n_k = _rows(krows)
    if qr is None:
        n_q = T
    if kr is None:
        n_k = T
    dq = np.zeros((n_q, H, D), np.float64)
    dk = np.zeros((n_k, Hkv, D), np.float64)
    dv = np.zeros((n_k, Hkv, D), np.float64)
    st = lib.orc_varlen_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(cu), n_seq, H, Hkv, D,
                            float(scale), _ptr(qr), n_q, _ptr(kr), n_k, _ptr(dq), _ptr(dk),
                            _ptr(dv), int(nthreads))
    if st != ORC_OK:
        raise ValueError("orc_varlen_bwd failed with status %d" % st)
    return dq, dk, dv


def chunk_bwd(q_slice, k_chunk, v_chunk, q_offset, kv_offset, causal, scale, out, lse, dout,
              qrows=None, krows=None, nthreads=0):
    """One ring step of the backward, given the slice's final out [Lq,H,D] and lse [Lq,H]:
    returns this chunk's share (dq [nq,H,D], dk [nk,Hkv,D], dv [nk,Hkv,D]) in fp64, for the
    selected slice rows / chunk rows (all by default)."""
    lib = _load()
    q, k, v = _f64(q_slice), _f64(k_chunk), _f64(v_chunk)
    o, l, do = _f64(out), _f64(lse), _f64(dout)
    Lq, H, D = q.shape
    Lk, Hkv = k.shape[0], k.shape[1]
    qr, n_q = _rows(qrows)
    kr, n_k = _rows(krows)
    if qr is None:
        n_q = Lq
    if kr is None:
        n_k = Lk
    dq = np.zeros((n_q, H, D), np.float64)
    dk = np.zeros((n_k, Hkv, D), np.float64)
    dv = np.zeros((n_k, Hkv, D), np.float64)
    st = lib.orc_chunk_bwd(_ptr(q), Lq, _ptr(k), _ptr(v), Lk, int(q_offset), int(kv_offset),
                           int(bool(causal)), H, Hkv, D, float(scale), _ptr(o), _ptr(l), _ptr(do),
                           _ptr(qr), n_q, _ptr(kr), n_k, _ptr(dq), _ptr(dk), _ptr(dv),
                           int(nthreads))
    if st != ORC_OK:
        raise ValueError("orc_chunk_bwd failed with status %d" % st)
    return dq, dk, dv


def count_pairs(Lq, Lk, q_offset=0, kv_offset=0, causal=True) -> int:
    return int(_load().orc_count_pairs(int(Lq), int(Lk), int(q_offset), int(kv_offset),
                                       int(bool(causal))))


def attn_flops(Lq, Lk, q_offset, kv_offset, causal, H, D, pass_) -> int:
    """FLOPs by enumeration of the visible pairs; pass_ 0 = fwd, 1 = bwd, 2 = fwd+bwd."""
    return int(_load().orc_attn_flops(int(Lq), int(Lk), int(q_offset), int(kv_offset),
                                      int(bool(causal)), int(H), int(D), int(pass_)))


def seq_flops(s, H, D, causal=True, pass_=0) -> int:
    """FLOPs of one whole sequence of s tokens attending to itself."""
    return attn_flops(s, s, 0, 0, causal, H, D, pass_)
