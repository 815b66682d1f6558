"""Python face of the C ABI: the same call names, torch tensors in, torch tensors out.

PyTorch provides device memory and the current HIP stream; every step of the computation runs
in libhdpattn.so.  Outputs not supplied by the caller are allocated here with torch.empty.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

import torch

from . import _lib

PASS_FWD, PASS_BWD, PASS_FWD_BWD = 0, 1, 2


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev_tensor(name: str, t: torch.Tensor, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got %d" % (name, ndim, t.dim()))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _shapes(fn: str, **named) -> None:
    """Every tensor must have exactly the shape the kernels index it with: a smaller or
    mis-shaped buffer would be read or written out of bounds on the device."""
    for name, (t, want) in named.items():
        if tuple(t.shape) != tuple(int(x) for x in want):
            raise ValueError("%s: %s has shape %s, expected %s" % (fn, name, tuple(t.shape), tuple(want)))


def _same_device(fn: str, *ts) -> None:
    devs = set(t.device for t in ts if t is not None)
    if len(devs) > 1:
        raise ValueError("%s: tensors on different devices %s" % (fn, sorted(map(str, devs))))


def _scale(D: int, scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def hdp_attn_varlen_fwd(q, k, v, cu_seqlens, scale=None, out=None, lse=None
                        ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Packed causal varlen attention, bf16.  q [T,H,D], k/v [T,Hkv,D], cu_seqlens int32 [n+1]."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(n, t, torch.bfloat16, 3)
    _dev_tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    T, H, D = q.shape
    Hkv = k.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _dev_tensor("out", out, torch.bfloat16, 3)
    _dev_tensor("lse", lse, torch.float32, 2)
    _shapes("hdp_attn_varlen_fwd", k=(k, (T, Hkv, D)), v=(v, (T, Hkv, D)), out=(out, (T, H, D)),
            lse=(lse, (T, H)))
    _same_device("hdp_attn_varlen_fwd", q, k, v, cu_seqlens, out, lse)
    st = _lib.lib().hdp_attn_varlen_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens),
                                        cu_seqlens.numel() - 1, H, Hkv, D, _scale(D, scale),
                                        _ptr(out), _ptr(lse), _stream())
    _lib.check("hdp_attn_varlen_fwd", st)
    return out, lse


def hdp_attn_varlen_fwd_f32(q, k, v, cu_seqlens, scale=None, out=None, lse=None
                            ) -> Tuple[torch.Tensor, torch.Tensor]:
    """fp32 form of hdp_attn_varlen_fwd."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(n, t, torch.float32, 3)
    _dev_tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    T, H, D = q.shape
    Hkv = k.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _dev_tensor("out", out, torch.float32, 3)
    _dev_tensor("lse", lse, torch.float32, 2)
    _shapes("hdp_attn_varlen_fwd_f32", k=(k, (T, Hkv, D)), v=(v, (T, Hkv, D)),
            out=(out, (T, H, D)), lse=(lse, (T, H)))
    _same_device("hdp_attn_varlen_fwd_f32", q, k, v, cu_seqlens, out, lse)
    st = _lib.lib().hdp_attn_varlen_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens),
                                            cu_seqlens.numel() - 1, H, Hkv, D, _scale(D, scale),
                                            _ptr(out), _ptr(lse), _stream())
    _lib.check("hdp_attn_varlen_fwd_f32", st)
    return out, lse


def hdp_attn_chunk_partial(q_slice, k_chunk, v_chunk, q_offset: int, kv_offset: int,
                           causal: bool = True, scale=None, o_partial=None, lse=None
                           ) -> Tuple[torch.Tensor, torch.Tensor]:
    """One ring step: q_slice [Lq,H,D] vs k/v chunk [Lk,Hkv,D] at global offsets (fp32 out)."""
    for n, t in (("q_slice", q_slice), ("k_chunk", k_chunk), ("v_chunk", v_chunk)):
        _dev_tensor(n, t, torch.bfloat16, 3)
    Lq, H, D = q_slice.shape
    Lk, Hkv = k_chunk.shape[0], k_chunk.shape[1]
    if o_partial is None:
        o_partial = torch.empty((Lq, H, D), dtype=torch.float32, device=q_slice.device)
    if lse is None:
        lse = torch.empty((Lq, H), dtype=torch.float32, device=q_slice.device)
    _dev_tensor("o_partial", o_partial, torch.float32, 3)
    _dev_tensor("lse", lse, torch.float32, 2)
    _shapes("hdp_attn_chunk_partial", v_chunk=(v_chunk, (Lk, Hkv, D)), k_chunk=(k_chunk, (Lk, Hkv, D)),
            o_partial=(o_partial, (Lq, H, D)), lse=(lse, (Lq, H)))
    _same_device("hdp_attn_chunk_partial", q_slice, k_chunk, v_chunk, o_partial, lse)
    st = _lib.lib().hdp_attn_chunk_partial(_ptr(q_slice), Lq, _ptr(k_chunk), _ptr(v_chunk), Lk,
                                           int(q_offset), int(kv_offset), int(bool(causal)), H,
                                           Hkv, D, _scale(D, scale), _ptr(o_partial), _ptr(lse),
                                           _stream())
    _lib.check("hdp_attn_chunk_partial", st)
    return o_partial, lse


def hdp_attn_chunk_merge(q_slice, k_chunk, v_chunk, q_offset: int, kv_offset: int, o_acc, lse_acc,
                         causal: bool = True, scale=None, out_bf16=None) -> None:
    """One ring step merged into the running (o_acc [Lq,H,D], lse_acc [Lq,H]) fp32, in place."""
    for n, t in (("q_slice", q_slice), ("k_chunk", k_chunk), ("v_chunk", v_chunk)):
        _dev_tensor(n, t, torch.bfloat16, 3)
    _dev_tensor("o_acc", o_acc, torch.float32, 3)
    _dev_tensor("lse_acc", lse_acc, torch.float32, 2)
    Lq, H, D = q_slice.shape
    Lk, Hkv = k_chunk.shape[0], k_chunk.shape[1]
    _shapes("hdp_attn_chunk_merge", k_chunk=(k_chunk, (Lk, Hkv, D)), v_chunk=(v_chunk, (Lk, Hkv, D)),
            o_acc=(o_acc, (Lq, H, D)), lse_acc=(lse_acc, (Lq, H)))
    if out_bf16 is not None:
        _dev_tensor("out_bf16", out_bf16, torch.bfloat16, 3)
        _shapes("hdp_attn_chunk_merge", out_bf16=(out_bf16, (Lq, H, D)))
    _same_device("hdp_attn_chunk_merge", q_slice, k_chunk, v_chunk, o_acc, lse_acc, out_bf16)
    st = _lib.lib().hdp_attn_chunk_merge(_ptr(q_slice), Lq, _ptr(k_chunk), _ptr(v_chunk), Lk,
                                         int(q_offset), int(kv_offset), int(bool(causal)), H, Hkv, D,
                                         _scale(D, scale), _ptr(o_acc), _ptr(lse_acc), _ptr(out_bf16),
                                         _stream())
    _lib.check("hdp_attn_chunk_merge", st)


def hdp_lse_merge(o_acc, lse_acc, o_part, lse_part, out_bf16=None) -> None:
    """In place: (o_acc, lse_acc) <- merge((o_acc, lse_acc), (o_part, lse_part))."""
    _dev_tensor("o_acc", o_acc, torch.float32, 3)
    _dev_tensor("lse_acc", lse_acc, torch.float32, 2)
    _dev_tensor("o_part", o_part, torch.float32, 3)
    _dev_tensor("lse_part", lse_part, torch.float32, 2)
    L, H, D = o_acc.shape
    if out_bf16 is not None:
        _dev_tensor("out_bf16", out_bf16, torch.bfloat16, 3)
        _shapes("hdp_lse_merge", out_bf16=(out_bf16, (L, H, D)))
    _shapes("hdp_lse_merge", lse_acc=(lse_acc, (L, H)), o_part=(o_part, (L, H, D)),
            lse_part=(lse_part, (L, H)))
    _same_device("hdp_lse_merge", o_acc, lse_acc, o_part, lse_part, out_bf16)
    st = _lib.lib().hdp_lse_merge(_ptr(o_acc), _ptr(lse_acc), _ptr(o_part), _ptr(lse_part), L, H,
                                  D, _ptr(out_bf16), _stream())
    _lib.check("hdp_lse_merge", st)


def hdp_attn_varlen_bwd(q, k, v, out, lse, dout, cu_seqlens, scale=None, dq=None, dk=None,
                        dv=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward of hdp_attn_varlen_fwd; returns (dq, dk, dv) in bf16."""
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _dev_tensor(n, t, torch.bfloat16, 3)
    _dev_tensor("lse", lse, torch.float32, 2)
    _dev_tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    T, H, D = q.shape
    Hkv = k.shape[1]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _dev_tensor(n, t, torch.bfloat16, 3)
    _shapes("hdp_attn_varlen_bwd", k=(k, (T, Hkv, D)), v=(v, (T, Hkv, D)), out=(out, (T, H, D)),
            lse=(lse, (T, H)), dout=(dout, (T, H, D)), dq=(dq, (T, H, D)), dk=(dk, (T, Hkv, D)),
            dv=(dv, (T, Hkv, D)))
    _same_device("hdp_attn_varlen_bwd", q, k, v, out, lse, dout, cu_seqlens, dq, dk, dv)
    st = _lib.lib().hdp_attn_varlen_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                        _ptr(dout), _ptr(cu_seqlens), cu_seqlens.numel() - 1, T,
                                        H, Hkv, D, _scale(D, scale), _ptr(dq), _ptr(dk), _ptr(dv),
                                        _stream())
    _lib.check("hdp_attn_varlen_bwd", st)
    return dq, dk, dv


def hdp_attn_chunk_bwd(q_slice, k_chunk, v_chunk, q_offset: int, kv_offset: int, out, lse, dout,
                       dq_acc, dk_acc, dv_acc, causal: bool = True, scale=None) -> None:
    """One ring step of the backward: adds this chunk's share to the fp32 accumulators
    dq_acc [Lq,H,D], dk_acc / dv_acc [Lk,Hkv,D] (in place)."""
    for n, t in (("q_slice", q_slice), ("k_chunk", k_chunk), ("v_chunk", v_chunk), ("out", out),
                 ("dout", dout)):
        _dev_tensor(n, t, torch.bfloat16, 3)
    _dev_tensor("lse", lse, torch.float32, 2)
    for n, t in (("dq_acc", dq_acc), ("dk_acc", dk_acc), ("dv_acc", dv_acc)):
        _dev_tensor(n, t, torch.float32, 3)
    Lq, H, D = q_slice.shape
    Lk, Hkv = k_chunk.shape[0], k_chunk.shape[1]
    _shapes("hdp_attn_chunk_bwd", k_chunk=(k_chunk, (Lk, Hkv, D)), v_chunk=(v_chunk, (Lk, Hkv, D)),
            out=(out, (Lq, H, D)), dout=(dout, (Lq, H, D)), lse=(lse, (Lq, H)),
            dq_acc=(dq_acc, (Lq, H, D)), dk_acc=(dk_acc, (Lk, Hkv, D)), dv_acc=(dv_acc, (Lk, Hkv, D)))
    _same_device("hdp_attn_chunk_bwd", q_slice, k_chunk, v_chunk, out, lse, dout, dq_acc, dk_acc, dv_acc)
    st = _lib.lib().hdp_attn_chunk_bwd(_ptr(q_slice), Lq, _ptr(k_chunk), _ptr(v_chunk), Lk,
                                       int(q_offset), int(kv_offset), int(bool(causal)), H, Hkv, D,
                                       _scale(D, scale), _ptr(out), _ptr(lse), _ptr(dout),
                                       _ptr(dq_acc), _ptr(dk_acc), _ptr(dv_acc), _stream())
    _lib.check("hdp_attn_chunk_bwd", st)


def hdp_seq_flops(s: int, H: int, D: int, causal: bool = True, pass_: int = PASS_FWD) -> int:
    return int(_lib.lib().hdp_seq_flops(int(s), int(H), int(D), int(bool(causal)), int(pass_)))


def hdp_chunk_flops(Lq: int, Lk: int, q_offset: int, kv_offset: int, causal: bool, H: int,
                    D: int, pass_: int = PASS_FWD) -> int:
    return int(_lib.lib().hdp_chunk_flops(int(Lq), int(Lk), int(q_offset), int(kv_offset),
                                          int(bool(causal)), int(H), int(D), int(pass_)))


def hdp_pair_chunks(s: int, n_ranks: int, rank: int):
    """Front/back pairing: [(offset, length) of chunk rank, (offset, length) of chunk 2N-1-rank]."""
    off = (ctypes.c_int64 * 2)()
    ln = (ctypes.c_int64 * 2)()
    st = _lib.lib().hdp_pair_chunks(int(s), int(n_ranks), int(rank), ctypes.addressof(off),
                                    ctypes.addressof(ln))
    _lib.check("hdp_pair_chunks", st)
    return [(int(off[0]), int(ln[0])), (int(off[1]), int(ln[1]))]


class Plan:
    """A plan from hdp_plan_shard: per unit, its ring (sequence index, -1 if packed) and its
    pieces [(sequence, offset, length)]; the flat arrays are kept for the other planner calls."""

    def __init__(self, lens, first, ring, pseq, poff, plen):
        self.lens, self.first, self.ring = lens, first, ring
        self.pseq, self.poff, self.plen = pseq, poff, plen

    def __len__(self):
        return len(self.ring)

    def units(self):
        return [(int(self.ring[j]), [(int(self.pseq[p]), int(self.poff[p]), int(self.plen[p]))
                                     for p in range(self.first[j], self.first[j + 1])])
                for j in range(len(self.ring))]


def _i64(xs):
    return (ctypes.c_int64 * max(1, len(xs)))(*[int(x) for x in xs])


def hdp_plan_shard(lens, C: int, pair: bool = False) -> Plan:
    L = _lib.lib()
    n = len(lens)
    lens_c = _i64(lens)
    nu, npc = ctypes.c_int32(0), ctypes.c_int32(0)
    st = L.hdp_plan_shard(ctypes.addressof(lens_c), n, int(C), int(bool(pair)), 0, 0,
                          ctypes.addressof(nu), ctypes.addressof(npc), None, None, None, None, None)
    if st not in (_lib.HDP_OK, _lib.HDP_ERR_OVERFLOW):
        _lib.check("hdp_plan_shard", st)
    U, Pn = nu.value, npc.value
    first = (ctypes.c_int32 * (U + 1))()
    ring = (ctypes.c_int32 * max(1, U))()
    pseq = (ctypes.c_int32 * max(1, Pn))()
    poff = (ctypes.c_int64 * max(1, Pn))()
    plen = (ctypes.c_int64 * max(1, Pn))()
    st = L.hdp_plan_shard(ctypes.addressof(lens_c), n, int(C), int(bool(pair)), U, Pn,
                          ctypes.addressof(nu), ctypes.addressof(npc), ctypes.addressof(first),
                          ctypes.addressof(ring), ctypes.addressof(pseq), ctypes.addressof(poff),
                          ctypes.addressof(plen))
    _lib.check("hdp_plan_shard", st)
    return Plan(lens_c, list(first), list(ring)[:U], pseq, poff, plen)


def hdp_plan_unit_flops(plan: Plan, H: int, D: int, pass_: int = PASS_FWD):
    U = len(plan)
    first = (ctypes.c_int32 * (U + 1))(*plan.first)
    ring = (ctypes.c_int32 * max(1, U))(*plan.ring)
    cost = (ctypes.c_uint64 * max(1, U))()
    st = _lib.lib().hdp_plan_unit_flops(ctypes.addressof(plan.lens), len(plan.lens) if U else 0, U,
                                        ctypes.addressof(first), ctypes.addressof(ring),
                                        ctypes.addressof(plan.pseq), ctypes.addressof(plan.poff),
                                        ctypes.addressof(plan.plen), int(H), int(D), int(pass_),
                                        ctypes.addressof(cost))
    _lib.check("hdp_plan_unit_flops", st)
    return [int(c) for c in cost][:U]


def hdp_plan_balance(cost, unit_ring, n_ranks: int, delta: int = 0):
    """Returns (rank of each unit, load of each rank)."""
    U = len(cost)
    c = (ctypes.c_uint64 * max(1, U))(*[int(x) for x in cost])
    r = (ctypes.c_int32 * max(1, U))(*[int(x) for x in unit_ring])
    ur = (ctypes.c_int32 * max(1, U))()
    load = (ctypes.c_uint64 * n_ranks)()
    st = _lib.lib().hdp_plan_balance(ctypes.addressof(c), ctypes.addressof(r), U, int(n_ranks),
                                     int(delta), ctypes.addressof(ur), ctypes.addressof(load))
    _lib.check("hdp_plan_balance", st)
    return [int(x) for x in ur][:U], [int(x) for x in load]


def hdp_probe_clock(iters: int = 20000) -> float:
    """Shader clock (MHz) sustained under back-to-back MFMAs on every CU (measurement helper)."""
    mhz = ctypes.c_double(0.0)
    _lib.check("hdp_probe_clock", _lib.lib().hdp_probe_clock(int(iters), ctypes.addressof(mhz), _stream()))
    return float(mhz.value)


def hdp_set_trace(trace: Optional[torch.Tensor]) -> None:
    """Per-workgroup forward trace into an int64 device tensor of 4 words per workgroup (None:
    off).  Measurement helper."""
    if trace is None:
        _lib.check("hdp_set_trace", _lib.lib().hdp_set_trace(None, 0))
        return
    _dev_tensor("trace", trace, torch.int64, 1)
    _lib.check("hdp_set_trace", _lib.lib().hdp_set_trace(trace.data_ptr(), trace.numel() // 4))


def hdp_set_item_trace(items: Optional[torch.Tensor], slots: int = 0) -> None:
    """Per-item forward timeline into an int64 device tensor of 4 x slots words per workgroup
    (None: off).  Measurement helper."""
    if items is None:
        _lib.check("hdp_set_item_trace", _lib.lib().hdp_set_item_trace(None, 0, 0))
        return
    _dev_tensor("items", items, torch.int64, 1)
    if slots <= 0:
        raise ValueError("slots must be positive")
    _lib.check("hdp_set_item_trace",
               _lib.lib().hdp_set_item_trace(items.data_ptr(), items.numel() // (4 * slots), int(slots)))


def hdp_release_workspace() -> None:
    _lib.check("hdp_release_workspace", _lib.lib().hdp_release_workspace())
