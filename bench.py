"""Throughput of the per-rank attention hot path on one MI355X.

Headline: causal varlen attention forward on one rank's 8192-token packed slice (skewed length
mix; GQA 32 query / 8 key-value heads; D = 128; bf16), as TFLOP/s of exact algorithmic FLOPs
(hdp_seq_flops: 4*H*D per visible (query, key) pair) and as a fraction of the bf16 dense MFMA
peak.  Method: about a second of untimed launches of the same step (the GPU reaches its steady
clock), then W untimed warm-up steps, then K timed steps (defaults 20 and 200, the pages' own
method: mean of 200 iterations after 20 warm-up), bracketed by device synchronisation.
One step = one call of hdp_attn_varlen_fwd over the resident slice.

Printed: one JSON line (rank 0).  `roofline.achieved` is the FLOPs of one launch divided by the
kernel's mean duration from per-launch HIP events on the launch stream; `roofline.traffic` is
the HBM byte count per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE counters recorded under
profiles/ (null if absent or taken on a different kernel source).  `cpu_baseline` times the
fp64 oracle on a bounded sample of the same slice on the host cores.  `detail` adds the other
rows of the hot path (ring chunks + LSE merge, 32K micro-batches, backward) for context; each
of them times at least 50 launches and at least 100 ms, whatever --steps says, and reports
per-launch mean / min / median / max.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_FP32_VECTOR_TFLOPS = 157.3   # MI355X fp32 vector (the fp32 path's roofline)
NOMINAL_MHZ = 2400.0          # the clock the bf16 peak is quoted at
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_packed_slice_8k.json")
# the forward kernel's sources: counters taken on another version of them do not apply
FWD_SRC = [os.path.join(ROOT, "variable_length_attention_amd", "csrc", f)
           for f in ("fwd_bf16.hip", "device_common.h", "hdp_internal.h")]


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch from the committed counter summary, if it matches this source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != source_hash(FWD_SRC):
        return None
    return t.get("hbm_bytes_per_launch")


def timed_launches(fn, steps: int, warmup: int, torch):
    """Runs fn() warmup+steps times.  Returns the mean ms per step over the bracket (device
    synchronised on both sides) and per-launch statistics from HIP events recorded around each
    call on the stream the kernels run on (torch's current stream)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    outer0 = torch.cuda.Event(enable_timing=True)
    outer1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    outer0.record()
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    outer1.record()
    torch.cuda.synchronize()
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return {"ms_step": outer0.elapsed_time(outer1) / steps, "launches": steps,
            "mean_ms": sum(per) / len(per), "min_ms": per[0], "median_ms": per[len(per) // 2],
            "max_ms": per[-1]}


def timed_floor(fn, torch, min_launches: int = 50, min_ms: float = 100.0, warmup: int = 3):
    """timed_launches with at least min_launches launches and at least min_ms of timed work,
    whatever --steps says (a few launches are timed first to size the run)."""
    probe = timed_launches(fn, 3, warmup, torch)
    n = max(min_launches, int(math.ceil(min_ms / max(probe["mean_ms"], 1e-3))))
    return timed_launches(fn, n, 2, torch)


def settle_clock(fn, torch, ms: float) -> dict:
    """Untimed launches of the headline step for about `ms` of wall time, so that the GPU has
    reached its steady clock under this load before the warm-up and timed steps begin."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(20):
            fn()
        n += 20
        torch.cuda.synchronize()
    return {"settle_launches": n, "settle_ms": round((time.perf_counter() - t0) * 1e3, 1)}


def us_stats(t: dict) -> dict:
    return {"launches": t["launches"], "mean_us": round(t["mean_ms"] * 1e3, 2),
            "min_us": round(t["min_ms"] * 1e3, 2), "median_us": round(t["median_ms"] * 1e3, 2),
            "max_us": round(t["max_ms"] * 1e3, 2)}


def cpu_baseline(w, q, k, v, cu):
    """The fp64 oracle on the whole slice (every row, all heads), repeated until about 10 s of
    wall time (at most 20 passes), scaled to TFLOP/s."""
    import oracle

    flops = sum(int(s) * (int(s) + 1) // 2 for s in w.lengths) * w.H * 4 * w.D
    times = []
    t_start = time.perf_counter()
    while not times or (time.perf_counter() - t_start < 10.0 and len(times) < 20):
        t0 = time.perf_counter()
        oracle.varlen_fwd(q, k, v, cu, w.scale)
        times.append(time.perf_counter() - t0)
    dt = sum(times) / len(times)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": "the whole 8192-token slice (all rows, all 32 heads, %.3g FLOP), %d passes, "
                      "mean %.2f s per pass" % (flops, len(times), dt)}


def detail_rows(torch, ops, synth):
    """Other rows of the hot path, timed the same way (context, not the headline)."""
    out = {}
    # ring-chunk share: 16 chunk partials + 15 LSE merges (and the same with the merge fused)
    w = synth.ring_chunks_128k()
    q, k, v = (t.cuda() for t in synth.ring_tensors(w))
    L = w.chunk_len
    acc_o = torch.empty((w.q_len, w.H, w.D), dtype=torch.float32, device="cuda")
    acc_l = torch.empty((w.q_len, w.H), dtype=torch.float32, device="cuda")
    po, pl = torch.empty_like(acc_o), torch.empty_like(acc_l)
    chunks = [(k[c * L:(c + 1) * L], v[c * L:(c + 1) * L]) for c in range(w.n_chunks)]

    def ring_step():
        ops.hdp_attn_chunk_partial(q, chunks[0][0], chunks[0][1], w.q_offset, 0, True, w.scale,
                                   o_partial=acc_o, lse=acc_l)
        for c in range(1, w.n_chunks):
            ops.hdp_attn_chunk_partial(q, chunks[c][0], chunks[c][1], w.q_offset, c * L, True,
                                       w.scale, o_partial=po, lse=pl)
            ops.hdp_lse_merge(acc_o, acc_l, po, pl)

    t_ring = timed_floor(ring_step, torch)
    ms = t_ring["ms_step"]
    fl = sum(ops.hdp_chunk_flops(w.q_len, L, w.q_offset, c * L, True, w.H, w.D) for c in range(w.n_chunks))
    # the same share with each step's merge fused into its epilogue (hdp_attn_chunk_merge)
    def ring_step_fused():
        acc_l.fill_(-float("inf"))
        for c in range(w.n_chunks):
            ops.hdp_attn_chunk_merge(q, chunks[c][0], chunks[c][1], w.q_offset, c * L, acc_o, acc_l, True, w.scale)

    t_fused = timed_floor(ring_step_fused, torch)
    t_merge = timed_floor(lambda: ops.hdp_lse_merge(acc_o, acc_l, po, pl), torch, min_launches=200)
    merge_ms = t_merge["mean_ms"]
    merge_bytes = w.q_len * w.H * (12 * w.D + 12)
    # the share's backward: 16 chunk backward steps into fp32 accumulators, given the merged
    # forward result (out rounded to bf16, lse) and a seeded dO
    ring_step()
    out_bf16 = acc_o.to(torch.bfloat16)
    dout = synth.ring_bwd_tensors(w)[2].cuda()
    dq_acc = torch.zeros_like(acc_o)
    dk_acc = torch.zeros((L, w.Hkv, w.D), dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros_like(dk_acc)

    def ring_bwd_step():
        for c in range(w.n_chunks):
            ops.hdp_attn_chunk_bwd(q, chunks[c][0], chunks[c][1], w.q_offset, c * L, out_bf16, acc_l,
                                   dout, dq_acc, dk_acc, dv_acc, causal=True, scale=w.scale)

    t_rbwd = timed_floor(ring_bwd_step, torch, min_launches=20)
    bms = t_rbwd["ms_step"]
    fb = sum(ops.hdp_chunk_flops(w.q_len, L, w.q_offset, c * L, True, w.H, w.D, 1) for c in range(w.n_chunks))
    out["ring_chunks_128k"] = {"ms_per_step": ms, "TFLOP/s": fl / (ms * 1e-3) / 1e12,
                               "step": us_stats(t_ring),
                               "fused_ms_per_step": t_fused["ms_step"],
                               "fused_TFLOP/s": fl / (t_fused["ms_step"] * 1e-3) / 1e12,
                               "fused_step": us_stats(t_fused),
                               "merge_us": merge_ms * 1e3,
                               "merge_GB/s": merge_bytes / (merge_ms * 1e-3) / 1e9,
                               "merge": us_stats(t_merge),
                               "bwd_ms_per_step": bms, "bwd_TFLOP/s": fb / (bms * 1e-3) / 1e12,
                               "bwd_step": us_stats(t_rbwd)}
    del q, k, v, chunks, acc_o, acc_l, po, pl, out_bf16, dout, dq_acc, dk_acc, dv_acc
    # the same 128K sequence over the same 16 ranks with front/back chunk pairing: rank k holds
    # query chunks k and 31-k (4096 tokens each) and meets all 32 chunks; every rank does the
    # same causal work (rank 0 and rank 15 timed), against the contiguous share above
    w = synth.ring_chunks_128k()
    S = w.n_chunks * w.chunk_len
    N = w.n_chunks
    _, kfull, vfull = synth.ring_tensors(w)
    kfull, vfull = kfull.cuda(), vfull.cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.tensor_seed + 7)
    qfull = torch.randn((S, w.H, w.D), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    allc = [c for r in range(N) for c in ops.hdp_pair_chunks(S, N, r)]
    pair_rows = {}
    for rank in (0, N - 1):
        mine = ops.hdp_pair_chunks(S, N, rank)
        bufs = [(torch.empty((ql, w.H, w.D), dtype=torch.float32, device="cuda"),
                 torch.empty((ql, w.H), dtype=torch.float32, device="cuda"),
                 torch.empty((ql, w.H, w.D), dtype=torch.float32, device="cuda"),
                 torch.empty((ql, w.H), dtype=torch.float32, device="cuda")) for _, ql in mine]
        steps_ = [(i, qo, ql, ko, kl) for i, (qo, ql) in enumerate(mine) for ko, kl in allc
                  if ko <= qo + ql - 1]

        def pair_step():
            first = [True, True]
            for i, qo, ql, ko, kl in steps_:
                ao, al, po_, pl_ = bufs[i]
                if first[i]:
                    ops.hdp_attn_chunk_partial(qfull[qo:qo + ql], kfull[ko:ko + kl], vfull[ko:ko + kl],
                                               qo, ko, True, w.scale, o_partial=ao, lse=al)
                    first[i] = False
                else:
                    ops.hdp_attn_chunk_partial(qfull[qo:qo + ql], kfull[ko:ko + kl], vfull[ko:ko + kl],
                                               qo, ko, True, w.scale, o_partial=po_, lse=pl_)
                    ops.hdp_lse_merge(ao, al, po_, pl_)

        t_pair = timed_floor(pair_step, torch)
        pms = t_pair["ms_step"]
        pfl = sum(ops.hdp_chunk_flops(ql, kl, qo, ko, True, w.H, w.D) for _, qo, ql, ko, kl in steps_)
        pair_rows["rank%d" % rank] = {"ms_per_step": pms, "GFLOP": pfl / 1e9,
                                      "TFLOP/s": pfl / (pms * 1e-3) / 1e12, "calls": len(steps_),
                                      "step": us_stats(t_pair)}
    out["ring_pairs_128k"] = pair_rows
    del kfull, vfull, qfull
    # backward (and forward + backward) on the 8K slice and on one 8K sequence
    for make in (synth.fwd_bwd_8k_slice, synth.fwd_bwd_8k_single):
        w = make()
        qq, kk, vv, dd = (t.cuda() for t in synth.varlen_tensors(w, with_dout=True))
        cu = torch.from_numpy(synth.cu_seqlens(w.lengths)).cuda()
        o, lse = ops.hdp_attn_varlen_fwd(qq, kk, vv, cu, w.scale)
        dq, dk, dv = torch.empty_like(qq), torch.empty_like(kk), torch.empty_like(vv)
        t_f = timed_floor(lambda: ops.hdp_attn_varlen_fwd(qq, kk, vv, cu, w.scale, out=o, lse=lse), torch)
        t_b = timed_floor(lambda: ops.hdp_attn_varlen_bwd(qq, kk, vv, o, lse, dd, cu, w.scale,
                                                          dq=dq, dk=dk, dv=dv), torch)
        fwd_ms, bwd_ms = t_f["mean_ms"], t_b["mean_ms"]
        ff = sum(ops.hdp_seq_flops(s, w.H, w.D, True, 0) for s in w.lengths)
        fb = sum(ops.hdp_seq_flops(s, w.H, w.D, True, 1) for s in w.lengths)
        out[w.name] = {"fwd_us": fwd_ms * 1e3, "bwd_us": bwd_ms * 1e3,
                       "fwd": us_stats(t_f), "bwd": us_stats(t_b),
                       "fwd_TFLOP/s": ff / (fwd_ms * 1e-3) / 1e12,
                       "bwd_TFLOP/s": fb / (bwd_ms * 1e-3) / 1e12,
                       "fwd_bwd_TFLOP/s": (ff + fb) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12}
        del qq, kk, vv, dd, o, lse, dq, dk, dv
    for make in (synth.microbatch_32k_long, synth.microbatch_32k_short):
        w = make()
        qq, kk, vv = (t.cuda() for t in synth.varlen_tensors(w))
        cu = torch.from_numpy(synth.cu_seqlens(w.lengths)).cuda()
        o = torch.empty_like(qq)
        lse = torch.empty((qq.shape[0], w.H), dtype=torch.float32, device="cuda")
        t_m = timed_floor(lambda: ops.hdp_attn_varlen_fwd(qq, kk, vv, cu, w.scale, out=o, lse=lse), torch)
        ms = t_m["mean_ms"]
        fl = sum(ops.hdp_seq_flops(s, w.H, w.D) for s in w.lengths)
        out[w.name] = {"n_seq": len(w.lengths), "GFLOP": fl / 1e9, "kernel_us": ms * 1e3,
                       "TFLOP/s": fl / (ms * 1e-3) / 1e12, "launch": us_stats(t_m)}
    # the tiny fp32 pack (4 sequences, 256 tokens, H = 4, D = 64): a VALU kernel, one lane per
    # row, launch-bound by design; its roofline is the fp32 vector peak
    w = synth.tiny_fp32_pack()
    qq, kk, vv = (t.cuda() for t in synth.varlen_tensors(w))
    cu = torch.from_numpy(synth.cu_seqlens(w.lengths)).cuda()
    o = torch.empty_like(qq)
    lse = torch.empty((qq.shape[0], w.H), dtype=torch.float32, device="cuda")
    t_t = timed_floor(lambda: ops.hdp_attn_varlen_fwd_f32(qq, kk, vv, cu, w.scale, out=o, lse=lse), torch,
                      min_launches=200)
    fl = sum(ops.hdp_seq_flops(s, w.H, w.D) for s in w.lengths)
    out[w.name] = {"n_seq": len(w.lengths), "GFLOP": fl / 1e9, "kernel_us": t_t["mean_ms"] * 1e3,
                   "fp32_tflops": fl / (t_t["mean_ms"] * 1e-3) / 1e12,
                   "frac_fp32_vector_peak": fl / (t_t["mean_ms"] * 1e-3) / 1e12 / PEAK_FP32_VECTOR_TFLOPS,
                   "launch": us_stats(t_t)}
    # every throughput also as a fraction of its roofline: TFLOP/s against the bf16 MFMA peak,
    # GB/s against HBM
    def add_fracs(row):
        for key in list(row):
            if isinstance(row[key], dict):
                add_fracs(row[key])
            elif key.endswith("TFLOP/s"):
                row[key[:-len("TFLOP/s")] + "frac_bf16_peak"] = row[key] / PEAK_BF16_TFLOPS
            elif key.endswith("GB/s"):
                row[key[:-len("GB/s")] + "frac_hbm"] = row[key] / PEAK_HBM_GBS
    for row in out.values():
        add_fracs(row)
    return out


def cu_timeline(torch, ops, synth, launches: int = 20) -> dict:
    """Per-workgroup busy time of the forward on the 8K slice and both 32K micro-batches: the
    persistent kernel runs one workgroup per CU, each records when it started and when it finished
    its last item (hdp_set_trace), and for each item when it started, when its first loads had
    landed and when its last step was done (hdp_set_item_trace).  Reported per workload, averaged
    over `launches` launches: finish time of the last / mean / first workgroup after the first one
    started, in us, the last workgroup of each XCD (workgroup w runs on XCD w mod 8), and each
    workgroup's time split into waiting for first loads, steps (fitted as a cost per 32-key unit
    plus a fixed cost per item) and item transitions (output stores, pop, next item's loads).
    Backward (8K slice, one 8K sequence): when each workgroup left the dK/dV queue and finished."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    trace = torch.zeros(4 * n_cu, dtype=torch.int64, device="cuda")
    slots = 32
    item_buf = torch.zeros(4 * slots * n_cu, dtype=torch.int64, device="cuda")
    out = {}
    for make in (synth.packed_slice_8k, synth.microbatch_32k_long, synth.microbatch_32k_short):
        w = make()
        qq, kk, vv = (t.cuda() for t in synth.varlen_tensors(w))
        cu = torch.from_numpy(synth.cu_seqlens(w.lengths)).cuda()
        o = torch.empty_like(qq)
        lse = torch.empty((qq.shape[0], w.H), dtype=torch.float32, device="cuda")

        def step():
            ops.hdp_attn_varlen_fwd(qq, kk, vv, cu, w.scale, out=o, lse=lse)

        settle_clock(step, torch, 300.0)
        rows, recs = [], []
        ops.hdp_set_trace(trace)
        ops.hdp_set_item_trace(item_buf, slots)
        try:
            for _ in range(launches):
                trace.zero_()
                item_buf.zero_()
                step()
                torch.cuda.synchronize()
                t = trace.view(n_cu, 4).cpu().numpy()
                rows.append(t.copy())
                recs.append(item_buf.view(n_cu, slots, 4).cpu().numpy())
        finally:
            ops.hdp_set_trace(None)
            ops.hdp_set_item_trace(None)
        # (records are read after the launches: host work between launches would let the clock drop)
        items_rows = []
        for t, it in zip(rows, recs):
            for b in range(n_cu):
                n = int(t[b, 2])
                for i in range(min(n, slots)):
                    if i + 1 < n and i + 1 >= slots:
                        continue                           # next start not recorded
                    nxt = it[b, i + 1, 0] if i + 1 < n else t[b, 1]
                    a0, a1, a2, nu = (int(x) for x in it[b, i])
                    items_rows.append((nu, (a1 - a0) / 100.0, (a2 - a1) / 100.0, (nxt - a2) / 100.0))
        fin, busy, items, xcd_last = [], [], [], []
        for t in rows:
            t0 = int(t[:, 0].min())
            f = (t[:, 1] - t0) / 100.0            # 100 MHz real-time counter -> us
            fin.append(f)
            busy.append((t[:, 1] - t[:, 0]) / 100.0)
            items.append(t[:, 2])
            xcd_last.append([float(f[x::8].max()) for x in range(8)])
        import numpy as np
        fin, busy, items = np.array(fin), np.array(busy), np.array(items)
        out[w.name] = {
            "n_seq": len(w.lengths), "launches": launches, "workgroups": n_cu,
            "last_finish_us": round(float(fin.max(axis=1).mean()), 2),
            "mean_finish_us": round(float(fin.mean(axis=1).mean()), 2),
            "first_finish_us": round(float(fin.min(axis=1).mean()), 2),
            "mean_busy_us": round(float(busy.mean()), 2),
            "busy_over_last_finish": round(float(busy.mean(axis=1).mean() / fin.max(axis=1).mean()), 4),
            "items_per_workgroup_min_mean_max": [int(items.min()), round(float(items.mean()), 2), int(items.max())],
            "xcd_last_finish_us": [round(float(x), 2) for x in np.array(xcd_last).mean(axis=0)],
        }
        r = np.array(items_rows, dtype=np.float64)
        nu, wait, steps, trans = r[:, 0], r[:, 1], r[:, 2], r[:, 3]
        per_unit, fixed = np.linalg.lstsq(np.vstack([nu, np.ones_like(nu)]).T, steps, rcond=None)[0]
        per_wg = 1.0 / (launches * n_cu)
        out[w.name]["items"] = {
            "records": int(len(r)),
            "per_workgroup_us_wait_steps_transitions": [round(float(wait.sum() * per_wg), 2), round(float(steps.sum() * per_wg), 2),
                                                        round(float(trans.sum() * per_wg), 2)],
            "per_item_us_wait_transition": [round(float(wait.mean()), 3), round(float(trans.mean()), 3)],
            "transition_us_p10_p90": [round(float(np.percentile(trans, 10)), 3), round(float(np.percentile(trans, 90)), 3)],
            "steps_us_per_unit_and_fixed_per_item": [round(float(per_unit), 4), round(float(fixed), 3)],
            "mean_units_per_item": round(float(nu.mean()), 2),
        }
        del qq, kk, vv, o, lse
    # backward: each workgroup records its start, when it left the dK/dV queue and its end
    for make in (synth.fwd_bwd_8k_slice, synth.fwd_bwd_8k_single):
        w = make()
        qq, kk, vv, dd = (t.cuda() for t in synth.varlen_tensors(w, with_dout=True))
        cu = torch.from_numpy(synth.cu_seqlens(w.lengths)).cuda()
        o, lse = ops.hdp_attn_varlen_fwd(qq, kk, vv, cu, w.scale)
        dq, dk, dv = torch.empty_like(qq), torch.empty_like(kk), torch.empty_like(vv)

        def bstep():
            ops.hdp_attn_varlen_bwd(qq, kk, vv, o, lse, dd, cu, w.scale, dq=dq, dk=dk, dv=dv)

        settle_clock(bstep, torch, 300.0)
        rows = []
        ops.hdp_set_trace(trace)
        try:
            for _ in range(launches):
                trace.zero_()
                bstep()
                torch.cuda.synchronize()
                rows.append(trace.view(n_cu, 4).cpu().numpy().copy())
        finally:
            ops.hdp_set_trace(None)
        import numpy as np
        left, fin, busy = [], [], []
        for t in rows:
            t0 = int(t[:, 0].min())
            left.append((t[:, 1] - t0) / 100.0)
            fin.append((t[:, 2] - t0) / 100.0)
            busy.append((t[:, 2] - t[:, 0]) / 100.0)
        left, fin, busy = np.array(left), np.array(fin), np.array(busy)
        mm = lambda a: [round(float(a.min(axis=1).mean()), 1), round(float(a.mean()), 1), round(float(a.max(axis=1).mean()), 1)]
        out["bwd." + w.name] = {
            "n_seq": len(w.lengths), "launches": launches, "workgroups": n_cu,
            "left_dkdv_queue_us_min_mean_max": mm(left),
            "finish_us_min_mean_max": mm(fin),
            "busy_over_last_finish": round(float(busy.mean(axis=1).mean() / fin.max(axis=1).mean()), 4),
        }
        del qq, kk, vv, dd, o, lse, dq, dk, dv
    return out


def run_sample(torch, ops, synth, name: str, launches: int) -> dict:
    """`launches` launches of one named workload with nothing else around them: the command a
    counter profile of one kernel runs (slice_fwd, long_fwd, short_fwd, ring_chunk, merge,
    slice_bwd, single_bwd, chunk_bwd_past, chunk_bwd_diag)."""
    if name in ("chunk_bwd_past", "chunk_bwd_diag"):
        # one backward ring step of the 128K share: chunk 0 (wholly in the past of the slice)
        # or chunk 15 (the slice's own diagonal chunk), into fp32 accumulators
        w = synth.ring_chunks_128k()
        q, k, v = (t.cuda() for t in synth.ring_tensors(w))
        o, lse, do = (t.cuda() for t in synth.ring_bwd_tensors(w))
        L = w.chunk_len
        c = 0 if name == "chunk_bwd_past" else w.n_chunks - 1
        kc, vc = k[c * L:(c + 1) * L], v[c * L:(c + 1) * L]
        dq = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
        dk = torch.zeros((L, w.Hkv, w.D), dtype=torch.float32, device="cuda")
        dv = torch.zeros_like(dk)
        fn = lambda: ops.hdp_attn_chunk_bwd(q, kc, vc, w.q_offset, c * L, o, lse, do, dq, dk, dv, True, w.scale)
    elif name in ("ring_chunk", "merge"):
        w = synth.ring_chunks_128k()
        q, k, v = (t.cuda() for t in synth.ring_tensors(w))
        L = w.chunk_len
        po, pl = ops.hdp_attn_chunk_partial(q, k[:L], v[:L], w.q_offset, 0, True, w.scale)
        acc_o, acc_l = po.clone(), pl.clone()
        if name == "ring_chunk":
            fn = lambda: ops.hdp_attn_chunk_partial(q, k[:L], v[:L], w.q_offset, 0, True, w.scale, o_partial=po, lse=pl)
        else:
            fn = lambda: ops.hdp_lse_merge(acc_o, acc_l, po, pl)
    else:
        make = {"slice_fwd": synth.packed_slice_8k, "long_fwd": synth.microbatch_32k_long,
                "short_fwd": synth.microbatch_32k_short, "slice_bwd": synth.fwd_bwd_8k_slice,
                "single_bwd": synth.fwd_bwd_8k_single}[name]
        w = make()
        qq, kk, vv, dd = (t.cuda() for t in synth.varlen_tensors(w, with_dout=True))
        cu = torch.from_numpy(synth.cu_seqlens(w.lengths)).cuda()
        o, lse = ops.hdp_attn_varlen_fwd(qq, kk, vv, cu, w.scale)
        if name.endswith("_fwd"):
            fn = lambda: ops.hdp_attn_varlen_fwd(qq, kk, vv, cu, w.scale, out=o, lse=lse)
        else:
            dq, dk, dv = torch.empty_like(qq), torch.empty_like(kk), torch.empty_like(vv)
            fn = lambda: ops.hdp_attn_varlen_bwd(qq, kk, vv, o, lse, dd, cu, w.scale, dq=dq, dk=dk, dv=dv)
    t = timed_launches(fn, launches, 2, torch)
    return {"sample": name, **us_stats(t)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=1000.0,
                    help="untimed launches of the headline step before its warm-up, so the timed "
                         "steps run at the steady clock")
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--sample", default=None,
                    help="only time --steps launches of one workload (slice_fwd, long_fwd, short_fwd, "
                         "ring_chunk, merge, slice_bwd, single_bwd, chunk_bwd_past, chunk_bwd_diag), for "
                         "counter profiles")
    ap.add_argument("--cu-timeline", action="store_true",
                    help="print only the per-workgroup (one per CU) finish-time summary of the forward "
                         "on the 8K slice and the 32K micro-batches")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first copy 512 MiB device-to-device 3 times (a known-size kernel that "
                         "calibrates the HBM byte counters of a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the per-rank kernel "
              "is the unit; a ring would move K/V between GPUs over RCCL). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch

    from variable_length_attention_amd import ops, synth

    torch.cuda.set_device(0)
    if args.cu_timeline:
        print(json.dumps({"cu_timeline": cu_timeline(torch, ops, synth)}), flush=True)
        return 0
    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.sample:
        print(json.dumps(run_sample(torch, ops, synth, args.sample, args.steps)), flush=True)
        return 0
    w = synth.packed_slice_8k()
    q, k, v = synth.varlen_tensors(w)
    cu = synth.cu_seqlens(w.lengths)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    cug = torch.from_numpy(cu).cuda()
    out = torch.empty_like(qg)
    lse = torch.empty((qg.shape[0], w.H), dtype=torch.float32, device="cuda")
    flops = sum(ops.hdp_seq_flops(s, w.H, w.D) for s in w.lengths)

    def step():
        ops.hdp_attn_varlen_fwd(qg, kg, vg, cug, w.scale, out=out, lse=lse)

    clock = settle_clock(step, torch, args.settle_ms)
    t = timed_launches(step, args.steps, args.warmup, torch)
    ms_step, ms_kernel = t["ms_step"], t["mean_ms"]
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    mhz = ops.hdp_probe_clock()
    clock["mfma_clock_mhz_after"] = round(mhz, 1)
    clock["note"] = ("untimed launches of the same step for settle_ms before the warm-up steps, so that "
                     "the timed steps run at the steady clock; mfma_clock_mhz_after is the shader clock "
                     "measured right after the timed steps under back-to-back MFMAs on every CU")
    result = {
        "metric": "varlen attn TFLOP/s on 8K-token packed slice; % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "packed_slice_8k: one rank's 8192-token slice, %d causal sequences "
                               "%s, H=32 Hkv=8 D=128 bf16, forward" % (len(w.lengths), w.lengths),
                   "tokens": int(cu[-1]), "n_seq": len(w.lengths), "gflop": round(flops / 1e9, 3),
                   "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": load_traffic(), "kernel_us": round(ms_kernel * 1e3, 2),
                     "launch": us_stats(t),
                     "peak_at_measured_clock": round(PEAK_BF16_TFLOPS * mhz / NOMINAL_MHZ, 1),
                     "frac_at_measured_clock": round(achieved / (PEAK_BF16_TFLOPS * mhz / NOMINAL_MHZ), 4)},
        "clock": clock,
    }
    if not args.no_detail:
        result["detail"] = detail_rows(torch, ops, synth)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, cu)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
