// Internal interface between the C ABI layer (api.cpp) and the kernel translation units.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace hdp {

// Work-queue counters: one per XCD queue plus a completion counter, each on its own 128-byte
// line, in two sets (the backward kernel drains two queues one after the other; set 1 has no
// completion counter of its own).  The last workgroup of a launch resets them, so they are
// zero between launches.
constexpr int kQueueStride = 32;                 // ints between counters
constexpr int kMaxQueues = 8;                    // one queue per XCD
constexpr int kCounterSetInts = (kMaxQueues + 1) * kQueueStride;
constexpr int kCounterInts = 2 * kCounterSetInts;

struct FwdArgs {
    const uint16_t* q;      // [rows][H][D] bf16
    const uint16_t* k;      // [keys][Hkv][D] bf16
    const uint16_t* v;
    const int32_t* cu;      // varlen: n_seq + 1 entries (device); chunk mode: unused
    int32_t n_seq;
    int32_t H, Hkv;
    float scale_log2;       // scale * log2(e)
    void* out;              // varlen: bf16 [T][H][D]; chunk: fp32 [Lq][H][D]
    float* lse;             // [rows][H]
    // chunk mode
    int32_t Lq, Lk;
    int32_t delta;          // q_offset - kv_offset clamped to [-Lq, Lk] (same visibility)
    int32_t causal;
    // scheduling
    int* counters;          // kCounterInts ints, zero on entry
    int32_t hpw;            // query heads per workgroup item (1, 2 or 4)
    int32_t nqueues;        // 8 (one per XCD) or 1
    // chunk-merge mode: out / lse are the running o_acc / lse_acc (read and written); out_bf16
    // is null or receives the merged result as bf16 [Lq][H][D]
    void* out_bf16;
    // measurement: null, or kTraceWords words per workgroup (real-time counter at start and
    // end, items processed, unused)
    long long* trace;
    // measurement: null, or item_slots records of kItemTraceWords words per workgroup, one per
    // item of its first item_slots (real-time counter at the item's start, when its first loads
    // had landed and when its last step was done; its 32-key units)
    long long* item_trace;
    int32_t item_slots;
};

constexpr int kTraceWords = 4;
constexpr int kItemTraceWords = 4;

struct F32Args {
    const float* q;
    const float* k;
    const float* v;
    const int32_t* cu;
    int32_t n_seq;
    int32_t H, Hkv, D;
    float scale_log2;
    float* out;
    float* lse;
};

struct MergeArgs {
    float* o_acc;
    float* lse_acc;
    const float* o_part;
    const float* lse_part;
    uint16_t* out_bf16;     // may be null
    int64_t rows;           // L * H
    int32_t D;
};

struct BwdArgs {
    const uint16_t* q;      // [T][H][D] bf16
    const uint16_t* k;      // [T][Hkv][D]
    const uint16_t* v;
    const uint16_t* out;    // forward output [T][H][D]
    const float* lse;       // forward lse [T][H]
    const uint16_t* dout;   // [T][H][D]
    const int32_t* cu;
    int32_t n_seq;
    int32_t T;              // caller's row count: every sequence is clamped to it
    int32_t H, Hkv;
    float scale;
    float scale_log2;
    float* rowvals;         // [H][T][2] workspace written by the row-values pass: pairs of
                            // lse * log2(e) and delta = rowsum(dO * out), rows of one head contiguous
    uint16_t* dq;           // varlen: bf16 [T][H][D]
    uint16_t* dk;           // varlen: bf16 [T][Hkv][D]
    uint16_t* dv;
    // chunk mode: q/out/dout/lse are the slice [Lq], k/v the chunk [Lk]; the results are added
    // to fp32 accumulators (dq_acc [Lq][H][D], dk_acc / dv_acc [Lk][Hkv][D])
    int32_t Lq, Lk;
    int32_t dpos;           // q_offset - kv_offset clamped to [-Lq, Lk] (same visibility)
    int32_t causal;
    float* dq_acc;
    float* dk_acc;
    float* dv_acc;
    int* counters;
    int32_t hpw;            // query heads per dQ item
    int32_t nqueues_q;      // queues of the dQ kernel (8 or 1)
    int32_t nqueues_kv;     // queues of the dK/dV kernel (8 or 1)
    // measurement: null, or kTraceWords words per workgroup (real-time counter at its start,
    // when it left the dK/dV queue and at its end; unused)
    long long* trace;
};

// Launchers (return hipSuccess or the launch error).  `grid` is the persistent grid size.
hipError_t launch_fwd_varlen(const FwdArgs& a, int D, int grid, hipStream_t s);
hipError_t launch_fwd_chunk(const FwdArgs& a, int D, int grid, hipStream_t s);
hipError_t launch_fwd_chunk_merge(const FwdArgs& a, int D, int grid, hipStream_t s);
hipError_t launch_fwd_f32(const F32Args& a, hipStream_t s);
hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t s);
// Writes n zero ints at p with a kernel (not a memset node, so the call may be recorded into a
// graph that is replayed).
hipError_t launch_fill_zero(int* p, int n, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, int D, int grid, hipStream_t s);

// The packed backward's host side, shared by the entry point that owns its workspace and the
// one that uses a fixed scratch: argument checks (a status; HDP_OK also for the no-op sizes),
// then the two launches with the given queue counters (zero on entry) and row-value workspace
// (2 * T * H floats).
int check_varlen_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                     const void* dout, const int32_t* cu_seqlens, int32_t n_seq, int32_t T, int32_t H,
                     int32_t Hkv, int32_t D, float scale, const void* dq, const void* dk, const void* dv);
int launch_varlen_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                      const void* dout, const int32_t* cu_seqlens, int32_t n_seq, int32_t T, int32_t H,
                      int32_t Hkv, int32_t D, float scale, void* dq, void* dk, void* dv, int* counters,
                      float* rowvals, int cus, hipStream_t stream);
hipError_t launch_bwd_chunk(const BwdArgs& a, int D, int grid, hipStream_t s);

}  // namespace hdp
