// C ABI of the per-rank attention library: argument checks, per-device workspace, FLOP cost
// model and kernel launches.  Every check happens on the host before any HIP call.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "hdp_attn.h"
#include "hdp_internal.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Library state is kept per (device, stream): each stream has its own work-queue counters and
// its own backward workspace, so calls that run concurrently on different streams of one device
// never share them.  Everything is allocated stream-ordered on the stream of the call that first
// needs it (no device-wide synchronisation); the counters are cleared by a fill kernel on that
// stream, and the kernels leave them at zero when they finish.
struct StreamState {
    int* counters = nullptr;   // hdp::kCounterInts ints, zero between launches
    void* ws = nullptr;        // backward workspace (lse in log2 units and delta, per row and head)
    size_t ws_bytes = 0;
};

struct DeviceState {
    int cus = 0;
    std::map<hipStream_t, StreamState> streams;
};

std::mutex g_mu;
std::map<int, DeviceState> g_dev;

// The calling thread's current device and the state of `stream` on it, created on first use.
int stream_state(hipStream_t stream, int* cus, StreamState** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return HDP_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    DeviceState& ds = g_dev[dev];
    if (ds.cus == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return HDP_ERR_HIP;
        ds.cus = n;
    }
    StreamState& st = ds.streams[stream];
    if (st.counters == nullptr) {
        int* c = nullptr;
        if (hipMallocAsync((void**)&c, sizeof(int) * hdp::kCounterInts, stream) != hipSuccess) return HDP_ERR_HIP;
        if (hdp::launch_fill_zero(c, hdp::kCounterInts, stream) != hipSuccess) {
            (void)hipFreeAsync(c, stream);
            return HDP_ERR_HIP;
        }
        st.counters = c;
    }
    *cus = ds.cus;
    *out = &st;
    return HDP_OK;
}

// Grows a stream's backward workspace to at least `bytes`, stream-ordered: the old buffer is
// released after the work already queued on the stream and the new one is ready before the
// work queued next.  A set HDP_TEST_FAIL_ALLOC makes every growth fail (error-path tests).
int ensure_workspace(StreamState* st, size_t bytes, hipStream_t stream) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (st->ws_bytes >= bytes) return HDP_OK;
    if (std::getenv("HDP_TEST_FAIL_ALLOC") != nullptr) return HDP_ERR_HIP;
    if (st->ws != nullptr) {
        if (hipFreeAsync(st->ws, stream) != hipSuccess) return HDP_ERR_HIP;
        st->ws = nullptr;
        st->ws_bytes = 0;
    }
    void* p = nullptr;
    if (hipMallocAsync(&p, bytes, stream) != hipSuccess) return HDP_ERR_HIP;
    st->ws = p;
    st->ws_bytes = bytes;
    return HDP_OK;
}

// Optional host-side check of cu_seqlens (a set HDP_VALIDATE): copies it to the host, which
// synchronises the stream, and requires cu[0] = 0, non-decreasing entries and cu[n] <= T
// (T < 0: no bound).  Off by default: the hot path never waits on the host.
int validate_cu(const int32_t* cu, int32_t n_seq, int64_t T, hipStream_t stream) {
    if (std::getenv("HDP_VALIDATE") == nullptr) return HDP_OK;
    std::vector<int32_t> h((size_t)n_seq + 1);
    if (hipMemcpyAsync(h.data(), cu, sizeof(int32_t) * h.size(), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return HDP_ERR_HIP;
    if (h[0] != 0) return HDP_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n_seq; ++i)
        if (h[i + 1] < h[i]) return HDP_ERR_INVALID_ARG;
    if (T >= 0 && h[n_seq] > T) return HDP_ERR_INVALID_ARG;
    return HDP_OK;
}

bool head_dim_ok(int D) { return D == 64 || D == 128; }

// Head counts above 65535 would let an output tile's byte range (32 rows of H heads) reach the
// kernels' drop offset for bounds-checked stores.
int check_heads(int32_t H, int32_t Hkv, int32_t D) {
    if (H <= 0 || Hkv <= 0 || D <= 0 || H % Hkv != 0) return HDP_ERR_INVALID_ARG;
    if (!head_dim_ok(D)) return HDP_ERR_UNSUPPORTED;
    if (H > 65535) return HDP_ERR_OVERFLOW;
    return HDP_OK;
}

// Query heads per workgroup item: 4 when a key/value head serves a multiple of 4 query heads.
int heads_per_item(int32_t H, int32_t Hkv) {
    const int G = H / Hkv;
    return (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
}

// Forward workgroup trace (measurement helper): a device buffer and its capacity in workgroups.
std::atomic<long long*> g_trace{nullptr};
std::atomic<int> g_trace_cap{0};
// Per-item forward timeline (measurement helper): buffer, capacity in workgroups, items each.
std::atomic<long long*> g_itrace{nullptr};
std::atomic<int> g_itrace_cap{0};
std::atomic<int> g_itrace_slots{0};

void schedule(int cus, const StreamState* st, int32_t H, int32_t Hkv, hdp::FwdArgs& a, int& grid) {
    a.hpw = heads_per_item(H, Hkv);
    grid = cus;
    const int nhb = H / a.hpw;
    a.nqueues = (nhb % hdp::kMaxQueues == 0 && grid % hdp::kMaxQueues == 0) ? hdp::kMaxQueues : 1;
    a.counters = st->counters;
    a.trace = g_trace_cap.load() >= grid ? g_trace.load() : nullptr;
    a.item_trace = g_itrace_cap.load() >= grid ? g_itrace.load() : nullptr;
    a.item_slots = a.item_trace != nullptr ? g_itrace_slots.load() : 0;
    if (a.item_slots <= 0) a.item_trace = nullptr;
}

// sum_{r=0}^{n-1} clamp(a + r, 0, cap), exactly.
unsigned __int128 sum_clamped(int64_t a, int64_t n, int64_t cap) {
    if (n <= 0 || cap <= 0) return 0;
    // r in [r1, r2): 0 < a + r < cap contributes a + r; r in [r2, n): contributes cap.
    int64_t r1 = std::max<int64_t>(0, 1 - a);
    int64_t r2 = std::max<int64_t>(0, cap - a);
    r1 = std::min(r1, n);
    r2 = std::min(std::max(r2, r1), n);
    const __int128 cnt = (__int128)(r2 - r1);
    const __int128 first = (__int128)a + r1;
    const __int128 last = (__int128)a + r2 - 1;
    __int128 s = cnt > 0 ? (first + last) * cnt / 2 : 0;
    s += (__int128)(n - r2) * cap;
    return (unsigned __int128)s;
}

uint64_t flops_from_pairs(unsigned __int128 pairs, int32_t H, int32_t D, int32_t pass) {
    uint64_t per;
    if (pass == HDP_PASS_FWD) per = 4ull * (uint64_t)D;
    else if (pass == HDP_PASS_BWD) per = 10ull * (uint64_t)D;
    else if (pass == HDP_PASS_FWD_BWD) per = 14ull * (uint64_t)D;
    else return UINT64_MAX;
    const unsigned __int128 f = pairs * (unsigned __int128)(uint64_t)H * per;
    if (f > (unsigned __int128)UINT64_MAX) return UINT64_MAX;
    return (uint64_t)f;
}

}  // namespace

namespace hdp {

int check_varlen_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                     const void* dout, const int32_t* cu_seqlens, int32_t n_seq, int32_t T, int32_t H,
                     int32_t Hkv, int32_t D, float scale, const void* dq, const void* dk, const void* dv) {
    if (n_seq < 0 || T < 0) return HDP_ERR_INVALID_ARG;
    if (int st = check_heads(H, Hkv, D)) return st;
    if (!std::isfinite(scale) || !(scale > 0.f)) return HDP_ERR_INVALID_ARG;
    if (n_seq == 0 || T == 0) return HDP_OK;
    if (!q || !k || !v || !out || !lse || !dout || !cu_seqlens || !dq || !dk || !dv)
        return HDP_ERR_INVALID_ARG;
    if ((int64_t)T * H > (int64_t)INT32_MAX) return HDP_ERR_OVERFLOW;
    return HDP_OK;
}

int launch_varlen_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                      const void* dout, const int32_t* cu_seqlens, int32_t n_seq, int32_t T, int32_t H,
                      int32_t Hkv, int32_t D, float scale, void* dq, void* dk, void* dv, int* counters,
                      float* rowvals, int cus, hipStream_t stream) {
    BwdArgs a{};
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.out = (const uint16_t*)out;
    a.lse = lse;
    a.dout = (const uint16_t*)dout;
    a.cu = cu_seqlens;
    a.n_seq = n_seq;
    a.T = T;
    a.H = H;
    a.Hkv = Hkv;
    a.scale = scale;
    a.scale_log2 = scale * kLog2e;
    a.rowvals = rowvals;
    a.dq = (uint16_t*)dq;
    a.dk = (uint16_t*)dk;
    a.dv = (uint16_t*)dv;
    a.counters = counters;
    a.hpw = heads_per_item(H, Hkv);
    const int grid = cus;
    const bool q8 = (H / a.hpw) % kMaxQueues == 0 && grid % kMaxQueues == 0;
    const bool kv8 = Hkv % kMaxQueues == 0 && grid % kMaxQueues == 0;
    a.nqueues_q = q8 ? kMaxQueues : 1;
    a.nqueues_kv = kv8 ? kMaxQueues : 1;
    a.trace = g_trace_cap.load() >= grid ? g_trace.load() : nullptr;
    return launch_bwd(a, D, grid, stream) == hipSuccess ? HDP_OK : HDP_ERR_HIP;
}

}  // namespace hdp

extern "C" {

const char* hdp_status_string(int status) {
    switch (status) {
        case HDP_OK: return "HDP_OK";
        case HDP_ERR_INVALID_ARG: return "HDP_ERR_INVALID_ARG: invalid argument";
        case HDP_ERR_UNSUPPORTED: return "HDP_ERR_UNSUPPORTED: unsupported head dim (64 or 128)";
        case HDP_ERR_HIP: return "HDP_ERR_HIP: HIP launch or allocation failed";
        case HDP_ERR_OVERFLOW: return "HDP_ERR_OVERFLOW: size does not fit the index types";
        case HDP_ERR_SCRATCH_LIMIT:
            return "HDP_ERR_SCRATCH_LIMIT: 4096 + 8*T*H bytes exceed the fixed scratch of the "
                   "no-allocation entry point (HDP_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown hdp status";
    }
}

uint64_t hdp_seq_flops(int64_t s, int32_t H, int32_t D, int32_t causal, int32_t pass) {
    if (pass != HDP_PASS_FWD && pass != HDP_PASS_BWD && pass != HDP_PASS_FWD_BWD) return UINT64_MAX;
    if (s <= 0 || H <= 0 || D <= 0) return 0;
    const unsigned __int128 us = (unsigned __int128)s;
    const unsigned __int128 pairs = causal ? us * (us + 1) / 2 : us * us;
    return flops_from_pairs(pairs, H, D, pass);
}

uint64_t hdp_chunk_flops(int32_t Lq, int32_t Lk, int64_t q_offset, int64_t kv_offset,
                         int32_t causal, int32_t H, int32_t D, int32_t pass) {
    if (pass != HDP_PASS_FWD && pass != HDP_PASS_BWD && pass != HDP_PASS_FWD_BWD) return UINT64_MAX;
    if (Lq <= 0 || Lk <= 0 || H <= 0 || D <= 0) return 0;
    unsigned __int128 pairs;
    if (causal) {
        // row r sees keys j with kv_offset + j <= q_offset + r: clamp(q_offset - kv_offset + 1 + r, 0, Lk)
        const __int128 a = (__int128)q_offset - kv_offset + 1;
        if (a > (__int128)INT64_MAX / 2 || a < (__int128)INT64_MIN / 2) return UINT64_MAX;
        pairs = sum_clamped((int64_t)a, Lq, Lk);
    } else {
        pairs = (unsigned __int128)Lq * (unsigned __int128)Lk;
    }
    return flops_from_pairs(pairs, H, D, pass);
}

int hdp_attn_varlen_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                        int32_t n_seq, int32_t H, int32_t Hkv, int32_t D, float scale,
                        void* out, float* lse, hipStream_t stream) {
    if (n_seq < 0) return HDP_ERR_INVALID_ARG;
    if (int st = check_heads(H, Hkv, D)) return st;
    if (!std::isfinite(scale) || !(scale > 0.f)) return HDP_ERR_INVALID_ARG;
    if (n_seq == 0) return HDP_OK;
    if (!q || !k || !v || !cu_seqlens || !out || !lse) return HDP_ERR_INVALID_ARG;
    if (int rc = validate_cu(cu_seqlens, n_seq, -1, stream)) return rc;
    int cus = 0;
    StreamState* st = nullptr;
    if (int rc = stream_state(stream, &cus, &st)) return rc;
    hdp::FwdArgs a{};
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.cu = cu_seqlens;
    a.n_seq = n_seq;
    a.H = H;
    a.Hkv = Hkv;
    a.scale_log2 = scale * kLog2e;
    a.out = out;
    a.lse = lse;
    a.causal = 1;
    int grid = 0;
    schedule(cus, st, H, Hkv, a, grid);
    return hdp::launch_fwd_varlen(a, D, grid, stream) == hipSuccess ? HDP_OK : HDP_ERR_HIP;
}

int hdp_attn_varlen_fwd_f32(const float* q, const float* k, const float* v,
                            const int32_t* cu_seqlens, int32_t n_seq, int32_t H, int32_t Hkv,
                            int32_t D, float scale, float* out, float* lse, hipStream_t stream) {
    if (n_seq < 0) return HDP_ERR_INVALID_ARG;
    if (int st = check_heads(H, Hkv, D)) return st;
    if (!std::isfinite(scale) || !(scale > 0.f)) return HDP_ERR_INVALID_ARG;
    if (n_seq == 0) return HDP_OK;
    if (!q || !k || !v || !cu_seqlens || !out || !lse) return HDP_ERR_INVALID_ARG;
    if (H > 65535) return HDP_ERR_OVERFLOW;
    if (int rc = validate_cu(cu_seqlens, n_seq, -1, stream)) return rc;
    hdp::F32Args a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.cu = cu_seqlens;
    a.n_seq = n_seq;
    a.H = H;
    a.Hkv = Hkv;
    a.D = D;
    a.scale_log2 = scale * kLog2e;
    a.out = out;
    a.lse = lse;
    return hdp::launch_fwd_f32(a, stream) == hipSuccess ? HDP_OK : HDP_ERR_HIP;
}

}  // extern "C"

namespace {

// The ring step's forward, either writing the partial (o, lse) or merging it into them.
int chunk_forward(const void* q_slice, int32_t Lq, const void* k_chunk, const void* v_chunk, int32_t Lk,
                  int64_t q_offset, int64_t kv_offset, int32_t causal, int32_t H, int32_t Hkv, int32_t D,
                  float scale, float* o, float* lse, void* out_bf16, bool merge, hipStream_t stream) {
    if (Lq < 0 || Lk < 0 || q_offset < 0 || kv_offset < 0) return HDP_ERR_INVALID_ARG;
    if (int st = check_heads(H, Hkv, D)) return st;
    if (!std::isfinite(scale) || !(scale > 0.f)) return HDP_ERR_INVALID_ARG;
    if (q_offset > INT64_MAX / 4 || kv_offset > INT64_MAX / 4) return HDP_ERR_OVERFLOW;
    if (Lq > (1 << 30) || Lk > (1 << 30)) return HDP_ERR_OVERFLOW;
    if (Lq == 0) return HDP_OK;
    if (!q_slice || !o || !lse) return HDP_ERR_INVALID_ARG;
    if (Lk > 0 && (!k_chunk || !v_chunk)) return HDP_ERR_INVALID_ARG;
    int cus = 0;
    StreamState* st = nullptr;
    if (int rc = stream_state(stream, &cus, &st)) return rc;
    hdp::FwdArgs a{};
    a.q = (const uint16_t*)q_slice;
    a.k = (const uint16_t*)k_chunk;
    a.v = (const uint16_t*)v_chunk;
    a.H = H;
    a.Hkv = Hkv;
    a.scale_log2 = scale * kLog2e;
    a.out = o;
    a.lse = lse;
    a.out_bf16 = out_bf16;
    a.Lq = Lq;
    a.Lk = Lk;
    // Key j is visible to row r iff j <= (q_offset - kv_offset) + r; for 0 <= j < Lk and
    // 0 <= r < Lq that only depends on the difference clamped to [-Lq, Lk].
    const int64_t d = q_offset - kv_offset;
    a.delta = (int32_t)std::max<int64_t>(-(int64_t)Lq, std::min<int64_t>(d, Lk));
    a.causal = causal ? 1 : 0;
    int grid = 0;
    schedule(cus, st, H, Hkv, a, grid);
    const hipError_t e = merge ? hdp::launch_fwd_chunk_merge(a, D, grid, stream) : hdp::launch_fwd_chunk(a, D, grid, stream);
    return e == hipSuccess ? HDP_OK : HDP_ERR_HIP;
}

}  // namespace

extern "C" {

int hdp_attn_chunk_partial(const void* q_slice, int32_t Lq, const void* k_chunk,
                           const void* v_chunk, int32_t Lk, int64_t q_offset, int64_t kv_offset,
                           int32_t causal, int32_t H, int32_t Hkv, int32_t D, float scale,
                           float* o_partial, float* lse, hipStream_t stream) {
    return chunk_forward(q_slice, Lq, k_chunk, v_chunk, Lk, q_offset, kv_offset, causal, H, Hkv, D, scale,
                         o_partial, lse, nullptr, false, stream);
}

int hdp_attn_chunk_merge(const void* q_slice, int32_t Lq, const void* k_chunk, const void* v_chunk,
                         int32_t Lk, int64_t q_offset, int64_t kv_offset, int32_t causal, int32_t H,
                         int32_t Hkv, int32_t D, float scale, float* o_acc, float* lse_acc,
                         void* out_bf16, hipStream_t stream) {
    return chunk_forward(q_slice, Lq, k_chunk, v_chunk, Lk, q_offset, kv_offset, causal, H, Hkv, D, scale,
                         o_acc, lse_acc, out_bf16, true, stream);
}

int hdp_lse_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                  int32_t L, int32_t H, int32_t D, void* out_bf16, hipStream_t stream) {
    if (L < 0 || H <= 0 || D <= 0) return HDP_ERR_INVALID_ARG;
    if (!head_dim_ok(D)) return HDP_ERR_UNSUPPORTED;
    if (L == 0) return HDP_OK;
    if (!o_acc || !lse_acc || !o_part || !lse_part) return HDP_ERR_INVALID_ARG;
    const int64_t rows = (int64_t)L * H;
    if (rows / (256 / (D / 4)) + 1 > INT32_MAX) return HDP_ERR_OVERFLOW;
    hdp::MergeArgs a{};
    a.o_acc = o_acc;
    a.lse_acc = lse_acc;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.out_bf16 = (uint16_t*)out_bf16;
    a.rows = rows;
    a.D = D;
    return hdp::launch_lse_merge(a, stream) == hipSuccess ? HDP_OK : HDP_ERR_HIP;
}

int hdp_attn_varlen_bwd(const void* q, const void* k, const void* v, const void* out,
                        const float* lse, const void* dout, const int32_t* cu_seqlens,
                        int32_t n_seq, int32_t T, int32_t H, int32_t Hkv, int32_t D,
                        float scale, void* dq, void* dk, void* dv, hipStream_t stream) {
    if (int rc = hdp::check_varlen_bwd(q, k, v, out, lse, dout, cu_seqlens, n_seq, T, H, Hkv, D, scale, dq, dk, dv))
        return rc;
    if (n_seq == 0 || T == 0) return HDP_OK;
    if (int rc = validate_cu(cu_seqlens, n_seq, T, stream)) return rc;
    int cus = 0;
    StreamState* st = nullptr;
    if (int rc = stream_state(stream, &cus, &st)) return rc;
    if (int rc = ensure_workspace(st, 2 * sizeof(float) * (size_t)T * (size_t)H, stream)) return rc;
    return hdp::launch_varlen_bwd(q, k, v, out, lse, dout, cu_seqlens, n_seq, T, H, Hkv, D, scale, dq, dk, dv,
                                  st->counters, (float*)st->ws, cus, stream);
}

int hdp_attn_chunk_bwd(const void* q_slice, int32_t Lq, const void* k_chunk, const void* v_chunk,
                       int32_t Lk, int64_t q_offset, int64_t kv_offset, int32_t causal,
                       int32_t H, int32_t Hkv, int32_t D, float scale, const void* out,
                       const float* lse, const void* dout, float* dq_acc, float* dk_acc,
                       float* dv_acc, hipStream_t stream) {
    if (Lq < 0 || Lk < 0 || q_offset < 0 || kv_offset < 0) return HDP_ERR_INVALID_ARG;
    if (int st = check_heads(H, Hkv, D)) return st;
    if (!std::isfinite(scale) || !(scale > 0.f)) return HDP_ERR_INVALID_ARG;
    if (q_offset > INT64_MAX / 4 || kv_offset > INT64_MAX / 4) return HDP_ERR_OVERFLOW;
    if (Lq > (1 << 30) || Lk > (1 << 30)) return HDP_ERR_OVERFLOW;
    if ((int64_t)Lq * H > (int64_t)INT32_MAX) return HDP_ERR_OVERFLOW;
    if (Lq == 0 || Lk == 0) return HDP_OK;
    if (!q_slice || !k_chunk || !v_chunk || !out || !lse || !dout || !dq_acc || !dk_acc || !dv_acc)
        return HDP_ERR_INVALID_ARG;
    int cus = 0;
    StreamState* st = nullptr;
    if (int rc = stream_state(stream, &cus, &st)) return rc;
    if (int rc = ensure_workspace(st, 2 * sizeof(float) * (size_t)Lq * (size_t)H, stream)) return rc;
    hdp::BwdArgs a{};
    a.q = (const uint16_t*)q_slice;
    a.k = (const uint16_t*)k_chunk;
    a.v = (const uint16_t*)v_chunk;
    a.out = (const uint16_t*)out;
    a.lse = lse;
    a.dout = (const uint16_t*)dout;
    a.T = Lq;
    a.H = H;
    a.Hkv = Hkv;
    a.scale = scale;
    a.scale_log2 = scale * kLog2e;
    a.rowvals = (float*)st->ws;
    a.Lq = Lq;
    a.Lk = Lk;
    // visibility depends only on q_offset - kv_offset clamped to [-Lq, Lk] (as in the forward)
    const int64_t d = q_offset - kv_offset;
    a.dpos = (int32_t)std::max<int64_t>(-(int64_t)Lq, std::min<int64_t>(d, Lk));
    a.causal = causal ? 1 : 0;
    a.dq_acc = dq_acc;
    a.dk_acc = dk_acc;
    a.dv_acc = dv_acc;
    a.counters = st->counters;
    a.hpw = heads_per_item(H, Hkv);
    const int grid = cus;
    const bool q8 = (H / a.hpw) % hdp::kMaxQueues == 0 && grid % hdp::kMaxQueues == 0;
    const bool kv8 = Hkv % hdp::kMaxQueues == 0 && grid % hdp::kMaxQueues == 0;
    a.nqueues_q = q8 ? hdp::kMaxQueues : 1;
    a.nqueues_kv = kv8 ? hdp::kMaxQueues : 1;
    a.trace = g_trace_cap.load() >= grid ? g_trace.load() : nullptr;
    return hdp::launch_bwd_chunk(a, D, grid, stream) == hipSuccess ? HDP_OK : HDP_ERR_HIP;
}

int hdp_set_trace(long long* trace, int32_t capacity) {
    if (capacity < 0 || (capacity > 0 && trace == nullptr)) return HDP_ERR_INVALID_ARG;
    g_trace_cap.store(0);
    g_trace.store(capacity > 0 ? trace : nullptr);
    g_trace_cap.store(capacity);
    return HDP_OK;
}

int hdp_set_item_trace(long long* items, int32_t capacity, int32_t slots) {
    if (capacity < 0 || slots < 0 || (capacity > 0 && (items == nullptr || slots == 0))) return HDP_ERR_INVALID_ARG;
    g_itrace_cap.store(0);
    g_itrace.store(capacity > 0 ? items : nullptr);
    g_itrace_slots.store(capacity > 0 ? slots : 0);
    g_itrace_cap.store(capacity);
    return HDP_OK;
}

int hdp_release_workspace(void) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return HDP_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    auto itr = g_dev.find(dev);
    if (itr == g_dev.end()) return HDP_OK;
    // every stream's queued work ends before its memory goes back
    if (hipDeviceSynchronize() != hipSuccess) return HDP_ERR_HIP;
    int rc = HDP_OK;
    for (auto& kv : itr->second.streams) {
        if (kv.second.ws && hipFreeAsync(kv.second.ws, nullptr) != hipSuccess) rc = HDP_ERR_HIP;
        if (kv.second.counters && hipFreeAsync(kv.second.counters, nullptr) != hipSuccess) rc = HDP_ERR_HIP;
    }
    g_dev.erase(itr);
    if (hipDeviceSynchronize() != hipSuccess) rc = HDP_ERR_HIP;
    return rc;
}

}  // extern "C"
