// Forward attention on gfx950 (CDNA4): bf16 MFMA, fp32 accumulation, online softmax.
//
// One kernel serves both forms of a rank's work (research digest "ByteScale: Communication-
// Efficient Scaling of LLM Training with a 2048K Context Length on 16384 GPUs"):
//   * varlen: many short sequences packed back to back, each attending only to itself under a
//     causal mask (digest §3.1-§3.2, §4);
//   * chunk: one slice of a long sequence against one key/value chunk of a ring step, with
//     global positions (digest §3.2); the output is the normalised fp32 partial plus its lse.
//
// Layout of the work.  A workgroup of 4 waves takes one item = (sequence, head block, query
// tile group).  With 4 or more query heads per key/value head, the 4 waves are 4 query heads
// that share one key/value head, so every K/V tile staged in LDS feeds 4 heads.  Each wave owns
// 64 query rows of one head, held as the B operand of v_mfma_f32_32x32x16_bf16:
//     S^T (keys x rows) = K (keys x D) * Q^T (D x rows)
//     O^T (D x rows)   += V^T (D x keys) * P^T (keys x rows)
// In this orientation every lane holds whole query rows, so the row max and row sum are
// in-lane reductions plus one swap between the two half-waves, and the softmax output P^T is
// already in the B-operand layout of the second product.  V^T is read from row-major LDS with
// the gfx950 transposing read ds_read_b64_tr_b16.  K and V tiles of 64 keys are double
// buffered in LDS; the next tile's global loads are in flight while the current one computes.
//
// Softmax uses exp2 with scale*log2(e) folded into one FMA, and a lazy running max: the
// accumulator is rescaled only when some row's max grows by more than 2^8, which keeps every
// P <= 256 (exact arithmetic is unchanged because the same reference max is used for the
// numerator and the denominator).
//
// Scheduling.  The kernel is persistent (one workgroup per CU).  Items are popped from a queue
// in order of decreasing cost, where the cost of a query tile is the number of key tiles it
// visits (the tile form of the O(s^2) cost of hdp_seq_flops): longest-processing-time first, so
// short items fill the gaps at the end instead of idling CUs.  With 8 head blocks there is one
// queue per XCD and head block b is served only by the XCD b mod 8, so each K/V head's tiles
// stay in one XCD's L2.  The order is decoded on the device from cu_seqlens, without a
// planning launch.
#include "hdp_internal.h"

namespace hdp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 64;      // two 32-row MFMA column tiles
constexpr int kNT = 2;
constexpr int kBN = 64;               // keys per LDS stage: two 32-key MFMA row tiles
constexpr float kLazy = 8.0f;         // rescale threshold, log2 units
constexpr float kLn2 = 0.693147180559945309f;

template <int D>
struct Cfg {
    static constexpr int kPitch = D + 8;                   // bf16 per LDS row (16-byte pad)
    static constexpr int kTile = kBN * kPitch;             // bf16 per K or V stage
    static constexpr int kChunks = D / 8;                  // 16-byte chunks per key row
    static constexpr int kLoads = kBN * kChunks / kThreads;
    static constexpr int kKS = D / 16;                     // k-steps of the score product
    static constexpr int kMT = D / 32;                     // D tiles of the value product
};

struct Item {
    int64_t qbase;   // packed row of query position 0
    int64_t kbase;   // packed row of key position 0
    int32_t s;       // query rows
    int32_t sk;      // keys
    int32_t hb;      // head block
    int32_t tg;      // query tile group
};

__device__ inline float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline int wave_sum(int x) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
__device__ inline int wave_max(int x) {
    for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
    return x;
}
__device__ inline uint32_t pack_bf16x2(float a, float b) {
    __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Sequence i clamped to [0, Tc]: start and length.
__device__ inline void seq_span(const int32_t* cu, int i, int Tc, int& a, int& len) {
    int s0 = min(max(cu[i], 0), Tc);
    int s1 = min(max(cu[i + 1], s0), Tc);
    a = s0;
    len = s1 - s0;
}

// Sum over sequences of max(0, ceil(len/W) - c), evaluated by one wave.
__device__ int levels_above(const int32_t* cu, int n_seq, int Tc, int W, int c, int lane) {
    int acc = 0;
    for (int i = lane; i < n_seq; i += 64) {
        int a, len;
        seq_span(cu, i, Tc, a, len);
        int nq = (len + W - 1) / W;
        acc += max(0, nq - c);
    }
    return wave_sum(acc);
}

template <int D, int MODE>
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(FwdArgs args) {
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][C::kTile];
    __shared__ int s_item[8];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;

    const int H = args.H, Hkv = args.Hkv;
    const int G = H / Hkv;
    const int hpw = args.hpw;
    const int qpw = 4 / hpw;
    const int W = kRowsPerWave * qpw;          // query rows per item
    const int nhb = H / hpw;
    const int nq_queues = args.nqueues;
    const int queue = blockIdx.x % nq_queues;
    const int nhbq = nhb / nq_queues;          // head blocks per queue
    const int64_t q_stride = (int64_t)H * D;
    const int64_t kv_stride = (int64_t)Hkv * D;

    // ---- per-launch totals (wave 0 only) ----
    int total = 0, maxc = 0, Tc = 0;
    if (wave == 0) {
        if (MODE == 0) {
            Tc = max(args.cu[args.n_seq], 0);
            int sum = 0, mx = 0;
            for (int i = lane; i < args.n_seq; i += 64) {
                int a, len;
                seq_span(args.cu, i, Tc, a, len);
                int nq = (len + W - 1) / W;
                sum += nq;
                mx = max(mx, nq);
            }
            total = wave_sum(sum) * nhbq;
            maxc = wave_max(mx);
        } else {
            total = ((args.Lq + W - 1) / W) * nhbq;
        }
    }

    for (;;) {
        // ---- pop and decode the next item (wave 0) ----
        if (wave == 0) {
            int k = 0;
            if (lane == 0) k = atomicAdd(&args.counters[queue * kQueueStride], 1);
            k = __shfl(k, 0);
            if (k >= total) {
                if (lane == 0) s_item[0] = -1;
            } else if (MODE == 0) {
                int lo = 1, hi = maxc;   // smallest level c with levels_above(c) * nhbq <= k
                while (lo < hi) {
                    int mid = (lo + hi) >> 1;
                    if (levels_above(args.cu, args.n_seq, Tc, W, mid, lane) * nhbq <= k) hi = mid;
                    else lo = mid + 1;
                }
                const int c = lo;
                const int j = k - levels_above(args.cu, args.n_seq, Tc, W, c, lane) * nhbq;
                int r = j / nhbq;
                const int hbq = j % nhbq;
                int seq = -1;
                for (int i0 = 0; i0 < args.n_seq && seq < 0; i0 += 64) {
                    int i = i0 + lane;
                    bool ok = false;
                    if (i < args.n_seq) {
                        int a, len;
                        seq_span(args.cu, i, Tc, a, len);
                        ok = (len + W - 1) / W >= c;
                    }
                    uint64_t m = __ballot(ok);
                    int cnt = __popcll(m);
                    if (r < cnt) {
                        int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
                        uint64_t hit = __ballot(ok && below == r);
                        seq = i0 + (int)__builtin_ctzll(hit);
                    } else {
                        r -= cnt;
                    }
                }
                if (seq < 0) {                 // cannot happen for k < total; stop safely
                    if (lane == 0) s_item[0] = -1;
                } else if (lane == 0) {
                    int a, len;
                    seq_span(args.cu, seq, Tc, a, len);
                    s_item[0] = a;
                    s_item[1] = len;
                    s_item[2] = queue + nq_queues * hbq;
                    s_item[3] = c - 1;
                }
            } else {
                if (lane == 0) {
                    const int nq = (args.Lq + W - 1) / W;
                    s_item[0] = 0;
                    s_item[1] = args.Lq;
                    s_item[2] = queue + nq_queues * (k % nhbq);
                    s_item[3] = nq - 1 - k / nhbq;
                }
            }
        }
        __syncthreads();
        if (s_item[0] < 0) break;
        Item it;
        it.qbase = s_item[0];
        it.kbase = MODE == 0 ? it.qbase : 0;
        it.s = s_item[1];
        it.sk = MODE == 0 ? it.s : args.Lk;
        it.hb = s_item[2];
        it.tg = s_item[3];
        const int64_t qpos0 = MODE == 0 ? 0 : args.q_offset;
        const int64_t kpos0 = MODE == 0 ? 0 : args.kv_offset;
        const bool causal = MODE == 0 ? true : (args.causal != 0);

        const int head = it.hb * hpw + (wave % hpw);
        const int g = (it.hb * hpw) / G;
        const int t = it.tg * qpw + wave / hpw;       // this wave's query tile
        const int r_lo = t * kRowsPerWave;
        const int r_hi = min(r_lo + kRowsPerWave, it.s) - 1;
        const bool wave_rows = r_lo < it.s;
        // key tiles the workgroup visits
        const int wg_rmax = min(it.s, (it.tg + 1) * W) - 1;
        int64_t jmax = it.sk - 1;
        if (causal) jmax = min(jmax, qpos0 + wg_rmax - kpos0);
        const int n_tiles = (wg_rmax < 0 || jmax < 0) ? 0 : (int)(jmax / kBN) + 1;

        // ---- Q^T fragments in registers ----
        u32x4 qf[kNT][C::kKS];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const int row = r_lo + nt * 32 + l32;
            const bool ok = row < it.s;
            const uint16_t* qp = args.q + (it.qbase + row) * q_stride + (int64_t)head * D + half * 8;
#pragma unroll
            for (int ks = 0; ks < C::kKS; ++ks)
                qf[nt][ks] = ok ? *(const u32x4*)(qp + ks * 16) : u32x4{0, 0, 0, 0};
        }

        f32x16 o[C::kMT][kNT];
#pragma unroll
        for (int mt = 0; mt < C::kMT; ++mt)
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) o[mt][nt] = f32x16{};
        float m[kNT], l[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) { m[nt] = -INFINITY; l[nt] = 0.f; }

        // ---- K/V tile staging ----
        u32x4 kreg[C::kLoads], vreg[C::kLoads];
        auto load_tile = [&](int jt) {
#pragma unroll
            for (int u = 0; u < C::kLoads; ++u) {
                const int c = tid + u * kThreads;
                const int key = c / C::kChunks, part = c % C::kChunks;
                const int j = jt * kBN + key;
                if (j < it.sk) {
                    const int64_t off = (it.kbase + j) * kv_stride + (int64_t)g * D + part * 8;
                    kreg[u] = *(const u32x4*)(args.k + off);
                    vreg[u] = *(const u32x4*)(args.v + off);
                } else {
                    kreg[u] = u32x4{0, 0, 0, 0};
                    vreg[u] = u32x4{0, 0, 0, 0};
                }
            }
        };
        auto store_tile = [&](int buf) {
#pragma unroll
            for (int u = 0; u < C::kLoads; ++u) {
                const int c = tid + u * kThreads;
                const int key = c / C::kChunks, part = c % C::kChunks;
                *(u32x4*)&smem[buf][0][key * C::kPitch + part * 8] = kreg[u];
                *(u32x4*)&smem[buf][1][key * C::kPitch + part * 8] = vreg[u];
            }
        };

        if (n_tiles > 0) {
            load_tile(0);
            store_tile(0);
        }
        __syncthreads();

        // per-lane constant parts of the transposing V reads
        const int gidx = lane >> 4;                  // 16-lane group
        const int tr_row = 4 * (gidx >> 1) + ((lane & 15) >> 2);
        const int tr_col = 16 * (gidx & 1) + 4 * (lane & 3);

        for (int jt = 0; jt < n_tiles; ++jt) {
            const int buf = jt & 1;
            if (jt + 1 < n_tiles) load_tile(jt + 1);
            const int64_t j0 = (int64_t)jt * kBN;
            bool active = wave_rows;
            if (causal && kpos0 + j0 > qpos0 + r_hi) active = false;
            if (active) {
                const uint16_t* Ks = smem[buf][0];
                const uint16_t* Vs = smem[buf][1];
                // Two 32-key sub-tiles per stage; each runs score, softmax and value products.
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    const int64_t js = j0 + kt * 32;
                    if (causal && kpos0 + js > qpos0 + r_hi) continue;
                    const bool full = (js + 31 < it.sk) && (!causal || kpos0 + js + 31 <= qpos0 + r_lo);
                    // S^T = K Q^T
                    f32x16 sacc[kNT];
#pragma unroll
                    for (int nt = 0; nt < kNT; ++nt) sacc[nt] = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < C::kKS; ++ks) {
                        const u32x4 araw = *(const u32x4*)&Ks[(kt * 32 + l32) * C::kPitch + ks * 16 + half * 8];
                        const bf16x8 a = __builtin_bit_cast(bf16x8, araw);
#pragma unroll
                        for (int nt = 0; nt < kNT; ++nt)
                            sacc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                a, __builtin_bit_cast(bf16x8, qf[nt][ks]), sacc[nt], 0, 0, 0);
                    }
                    if (!full) {
#pragma unroll
                        for (int nt = 0; nt < kNT; ++nt) {
                            const int64_t qpos = qpos0 + r_lo + nt * 32 + l32;
#pragma unroll
                            for (int i = 0; i < 16; ++i) {
                                const int64_t j = js + 8 * (i >> 2) + 4 * half + (i & 3);
                                const bool vis = j < it.sk && (!causal || kpos0 + j <= qpos);
                                if (!vis) sacc[nt][i] = -INFINITY;
                            }
                        }
                    }
                    // online softmax (rows live in lanes)
                    float tmax[kNT];
                    bool need = false;
#pragma unroll
                    for (int nt = 0; nt < kNT; ++nt) {
                        float mx = -INFINITY;
#pragma unroll
                        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[nt][i]);
                        mx = xhalf_max(mx);
                        tmax[nt] = mx * args.scale_log2;
                        need |= tmax[nt] > m[nt] + kLazy;
                    }
                    if (__ballot(need)) {
#pragma unroll
                        for (int nt = 0; nt < kNT; ++nt) {
                            const float mn = fmaxf(m[nt], tmax[nt]);
                            const float alpha = (m[nt] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[nt] - mn);
                            m[nt] = mn;
                            l[nt] *= alpha;
#pragma unroll
                            for (int mt = 0; mt < C::kMT; ++mt) o[mt][nt] *= alpha;
                        }
                    }
                    bf16x8 pb[kNT][2];
#pragma unroll
                    for (int nt = 0; nt < kNT; ++nt) {
                        const float mb = (m[nt] == -INFINITY) ? 0.f : m[nt];
                        float ls = 0.f;
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[nt][i], args.scale_log2, -mb));
                            ls += p;
                            pb[nt][i >> 3][i & 7] = (__bf16)p;
                        }
                        l[nt] += ls;
                    }
                    // O^T += V^T P^T
#pragma unroll
                    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
                        for (int mt = 0; mt < C::kMT; ++mt) {
                            const int row0 = kt * 32 + 16 * ks2 + tr_row;
                            const uint16_t* p0 = &Vs[row0 * C::kPitch + mt * 32 + tr_col];
                            const uint16_t* p1 = p0 + 8 * C::kPitch;
                            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
                            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
                            bf16x8 a;
                            a.lo = __builtin_bit_cast(__bf16 __attribute__((ext_vector_type(4))), lo);
                            a.hi = __builtin_bit_cast(__bf16 __attribute__((ext_vector_type(4))), hi);
#pragma unroll
                            for (int nt = 0; nt < kNT; ++nt)
                                o[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[nt][ks2], o[mt][nt], 0, 0, 0);
                        }
                }
            }
            if (jt + 1 < n_tiles) store_tile(buf ^ 1);
            __syncthreads();
        }

        // ---- epilogue ----
        if (wave_rows) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                const float lt = xhalf_sum(l[nt]);
                const float inv = lt > 0.f ? 1.f / lt : 0.f;
                const float mb = (m[nt] == -INFINITY) ? 0.f : m[nt];
                const float lse = lt > 0.f ? (mb + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
                const int row = r_lo + nt * 32 + l32;
                if (row < it.s) {
                    const int64_t orow = (it.qbase + row) * (int64_t)H + head;
                    if (MODE == 0) {
                        uint16_t* op = (uint16_t*)args.out + orow * D;
#pragma unroll
                        for (int mt = 0; mt < C::kMT; ++mt)
#pragma unroll
                            for (int a4 = 0; a4 < 4; ++a4) {
                                const int d0 = mt * 32 + 8 * a4 + 4 * half;
                                u32x2 w;
                                w[0] = pack_bf16x2(o[mt][nt][4 * a4 + 0] * inv, o[mt][nt][4 * a4 + 1] * inv);
                                w[1] = pack_bf16x2(o[mt][nt][4 * a4 + 2] * inv, o[mt][nt][4 * a4 + 3] * inv);
                                *(u32x2*)(op + d0) = w;
                            }
                    } else {
                        float* op = (float*)args.out + orow * D;
#pragma unroll
                        for (int mt = 0; mt < C::kMT; ++mt)
#pragma unroll
                            for (int a4 = 0; a4 < 4; ++a4) {
                                const int d0 = mt * 32 + 8 * a4 + 4 * half;
                                float4 w = make_float4(o[mt][nt][4 * a4 + 0] * inv, o[mt][nt][4 * a4 + 1] * inv,
                                                       o[mt][nt][4 * a4 + 2] * inv, o[mt][nt][4 * a4 + 3] * inv);
                                *(float4*)(op + d0) = w;
                            }
                    }
                    if (half == 0) args.lse[orow] = lse;
                }
            }
        }
        __syncthreads();
    }

    // ---- the last workgroup out resets the queue counters for the next launch ----
    if (tid == 0) {
        __threadfence();
        int* done = &args.counters[kMaxQueues * kQueueStride];
        if (atomicAdd(done, 1) == (int)gridDim.x - 1) {
            for (int qi = 0; qi < kMaxQueues; ++qi) atomicExch(&args.counters[qi * kQueueStride], 0);
            atomicExch(done, 0);
            __threadfence();
        }
    }
}

}  // namespace

hipError_t launch_fwd_varlen(const FwdArgs& a, int D, int grid, hipStream_t s) {
    if (D == 128) hipLaunchKernelGGL((fwd_kernel<128, 0>), dim3(grid), dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((fwd_kernel<64, 0>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fwd_chunk(const FwdArgs& a, int D, int grid, hipStream_t s) {
    if (D == 128) hipLaunchKernelGGL((fwd_kernel<128, 1>), dim3(grid), dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((fwd_kernel<64, 1>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace hdp
