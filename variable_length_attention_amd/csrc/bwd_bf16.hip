// Backward of packed variable-length causal attention on gfx950: bf16 MFMA, fp32 accumulation.
//
// The pages show forward and backward time per training step (research digest "ByteScale:
// Communication-Efficient Scaling of LLM Training with a 2048K Context Length on 16384 GPUs",
// §5, Figure 18) but print no formulas; this is the chain rule of the forward kernel.  With
// P = exp(scale*S - lse) (lse from the forward), delta = rowsum(dO * O):
//     dV = P^T dO,   dS = P * (dO V^T - delta),   dQ = scale dS K,   dK = scale dS^T Q,
// dK and dV summed over the query heads that share a key/value head.
//
// Two kernels, no atomics, so every gradient is deterministic:
//   * dQ kernel, query-major (one item = 32 rows x 4 query heads, a wave per head):
//         S^T = K Q^T,  dP^T = V dO^T,  dS^T = P^T * (dP^T - delta),  dQ^T += K^T dS^T.
//     Rows live in lanes (as in the forward), so lse and delta are one value per lane and dS^T
//     is already the B operand of the last product; K^T comes from transposing LDS reads.  It
//     also computes delta from dO and O and writes it for the second kernel.
//   * dK/dV kernel, key-major (one item = 128 keys of one key/value head, 32 keys per wave):
//         S = Q K^T,  dP = dO V^T,  dS = P * (dP - delta),  dV += P^T dO,  dK += dS^T Q,
//     for every 32-row unit of the sequence at or after the keys and every query head of the
//     group.  Keys live in lanes, so P and dS are directly the A operands of the two
//     accumulating products; dO and Q come from transposing LDS reads.
// The score products are recomputed in both kernels (seven products per pair instead of five):
// the price of keeping dS out of memory and dQ free of atomics.
#include "device_common.h"

namespace hdp {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kUnit = 32;          // keys (dQ kernel) or rows (dK/dV kernel) per step
constexpr int kStage = 64;         // keys per K/V stage of the dQ kernel
constexpr int kStages = 3;
constexpr int kKeyTile = 128;      // keys per dK/dV item

template <int D>
struct Cfg {
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = D / 8;
    static constexpr int kRowsPerBlock = 64 / kChunks;           // rows per 1 KB wave load
    static constexpr int kKS = D / 16;
    static constexpr int kMT = D / 32;
};

// ---- LDS tile helpers: rows of D bf16, 16-byte slots XOR-swizzled by swz(row) ----

// A-operand fragment rows (row = tile row of this lane): 8 bf16 of d = ks*16 + half*8.
template <int D>
__device__ inline void lds_rows_frag(const unsigned char* tile, int row, int half, u32x4 (&f)[Cfg<D>::kKS]) {
#pragma unroll
    for (int ks = 0; ks < Cfg<D>::kKS; ++ks) {
        const int slot = (2 * ks + half) ^ swz(row);
        f[ks] = *(const u32x4*)(tile + row * Cfg<D>::kRowBytes + slot * 16);
    }
}

// Transposed fragments over 32 tile rows starting at r_base: for k-step ks2 and D tile mt, lane l
// receives 8 values of column mt*32 + l%32 from the rows 16*ks2 + 8*(i/4) + 4*(l/32) + (i%4),
// the row order in which an MFMA accumulator holds its rows (see the forward kernel).
template <int D>
__device__ inline void lds_cols_frag(const unsigned char* tile, int r_base, int lane, bf16x8 (&f)[2][Cfg<D>::kMT]) {
    const int gidx = lane >> 4;
    const int tr_row = 4 * (gidx >> 1) + ((lane & 15) >> 2);
    const int tr_col = 16 * (gidx & 1) + 4 * (lane & 3);
    const int tr_sub = (lane & 1) * 8;
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int mt = 0; mt < Cfg<D>::kMT; ++mt) {
            const int chunk = (mt * 32 + tr_col) >> 3;
            const int r0 = r_base + 16 * ks2 + tr_row;
            const int r1 = r0 + 8;
            const unsigned char* p0 = tile + r0 * Cfg<D>::kRowBytes + ((chunk ^ swz(r0)) << 4) + tr_sub;
            const unsigned char* p1 = tile + r1 * Cfg<D>::kRowBytes + ((chunk ^ swz(r1)) << 4) + tr_sub;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
            f[ks2][mt].lo = __builtin_bit_cast(bf16x4, lo);
            f[ks2][mt].hi = __builtin_bit_cast(bf16x4, hi);
        }
}

// Issues one 1 KB wave load of rows [blk*kRowsPerBlock, +kRowsPerBlock) of a tile: row r of the
// tile is global row base_row + r (clamped to last_row) at src + row * stride (elements).
template <int D>
__device__ inline void dma_block(const uint16_t* src, int64_t stride, int64_t base_row, int last_row,
                                 int blk, int lane, unsigned char* tile) {
    const int row = blk * Cfg<D>::kRowsPerBlock + lane / Cfg<D>::kChunks;
    const int slot = lane % Cfg<D>::kChunks;
    const int chunk = slot ^ swz(row);
    const int64_t r = base_row + min(row, last_row);
    __builtin_amdgcn_global_load_lds(src + r * stride + chunk * 8, (lds_void*)(tile + blk * 1024), 16, 0, 0);
}

__device__ inline void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// =============================================================================================
// dQ kernel
// =============================================================================================
template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(BwdArgs args) {
    using C = Cfg<D>;
    constexpr int kTile = kStage * C::kRowBytes;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages][2][kTile];
    __shared__ int s_item[4];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int H = args.H, Hkv = args.Hkv, G = H / Hkv;
    const int hpw = args.hpw;
    const int W = kUnit * (kWaves / hpw);          // query rows per item
    const int nhbq = (H / hpw) / args.nqueues_q;
    const int queue = blockIdx.x % args.nqueues_q;
    const int64_t q_stride = (int64_t)H * D, kv_stride = (int64_t)Hkv * D;
    const float c2 = args.scale_log2;

    QueuePlan plan{0, 0, 0, 0};
    if (wave == 0) plan = queue_plan(args.cu, args.n_seq, W, nhbq, lane, args.T);

    for (;;) {
        if (wave == 0) {
            int k = 0;
            if (lane == 0) k = atomicAdd(&args.counters[queue * kQueueStride], 1);
            k = __shfl(k, 0);
            int a = 0, len = 0, hbq = 0, c = 0;
            const bool ok = k < plan.total &&
                            queue_decode(args.cu, args.n_seq, plan, W, nhbq, k, lane, a, len, hbq, c);
            if (lane == 0) {
                s_item[0] = ok ? a : -1;
                s_item[1] = len;
                s_item[2] = queue + args.nqueues_q * hbq;
                s_item[3] = c - 1;
            }
        }
        __syncthreads();
        const int a0 = __builtin_amdgcn_readfirstlane(s_item[0]);
        if (a0 < 0) break;
        const int64_t base = a0;
        const int s = __builtin_amdgcn_readfirstlane(s_item[1]);
        const int hb = __builtin_amdgcn_readfirstlane(s_item[2]);
        const int tg = __builtin_amdgcn_readfirstlane(s_item[3]);
        const int head = hb * hpw + (wave % hpw);
        const int g = (hb * hpw) / G;
        const int r_lo = tg * W + (wave / hpw) * kUnit;
        const int row = r_lo + l32;                      // this lane's query row
        const bool row_ok = row < s;
        const int wg_rmax = min(s, (tg + 1) * W) - 1;
        const int n_units = wg_rmax / kUnit + 1;         // keys 0 .. wg_rmax
        const int n_stages = (n_units + 1) / 2;

        // Q^T and dO^T fragments, delta = rowsum(dO * O), lse in log2 units
        u32x4 qf[C::kKS], df[C::kKS];
        float dpart = 0.f;
        {
            const int64_t off = (base + row) * q_stride + (int64_t)head * D + half * 8;
#pragma unroll
            for (int ks = 0; ks < C::kKS; ++ks) {
                qf[ks] = row_ok ? *(const u32x4*)(args.q + off + ks * 16) : u32x4{0, 0, 0, 0};
                df[ks] = row_ok ? *(const u32x4*)(args.dout + off + ks * 16) : u32x4{0, 0, 0, 0};
                const u32x4 of = row_ok ? *(const u32x4*)(args.out + off + ks * 16) : u32x4{0, 0, 0, 0};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dpart = __builtin_fmaf(bf16_lo(df[ks][e]), bf16_lo(of[e]), dpart);
                    dpart = __builtin_fmaf(bf16_hi(df[ks][e]), bf16_hi(of[e]), dpart);
                }
            }
        }
        const float delta = xhalf_sum(dpart);
        const float lse2 = row_ok ? args.lse[(base + row) * H + head] * kLog2e : 0.f;
        if (row_ok && half == 0) args.delta[(base + row) * H + head] = delta;

        f32x16 acc[C::kMT];
#pragma unroll
        for (int mt = 0; mt < C::kMT; ++mt) acc[mt] = f32x16{};

        auto load_stage = [&](int st) {
            unsigned char* kb = smem[st % kStages][0];
            unsigned char* vb = smem[st % kStages][1];
            constexpr int kBlocks = kStage / C::kRowsPerBlock;      // per tile
#pragma unroll
            for (int i = 0; i < kBlocks / kWaves; ++i) {
                const int blk = wave * (kBlocks / kWaves) + i;
                dma_block<D>(args.k + (int64_t)g * D, kv_stride, base + st * kStage, s - 1 - st * kStage, blk, lane, kb);
                dma_block<D>(args.v + (int64_t)g * D, kv_stride, base + st * kStage, s - 1 - st * kStage, blk, lane, vb);
            }
        };
        load_stage(0);
        if (n_stages > 1) load_stage(1);
        wait_vm0();
        __syncthreads();

        for (int u = 0; u < n_units; ++u) {
            if (u & 1) {
                wait_vm0();
                __syncthreads();
                const int st = (u + 3) >> 1;
                if (st < n_stages) load_stage(st);
            }
            const int j0 = u * kUnit;
            if (j0 > r_lo + kUnit - 1) continue;             // every key after every row
            const unsigned char* kb = smem[(u >> 1) % kStages][0];
            const unsigned char* vb = smem[(u >> 1) % kStages][1];
            const int trow = (u & 1) * 32;
            u32x4 kf[C::kKS], vf[C::kKS];
            lds_rows_frag<D>(kb, trow + l32, half, kf);
            lds_rows_frag<D>(vb, trow + l32, half, vf);
            f32x16 S = f32x16{}, dP = f32x16{};
#pragma unroll
            for (int ks = 0; ks < C::kKS; ++ks) {
                S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[ks]),
                                                            __builtin_bit_cast(bf16x8, qf[ks]), S, 0, 0, 0);
                dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf[ks]),
                                                             __builtin_bit_cast(bf16x8, df[ks]), dP, 0, 0, 0);
            }
            // key jl = 8*(i/4) + 4*half + (i%4) of the unit is visible iff j0 + jl <= row
            const bool full = j0 + kUnit - 1 <= r_lo;
            const int li = row - j0 - 4 * half;
            bf16x8 ds[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const bool vis = full || (8 * (i >> 2) + (i & 3)) <= li;
                const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(S[i], c2, -lse2)) : 0.f;
                ds[i >> 3][i & 7] = (__bf16)(p * (dP[i] - delta));
            }
            bf16x8 kt[2][C::kMT];
            lds_cols_frag<D>(kb, trow, lane, kt);
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
                for (int mt = 0; mt < C::kMT; ++mt)
                    acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[ks2][mt], ds[ks2], acc[mt], 0, 0, 0);
        }

        // dQ = scale * acc; lane holds d = mt*32 + 8*a4 + 4*half + (0..3) of its row
        if (row_ok) {
            uint16_t* op = args.dq + ((base + row) * H + head) * D;
#pragma unroll
            for (int mt = 0; mt < C::kMT; ++mt)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int d0 = mt * 32 + 8 * a4 + 4 * half;
                    u32x2 w;
                    w[0] = pack_bf16x2(acc[mt][4 * a4 + 0] * args.scale, acc[mt][4 * a4 + 1] * args.scale);
                    w[1] = pack_bf16x2(acc[mt][4 * a4 + 2] * args.scale, acc[mt][4 * a4 + 3] * args.scale);
                    *(u32x2*)(op + d0) = w;
                }
        }
        __syncthreads();
    }
    if (tid == 0) queue_finish(args.counters);
}

// =============================================================================================
// dK/dV kernel
// =============================================================================================
template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs args) {
    using C = Cfg<D>;
    constexpr int kTile = kUnit * C::kRowBytes;     // 32 rows of Q or dO
    constexpr int kBlocks = kUnit / C::kRowsPerBlock;   // 1 KB loads per tile
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages][2][kTile];
    __shared__ int s_item[4];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int H = args.H, Hkv = args.Hkv, G = H / Hkv;
    const int nhbq = Hkv / args.nqueues_kv;
    const int queue = blockIdx.x % args.nqueues_kv;
    const int64_t q_stride = (int64_t)H * D, kv_stride = (int64_t)Hkv * D;
    const float c2 = args.scale_log2;

    QueuePlan plan{0, 0, 0, 0};
    if (wave == 0) plan = queue_plan(args.cu, args.n_seq, kKeyTile, nhbq, lane, args.T);

    for (;;) {
        if (wave == 0) {
            int k = 0;
            if (lane == 0) k = atomicAdd(&args.counters[queue * kQueueStride], 1);
            k = __shfl(k, 0);
            int a = 0, len = 0, hbq = 0, c = 0;
            const bool ok = k < plan.total &&
                            queue_decode(args.cu, args.n_seq, plan, kKeyTile, nhbq, k, lane, a, len, hbq, c);
            if (lane == 0) {
                s_item[0] = ok ? a : -1;
                s_item[1] = len;
                s_item[2] = queue + args.nqueues_kv * hbq;
                // level c = tiles from this one to the end: earlier key tiles see more rows
                s_item[3] = (len + kKeyTile - 1) / kKeyTile - c;
            }
        }
        __syncthreads();
        const int a0 = __builtin_amdgcn_readfirstlane(s_item[0]);
        if (a0 < 0) break;
        const int64_t base = a0;
        const int s = __builtin_amdgcn_readfirstlane(s_item[1]);
        const int g = __builtin_amdgcn_readfirstlane(s_item[2]);
        const int kt = __builtin_amdgcn_readfirstlane(s_item[3]);
        const int kj0 = kt * kKeyTile + wave * kUnit;   // this wave's first key
        const int key = kj0 + l32;                      // this lane's key (B-operand column)

        // K^T and V^T fragments of this wave's 32 keys
        u32x4 kf[C::kKS], vf[C::kKS];
        {
            const bool ok = key < s;
            const int64_t off = (base + key) * kv_stride + (int64_t)g * D + half * 8;
#pragma unroll
            for (int ks = 0; ks < C::kKS; ++ks) {
                kf[ks] = ok ? *(const u32x4*)(args.k + off + ks * 16) : u32x4{0, 0, 0, 0};
                vf[ks] = ok ? *(const u32x4*)(args.v + off + ks * 16) : u32x4{0, 0, 0, 0};
            }
        }
        f32x16 dk[C::kMT], dv[C::kMT];
#pragma unroll
        for (int mt = 0; mt < C::kMT; ++mt) { dk[mt] = f32x16{}; dv[mt] = f32x16{}; }

        // stages: (row unit ru, head hh) for ru = ru0 .. n_ru-1, hh = 0 .. G-1
        const int ru0 = kt * (kKeyTile / kUnit);
        const int n_ru = (s + kUnit - 1) / kUnit;
        const int n_stages = (n_ru - ru0) * G;
        auto load_stage = [&](int st) {
            const int ru = ru0 + st / G, hh = st % G;
            const int head = g * G + hh;
            unsigned char* qb = smem[st % kStages][0];
            unsigned char* db = smem[st % kStages][1];
#pragma unroll
            for (int i = 0; i < kBlocks / kWaves; ++i) {
                const int blk = wave * (kBlocks / kWaves) + i;
                dma_block<D>(args.q + (int64_t)head * D, q_stride, base + ru * kUnit, s - 1 - ru * kUnit, blk, lane, qb);
                dma_block<D>(args.dout + (int64_t)head * D, q_stride, base + ru * kUnit, s - 1 - ru * kUnit, blk, lane, db);
            }
        };
        // lse (log2 units) and delta of the lane's 16 accumulator rows 8*(i/4) + 4*half + (i%4)
        auto load_rowvals = [&](int st, float (&l2)[16], float (&dl)[16]) {
            const int ru = ru0 + st / G, hh = st % G;
            const int head = g * G + hh;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = ru * kUnit + 8 * (i >> 2) + 4 * half + (i & 3);
                const int rc = min(r, s - 1);
                const int64_t o = (base + rc) * H + head;
                l2[i] = args.lse[o] * kLog2e;
                dl[i] = args.delta[o];
            }
        };

        if (n_stages > 0) {
            load_stage(0);
            if (n_stages > 1) load_stage(1);
        }
        float l2[16], dl[16];
        if (n_stages > 0) load_rowvals(0, l2, dl);
        wait_vm0();
        __syncthreads();

        for (int st = 0; st < n_stages; ++st) {
            if (st + 2 < n_stages) load_stage(st + 2);
            const int ru = ru0 + st / G;
            const int r0 = ru * kUnit;
            if (kj0 <= r0 + kUnit - 1) {                 // some key of this wave is visible
                const unsigned char* qb = smem[st % kStages][0];
                const unsigned char* db = smem[st % kStages][1];
                u32x4 qr[C::kKS], dr[C::kKS];
                lds_rows_frag<D>(qb, l32, half, qr);
                lds_rows_frag<D>(db, l32, half, dr);
                f32x16 S = f32x16{}, dP = f32x16{};
#pragma unroll
                for (int ks = 0; ks < C::kKS; ++ks) {
                    S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qr[ks]),
                                                                __builtin_bit_cast(bf16x8, kf[ks]), S, 0, 0, 0);
                    dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, dr[ks]),
                                                                 __builtin_bit_cast(bf16x8, vf[ks]), dP, 0, 0, 0);
                }
                // S[i]: row r0 + 8*(i/4) + 4*half + (i%4), key = this lane's key
                const bool full = kj0 + kUnit - 1 <= r0 && r0 + kUnit <= s;
                bf16x8 pb[2], sb[2];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = r0 + 8 * (i >> 2) + 4 * half + (i & 3);
                    const bool vis = full || (key <= r && r < s);
                    const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(S[i], c2, -l2[i])) : 0.f;
                    pb[i >> 3][i & 7] = (__bf16)p;
                    sb[i >> 3][i & 7] = (__bf16)(p * (dP[i] - dl[i]));
                }
                bf16x8 dt[2][C::kMT], qt[2][C::kMT];
                lds_cols_frag<D>(db, 0, lane, dt);
                lds_cols_frag<D>(qb, 0, lane, qt);
#pragma unroll
                for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
                    for (int mt = 0; mt < C::kMT; ++mt) {
                        dv[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pb[ks2], dt[ks2][mt], dv[mt], 0, 0, 0);
                        dk[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sb[ks2], qt[ks2][mt], dk[mt], 0, 0, 0);
                    }
            }
            if (st + 1 < n_stages) load_rowvals(st + 1, l2, dl);
            wait_vm0();
            __syncthreads();
        }

        // dK = scale * dk, dV = dv; accumulator element i of D tile mt is key
        // kj0 + 8*(i/4) + 4*half + (i%4), column mt*32 + l32
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kr = kj0 + 8 * (i >> 2) + 4 * half + (i & 3);
            if (kr < s) {
                uint16_t* kp = args.dk + ((base + kr) * Hkv + g) * D + l32;
                uint16_t* vp = args.dv + ((base + kr) * Hkv + g) * D + l32;
#pragma unroll
                for (int mt = 0; mt < C::kMT; ++mt) {
                    kp[mt * 32] = __builtin_bit_cast(uint16_t, (__bf16)(dk[mt][i] * args.scale));
                    vp[mt * 32] = __builtin_bit_cast(uint16_t, (__bf16)dv[mt][i]);
                }
            }
        }
        __syncthreads();
    }
    if (tid == 0) queue_finish(args.counters);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int D, int grid, hipStream_t s) {
    if (D == 128) {
        hipLaunchKernelGGL((bwd_dq_kernel<128>), dim3(grid), dim3(kThreads), 0, s, a);
        hipLaunchKernelGGL((bwd_dkdv_kernel<128>), dim3(grid), dim3(kThreads), 0, s, a);
    } else {
        hipLaunchKernelGGL((bwd_dq_kernel<64>), dim3(grid), dim3(kThreads), 0, s, a);
        hipLaunchKernelGGL((bwd_dkdv_kernel<64>), dim3(grid), dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace hdp
