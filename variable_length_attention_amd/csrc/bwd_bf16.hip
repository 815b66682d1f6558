// Backward of packed variable-length causal attention on gfx950: bf16 MFMA, fp32 accumulation.
//
// The pages show forward and backward time per training step (research digest "ByteScale:
// Communication-Efficient Scaling of LLM Training with a 2048K Context Length on 16384 GPUs",
// §5, Figure 18) but print no formulas; this is the chain rule of the forward kernel.  With
// P = exp(scale*S - lse) (lse from the forward), delta = rowsum(dO * O):
//     dV = P^T dO,   dS = P * (dO V^T - delta),   dQ = scale dS K,   dK = scale dS^T Q,
// dK and dV summed over the query heads that share a key/value head.
//
// A row-values pass and one persistent kernel with two bodies, no atomics on gradients, so
// every gradient is deterministic:
//   * row values: lse in log2 units and delta = rowsum(dO * O) of every (row, head), written
//     head-major as pairs ([H][T][2]: the rows of one head contiguous) for the dK/dV body;
//   * dK/dV body, key-major (one item = 128 keys of one key/value head, 32 keys per wave):
//         S = Q K^T,  dP = dO V^T,  dS = P * (dP - delta),  dV += P^T dO,  dK += dS^T Q,
//     for every 32-row unit of the sequence at or after the keys and every query head of the
//     group.  Keys live in lanes, so P and dS are directly the A operands of the two
//     accumulating products; dO and Q come from transposing LDS reads.  Software-pipelined
//     like the forward (see the body);
//   * dQ body, query-major (one item = 32 rows x 4 query heads, a wave per head):
//         S^T = K Q^T,  dP^T = V dO^T,  dS^T = P^T * (dP^T - delta),  dQ^T += K^T dS^T.
//     Rows live in lanes (as in the forward), so lse and delta are one value per lane and dS^T
//     is already the B operand of the last product; K^T comes from transposing LDS reads.
// The kernel drains the dK/dV queue first and the dQ queue after it, so that workgroups left
// without dK/dV items while the largest ones finish take dQ items instead of idling.
// The score products are recomputed in both kernels (seven products per pair instead of five):
// the price of keeping dS out of memory and dQ free of atomics.
#include <algorithm>

#include "device_common.h"

namespace hdp {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kUnit = 32;          // keys (dQ body) or rows (dK/dV body) per step
constexpr int kStage = 64;         // keys per K/V stage of the dQ body
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
    lds_dma16(src + r * stride + chunk * 8, lds_addr(tile + blk * 1024));
}

__device__ inline void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// =============================================================================================
// dQ body
// =============================================================================================
// MODE 0: packed sequences (rows and keys of one sequence, causal); MODE 1: one ring step, the
// slice's rows [Lq] against one chunk's keys [Lk] at a position offset, adding this chunk's
// share of dQ to an fp32 accumulator.
//
// Software-pipelined like the forward, over units of 32 keys: step u issues the dQ product of
// unit u-1 (8 MFMAs) and the S and dP products of unit u+1 (16 MFMAs) around the elementwise
// part of unit u (P = exp2(S c - lse2), dS = P (dP - delta), one element per slot).  K and V
// arrive through direct global->LDS loads in a ring of three 64-key stages; the K and V rows
// for the products of unit u+1 are read two per dQ slot, the transposed K fragments of unit u
// (for the next step) one per two S/dP slots, once the dQ product of unit u-1 is issued.
template <int D>
constexpr int dq_lds_bytes() { return kStages * 2 * kStage * Cfg<D>::kRowBytes + 8 * (int)sizeof(int); }

template <int D, int MODE>
__device__ __attribute__((always_inline)) inline void dq_body(const BwdArgs& args, unsigned char* lds, int* counters) {
    using C = Cfg<D>;
    constexpr int kTile = kStage * C::kRowBytes;
    constexpr int kBPW = kStage / C::kRowsPerBlock / kWaves;   // 1 KB stage loads per wave and tile
    // LDS: kStages ring buffers of [K tile][V tile], then the two item slots
    int* s_item = (int*)(lds + kStages * 2 * kTile);

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
    const bool causal = MODE == 0 ? true : (args.causal != 0);
    const int dpos = MODE == 0 ? 0 : args.dpos;    // query position minus key position

    // per-lane LDS offsets: row fragments (A operand: row l32 of a 32-row unit, slot
    // (2 ks + half) ^ swz), transposed fragments (as the forward's V^T reads), stage loads
    int rofs[4];
    {
        const int t = half ^ swz(l32);
#pragma unroll
        for (int j = 0; j < 4; ++j) rofs[j] = l32 * C::kRowBytes + 16 * ((2 * j) ^ t);
    }
    int tofs[2];
    {
        const int gidx = lane >> 4;
        const int tr_row = 4 * (gidx >> 1) + ((lane & 15) >> 2);
        const int tr_col = 16 * (gidx & 1) + 4 * (lane & 3);
        const int t = (tr_col >> 3) ^ swz(tr_row);
#pragma unroll
        for (int j = 0; j < 2; ++j) tofs[j] = tr_row * C::kRowBytes + 16 * ((4 * j) ^ t) + (lane & 1) * 8;
    }
    // whole-stage loads: this lane's byte offset in each of its 1 KB blocks from the stage's
    // first key row of the head, minus the block's LDS offset that the load instruction's
    // immediate adds back to both addresses (row >= kRowsPerBlock i keeps it >= 0)
    uint32_t voffk[kBPW];
#pragma unroll
    for (int i = 0; i < kBPW; ++i) {
        const int row = (wave * kBPW + i) * C::kRowsPerBlock + lane / C::kChunks;
        const int chunk = (lane % C::kChunks) ^ swz(row);
        voffk[i] = (uint32_t)((row * kv_stride + chunk * 8) * 2) - 1024u * i;
    }
    const uint32_t ring0 = lds_addr(lds);              // LDS byte address of stage buffer 0

    QueuePlan plan{0, 0, 0, 0, 0, 0, 0, 0};
    if (wave == 0) {
        if (MODE == 0) plan = queue_plan(args.cu, args.n_seq, W, nhbq, lane, args.T);
        else plan.total = ((args.Lq + W - 1) / W) * nhbq;
    }
    auto publish = [&](int k, int slot) {
        int a = 0, len = 0, hbq = 0, c = 0;
        bool ok = k < plan.total;
        if (ok) {
            if (MODE == 0) {
                ok = queue_decode(args.cu, args.n_seq, plan, W, nhbq, k, lane, a, len, hbq, c);
            } else {
                len = args.Lq;
                hbq = k % nhbq;
                c = ((args.Lq + W - 1) / W) - k / nhbq;
            }
        }
        if (lane == 0) {
            s_item[4 * slot + 0] = ok ? a : -1;
            s_item[4 * slot + 1] = len;
            s_item[4 * slot + 2] = queue + args.nqueues_q * hbq;
            s_item[4 * slot + 3] = c - 1;
        }
    };
    auto pop = [&]() {
        int k = 0;
        if (lane == 0) k = atomicAdd(&counters[queue * kQueueStride], 1);
        return k;
    };
    if (wave == 0) publish(__builtin_amdgcn_readfirstlane(pop()), 0);
    __syncthreads();

    for (int it = 0;; ++it) {
        const int slot = it & 1;
        const int a0 = __builtin_amdgcn_readfirstlane(s_item[4 * slot + 0]);
        if (a0 < 0) break;
        int k_next = 0;
        const int64_t base = a0;                         // first row (and, packed, first key)
        const int s = __builtin_amdgcn_readfirstlane(s_item[4 * slot + 1]);
        const int sk = MODE == 0 ? s : args.Lk;          // keys
        const int hb = __builtin_amdgcn_readfirstlane(s_item[4 * slot + 2]);
        const int tg = __builtin_amdgcn_readfirstlane(s_item[4 * slot + 3]);
        const int head = hb * hpw + (wave % hpw);
        const int g = (hb * hpw) / G;
        const int r_lo = tg * W + (wave / hpw) * kUnit;
        const int row = r_lo + l32;                      // this lane's query row
        const bool row_ok = row < s;
        const int wg_rmax = min(s, (tg + 1) * W) - 1;
        int jmax = sk - 1;                               // last key any row of the item sees
        if (causal) jmax = min(jmax, wg_rmax + dpos);
        const int n_units = jmax < 0 ? 0 : jmax / kUnit + 1;
        const int n_stages = (n_units + 1) / 2;
        const int64_t kbase = MODE == 0 ? base : 0;

        // stage st (64 keys) into ring buffer buf (= st mod 3); the last stage clamps its rows
        // into the key range
        auto load_stage = [&](int st, int buf) {
            const uint32_t lk = ring0 + (uint32_t)buf * (2 * kTile) + wave * kBPW * 1024;
            const int j0 = st * kStage;
            if (j0 + kStage <= sk) {
                const int64_t sofs = (kbase + j0) * kv_stride + (int64_t)g * D;
                lds_dma16_tiles<kBPW>(args.k + sofs, args.v + sofs, voffk, lk, lk + kTile);
            } else {
#pragma unroll
                for (int i = 0; i < kBPW; ++i) {
                    const int row = (wave * kBPW + i) * C::kRowsPerBlock + lane / C::kChunks;
                    const int chunk = (lane % C::kChunks) ^ swz(row);
                    const int64_t off = (kbase + min(j0 + row, sk - 1)) * kv_stride + (int64_t)g * D + chunk * 8;
                    lds_dma16(args.k + off, lk + 1024 * i);
                    lds_dma16(args.v + off, lk + kTile + 1024 * i);
                }
            }
        };
        if (n_units > 0) {
            load_stage(0, 0);
            if (n_stages > 1) load_stage(1, 1);
        }
        int lbuf = 2;                                    // ring buffer of the next stage load
        int cbuf = 0;                                    // ring buffer of the current unit's stage

        // Q^T and dO^T fragments; lse in log2 units and delta from the row-values pass
        u32x4 qf[C::kKS], df[C::kKS];
        {
            const int64_t off = (base + row) * q_stride + (int64_t)head * D + half * 8;
#pragma unroll
            for (int ks = 0; ks < C::kKS; ++ks) {
                qf[ks] = row_ok ? *(const u32x4*)(args.q + off + ks * 16) : u32x4{0, 0, 0, 0};
                df[ks] = row_ok ? *(const u32x4*)(args.dout + off + ks * 16) : u32x4{0, 0, 0, 0};
            }
        }
        const int Trv = MODE == 0 ? args.T : args.Lq;    // row stride of the lse2/delta planes
        const f32x2 rv = row_ok ? *(const f32x2*)(args.rowvals + 2 * ((int64_t)head * Trv + base + row)) : f32x2{0.f, 0.f};
        const float lse2 = rv[0], delta = rv[1];
        wait_vm0();
        __syncthreads();

        // LDS byte address of the 32 rows of a unit: ring buffer buf, half h of its stage
        auto unit_base = [&](int buf, int h) { return ring0 + (uint32_t)buf * (2 * kTile) + (uint32_t)h * (32 * C::kRowBytes); };
        auto read_rows = [&](uint32_t ub, int kv, u32x4 (&f)[C::kKS]) {
            const uint32_t b = ub + kv * kTile;
            uint32_t a[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) a[j] = lds_add(b, rofs[j]);
#pragma unroll
            for (int ks = 0; ks < C::kKS; ++ks) f[ks] = *(const lds_u32x4*)(uintptr_t)(a[ks & 3] + 128 * (ks >> 2));
        };
        // transposed K fragment (ks2, mt) of the unit at ub; a = per-lane column bases (cols_addr)
        auto cols_addr = [&](uint32_t ub, uint32_t (&a)[2]) {
            a[0] = lds_add(ub, tofs[0]);
            a[1] = lds_add(ub, tofs[1]);
        };
        auto read_col = [&](const uint32_t (&a)[2], int ks2, int mt, bf16x8& f) {
            const uint32_t p0 = a[mt & 1] + 128 * (mt >> 1) + 16 * ks2 * C::kRowBytes;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)p0);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(p0 + 8 * C::kRowBytes));
            f.lo = __builtin_bit_cast(bf16x4, lo);
            f.hi = __builtin_bit_cast(bf16x4, hi);
        };
        // key j of the item is visible to this lane's row iff j <= lim (and the row exists);
        // invisible elements of a unit get S = -inf, so P = 0 and dS = 0
        const int lim = row_ok ? (causal ? min(row + dpos, sk - 1) : sk - 1) : -1;
        auto unit_full = [&](int u) {
            const int j0 = u * kUnit;
            return j0 + kUnit - 1 <= (causal ? min(r_lo + dpos, sk - 1) : sk - 1) && r_lo + kUnit <= s;
        };
        auto apply_mask = [&](int u, f32x16& S) {
            const int li = max(-1, min(lim - u * kUnit, kUnit)) - 4 * half;
#pragma unroll
            for (int i = 0; i < 16; ++i) S[i] = (8 * (i >> 2) + (i & 3)) > li ? -INFINITY : S[i];
        };
        auto stage_turn = [&](int u) {
            wait_vm0();
            __syncthreads();
            const int st = (u + 3) >> 1;
            if (st < n_stages) load_stage(st, lbuf);
            lbuf = lbuf == kStages - 1 ? 0 : lbuf + 1;
        };

        f32x16 acc[C::kMT];
#pragma unroll
        for (int mt = 0; mt < C::kMT; ++mt) acc[mt] = f32x16{};
        bf16x8 kt[2][C::kMT];                           // K^T fragments of the previous unit

        // step u: dQ of u-1 (operands Tp, kt), S/dP of u+1 into Sn/Dn, elementwise of u from
        // Sc/Dc into Tc
        auto step = [&](int u, bool odd, f32x16& Sc, f32x16& Dc, f32x16& Sn, f32x16& Dn,
                        const bf16x8 (&Tp)[2], bf16x8 (&Tc)[2]) {
            if (odd) stage_turn(u);
            u32x4 kf[C::kKS], vf[C::kKS];
            // rows of unit u + 1: the second half of this stage (u even) or the first half of
            // the next (u odd); past the end, unit u again (a harmless re-read)
            const int nbuf = cbuf == kStages - 1 ? 0 : cbuf + 1;
            const uint32_t un_base = u + 1 >= n_units ? unit_base(cbuf, odd) : odd ? unit_base(nbuf, 0) : unit_base(cbuf, 1);
            uint32_t ra[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) ra[j] = lds_add(un_base, rofs[j]);
            __builtin_amdgcn_sched_barrier(0);
            constexpr int kDQ = 2 * C::kMT;              // dQ MFMAs
            constexpr int kSD = 2 * C::kKS;              // S and dP MFMAs
            constexpr int kSlots = kDQ + kSD > 16 ? kDQ + kSD : 16;
            static_assert(kSD == 2 * kDQ, "a transposed fragment every second S/dP slot");
            uint32_t tw[8], ca[2];
            float te = 0.f;
#pragma unroll
            for (int k = 0; k < kSlots; ++k) {
                if (k < kDQ) {
                    // K and V rows of unit u + 1, two reads per dQ slot in the order the S and
                    // dP products use them
#pragma unroll
                    for (int r = 0; r < kSD / kDQ; ++r) {
                        const int j = k * (kSD / kDQ) + r, ks = j >> 1;
                        const uint32_t a = ra[ks & 3] + (j & 1) * kTile + 128 * (ks >> 2);
                        if (j & 1) vf[ks] = *(const lds_u32x4*)(uintptr_t)a;
                        else kf[ks] = *(const lds_u32x4*)(uintptr_t)a;
                    }
                }
                if (k >= kDQ && k < kDQ + kSD && ((k - kDQ) & 1) == 0) {
                    // K^T of unit u for the next step (its dQ products of u - 1 are issued), one
                    // fragment every second S/dP slot in the order the next step uses them
                    const int f = (k - kDQ) >> 1;
                    if (f == 0) cols_addr(unit_base(cbuf, odd), ca);
                    read_col(ca, f / C::kMT, f % C::kMT, kt[f / C::kMT][f % C::kMT]);
                }
                if (k < kDQ) {
                    const int ks2 = k / C::kMT, mt = k % C::kMT;
                    acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[ks2][mt], Tp[ks2], acc[mt], 0, 0, 0);
                } else if (k < kDQ + kSD) {
                    const int j = k - kDQ, ks = j >> 1;
                    if (j == 0) Sn = f32x16{};
                    if (j == 1) Dn = f32x16{};
                    if ((j & 1) == 0) Sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[ks]), __builtin_bit_cast(bf16x8, qf[ks]), Sn, 0, 0, 0);
                    else Dn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf[ks]), __builtin_bit_cast(bf16x8, df[ks]), Dn, 0, 0, 0);
                }
                if (k < 16) {
                    const int i = k;
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(Sc[i], c2, -lse2));
                    const float t = p * (Dc[i] - delta);
                    if (i & 1) {
                        tw[i >> 1] = pack_bf16x2(te, t);
                        asm volatile("" : "+v"(tw[i >> 1]));
                    } else {
                        te = t;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
                Tc[h] = __builtin_bit_cast(bf16x8, u32x4{tw[4 * h], tw[4 * h + 1], tw[4 * h + 2], tw[4 * h + 3]});
            if (u + 1 < n_units && !unit_full(u + 1)) apply_mask(u + 1, Sn);
            if (odd) cbuf = nbuf;
        };

        if (n_units > 0) {
            f32x16 SA, DA, SB, DB;
            bf16x8 TA[2], TB[2];
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
                for (int mt = 0; mt < C::kMT; ++mt) kt[ks2][mt] = bf16x8{};
            TA[0] = bf16x8{};
            TA[1] = bf16x8{};
            {
                u32x4 kf[C::kKS], vf[C::kKS];
                read_rows(unit_base(0, 0), 0, kf);
                read_rows(unit_base(0, 0), 1, vf);
                SA = f32x16{};
                DA = f32x16{};
#pragma unroll
                for (int ks = 0; ks < C::kKS; ++ks) {
                    SA = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[ks]), __builtin_bit_cast(bf16x8, qf[ks]), SA, 0, 0, 0);
                    DA = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf[ks]), __builtin_bit_cast(bf16x8, df[ks]), DA, 0, 0, 0);
                }
            }
            if (!unit_full(0)) apply_mask(0, SA);
            int u = 0;
            for (; u + 1 < n_units; u += 2) {
                step(u, false, SA, DA, SB, DB, TA, TB);
                step(u + 1, true, SB, DB, SA, DA, TB, TA);
            }
            const bf16x8 (&TL)[2] = (u < n_units) ? TB : TA;
            if (u < n_units) step(u, false, SA, DA, SB, DB, TA, TB);
            // the dQ product of the last unit (its K^T was read in its step)
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
                for (int mt = 0; mt < C::kMT; ++mt)
                    acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[ks2][mt], TL[ks2], acc[mt], 0, 0, 0);
        }

        // the next item is taken when this workgroup is about to be free (taking it earlier
        // would hand out large items before it is known which workgroup finishes first)
        if (wave == 0) k_next = pop();
        // dQ = scale * acc; lane holds d = mt*32 + 8*a4 + 4*half + (0..3) of its row
        if (row_ok) {
            if (MODE == 0) {
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
            } else if (n_units > 0) {
                float* op = args.dq_acc + ((int64_t)row * H + head) * D;
#pragma unroll
                for (int mt = 0; mt < C::kMT; ++mt)
#pragma unroll
                    for (int a4 = 0; a4 < 4; ++a4) {
                        const int d0 = mt * 32 + 8 * a4 + 4 * half;
                        f32x4 w = *(const f32x4*)(op + d0);
#pragma unroll
                        for (int e = 0; e < 4; ++e) w[e] += acc[mt][4 * a4 + e] * args.scale;
                        *(f32x4*)(op + d0) = w;
                    }
            }
        }
        if (wave == 0) publish(__builtin_amdgcn_readfirstlane(k_next), slot ^ 1);
        __syncthreads();
    }
}

// =============================================================================================
// dK/dV body
// =============================================================================================
// Item = 128 keys of one key/value head (wave w owns keys 32w..32w+31 of the tile, as the B
// operand: K^T and V^T fragments stay in registers).  Its steps walk the stages (row unit of 32
// rows, query head of the group) from the end of the sequence down to the diagonal.  Step st issues
// the dV/dK products of stage st-1 (16 MFMAs) and the S/dP products of stage st+1 (16 MFMAs)
// around the elementwise part of stage st (P = exp2(S c - lse2), dS = P (dP - delta)), one
// element per slot.  Q and dO tiles (32 rows each) and the stage's 32 (lse2, delta) pairs
// arrive in LDS through direct global->LDS loads, in a ring of eight stages five steps ahead.
// LDS: the eight stages plus the two item slots (the layout is checked against the body's own
// in a static_assert)
template <int D>
constexpr int dkdv_lds_bytes() { return 8 * (2 * kUnit * Cfg<D>::kRowBytes + 2 * kUnit * 4) + 8 * (int)sizeof(int); }

template <int D, int MODE>
__device__ __attribute__((always_inline)) inline void dkdv_body(const BwdArgs& args, unsigned char* lds, int* counters) {
    using C = Cfg<D>;
    constexpr int kTile = kUnit * C::kRowBytes;           // 32 rows of Q or dO
    constexpr int kBlocks = kUnit / C::kRowsPerBlock;      // 1 KB loads per tile
    constexpr int kBPW = kBlocks / kWaves;                 // per wave
    // Ring of eight 32-row stages, synchronised every third step.  Step s loads stage s+5 into
    // the buffer of stage s-3, whose last reads (step s-3) every wave has finished by the
    // barrier of the step b = s, s-1 or s-2 that is a multiple of 3.  Steps b .. b+2 read the
    // rows of stages b+1 .. b+3 and the columns of stages b .. b+2, so the barrier of step b
    // first waits for every load but those of step b-1 (stage b+4).
    constexpr int kRing = 8;
    constexpr int kAhead = 5;
    constexpr int kSyncEvery = 3;
    constexpr int kLoadsPerStage = 2 * kBPW + 1;          // vector memory ops per stage, per wave
    struct Stage {
        unsigned char q[kTile];
        unsigned char d[kTile];
        float rv[kUnit][2];                                // (lse2, delta) of the 32 rows
    };
    static_assert(kRing * sizeof(Stage) + 8 * sizeof(int) == (size_t)dkdv_lds_bytes<D>(), "LDS layout");
    constexpr uint32_t kStageBytes = sizeof(Stage);
    constexpr uint32_t kRvOfs = 2 * kTile;                 // byte offset of rv in a stage
    Stage* ring = (Stage*)lds;
    int* s_item = (int*)(lds + kRing * sizeof(Stage));

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
    const int Trv = MODE == 0 ? args.T : args.Lq;          // row stride of the lse2/delta planes
    const bool causal = MODE == 0 ? true : (args.causal != 0);
    const int dpos = MODE == 0 ? 0 : args.dpos;            // query position minus key position

    // per-lane LDS offsets: row fragments (A operand: row l32, slot (2ks+half)^swz), transposed
    // fragments (B operand over 16 rows x 32 columns, as the forward's V^T reads), stage loads
    int rofs[4];
    {
        const int t = half ^ swz(l32);
#pragma unroll
        for (int j = 0; j < 4; ++j) rofs[j] = l32 * C::kRowBytes + 16 * ((2 * j) ^ t);
    }
    const int gidx = lane >> 4;
    const int tr_row = 4 * (gidx >> 1) + ((lane & 15) >> 2);
    const int tr_col = 16 * (gidx & 1) + 4 * (lane & 3);
    int tofs[2];
    {
        const int t = (tr_col >> 3) ^ swz(tr_row);
#pragma unroll
        for (int j = 0; j < 2; ++j) tofs[j] = tr_row * C::kRowBytes + 16 * ((4 * j) ^ t) + (lane & 1) * 8;
    }
    // whole-stage loads: this lane's byte offset in each of its 1 KB blocks from the stage's
    // first row of the head, minus the block's LDS offset that the load instruction's immediate
    // adds back to both addresses (row >= kRowsPerBlock i, so the difference stays >= 0)
    uint32_t voffq[kBPW];
#pragma unroll
    for (int i = 0; i < kBPW; ++i) {
        const int row = (wave * kBPW + i) * C::kRowsPerBlock + lane / C::kChunks;
        const int chunk = (lane % C::kChunks) ^ swz(row);
        voffq[i] = (uint32_t)((row * q_stride + chunk * 8) * 2) - 1024u * i;
    }
    const uint32_t ring0 = lds_addr(lds);              // LDS byte address of stage buffer 0

    QueuePlan plan{0, 0, 0, 0, 0, 0, 0, 0};
    if (wave == 0) {
        if (MODE == 0) plan = queue_plan(args.cu, args.n_seq, kKeyTile, nhbq, lane, args.T);
        else plan.total = ((args.Lk + kKeyTile - 1) / kKeyTile) * nhbq;
    }
    auto publish = [&](int k, int slot) {
        int a = 0, len = 0, hbq = 0, c = 0, kt = 0;
        bool ok = k < plan.total;
        if (ok) {
            if (MODE == 0) {
                ok = queue_decode(args.cu, args.n_seq, plan, kKeyTile, nhbq, k, lane, a, len, hbq, c);
                // level c = tiles from this one to the end: earlier key tiles see more rows
                kt = (len + kKeyTile - 1) / kKeyTile - c;
            } else {
                len = args.Lk;
                hbq = k % nhbq;
                kt = k / nhbq;                           // earlier key tiles see more rows
            }
        }
        if (lane == 0) {
            s_item[4 * slot + 0] = ok ? a : -1;
            s_item[4 * slot + 1] = len;
            s_item[4 * slot + 2] = queue + args.nqueues_kv * hbq;
            s_item[4 * slot + 3] = kt;
        }
    };
    auto pop = [&]() {
        int k = 0;
        if (lane == 0) k = atomicAdd(&counters[queue * kQueueStride], 1);
        return k;
    };
    if (wave == 0) publish(__builtin_amdgcn_readfirstlane(pop()), 0);
    __syncthreads();

    for (int it = 0;; ++it) {
        const int slot = it & 1;
        const int a0 = __builtin_amdgcn_readfirstlane(s_item[4 * slot + 0]);
        if (a0 < 0) break;
        int k_next = 0;
        const int64_t base = a0;                        // packed: the sequence's first token
        const int sk = __builtin_amdgcn_readfirstlane(s_item[4 * slot + 1]);   // keys
        const int s = MODE == 0 ? sk : args.Lq;         // rows
        const int g = __builtin_amdgcn_readfirstlane(s_item[4 * slot + 2]);
        const int kt = __builtin_amdgcn_readfirstlane(s_item[4 * slot + 3]);
        const int kj0 = kt * kKeyTile + wave * kUnit;   // this wave's first key
        const int key = kj0 + l32;                      // this lane's key (B-operand column)
        const int n_ru = (s + kUnit - 1) / kUnit;
        // first row unit with a row that sees a key of the tile
        const int ru0 = causal ? max(0, kt * kKeyTile - dpos) / kUnit : 0;
        // stages (row unit, head), row units from the last one down to the key tile's diagonal:
        // the items of one key/value head start together at the sequence's end and move down
        // in step, so the workgroups of an XCD read the same Q/dO rows through its L2
        const int n_st = max(0, n_ru - ru0) * G;

        // K^T and V^T fragments of this wave's 32 keys
        u32x4 kf[C::kKS], vf[C::kKS];
        {
            const bool ok = key < sk;
            const int64_t off = (base + key) * kv_stride + (int64_t)g * D + half * 8;
#pragma unroll
            for (int ks = 0; ks < C::kKS; ++ks) {
                kf[ks] = ok ? *(const u32x4*)(args.k + off + ks * 16) : u32x4{0, 0, 0, 0};
                vf[ks] = ok ? *(const u32x4*)(args.v + off + ks * 16) : u32x4{0, 0, 0, 0};
            }
        }

        // stage st -> ring buffer st mod 8: Q and dO rows and the rows' (lse2, delta) pairs.
        // (row unit, head of the group) of a stage: row units from the last one down, the group's
        // heads innermost.  Steps advance these by one stage at a time (no division per step).
        struct StageAt { int st, ru, hh; };
        auto stage_at = [&](int st) { return StageAt{st, n_ru - 1 - st / G, st % G}; };
        auto advance = [&](StageAt& x) {
            ++x.st;
            if (++x.hh == G) {
                x.hh = 0;
                --x.ru;
            }
        };
        // LDS byte address of stage st's buffer (uniform)
        auto stage_lds = [&](int st) { return ring0 + (uint32_t)(st & (kRing - 1)) * kStageBytes; };
        auto load_stage = [&](const StageAt& x) {
            const int head = g * G + x.hh;
            const int r0 = x.ru * kUnit;
            const uint32_t lq = stage_lds(x.st) + wave * kBPW * 1024;
            const uint32_t lrv = stage_lds(x.st) + kRvOfs;
            // every wave loads the same 256 bytes of row values (32 rows x (lse2, delta)), so
            // all waves count the same memory ops.  The chunk form (fp32 read-modify-write
            // epilogue) keeps the per-load path: with both paths it no longer fits its registers.
            if (MODE == 0 && r0 + kUnit <= s) {
                // the (row, head) index stays below T x H <= INT32_MAX (checked on the host), so
                // it is a 32-bit product; only the byte offset is 64-bit
                const uint32_t qi = (uint32_t)(((int)base + r0) * H + head);
                const uint64_t qb = (uint64_t)qi * (uint64_t)(D * 2);
                const unsigned char* sq = (const unsigned char*)args.q + qb;
                const unsigned char* sd = (const unsigned char*)args.dout + qb;
                if constexpr (kBPW == 1) lds_dma16_pairs<1>(sq, sd, voffq, lq, lq + kTile);
                else lds_dma16_tiles<kBPW>(sq, sd, voffq, lq, lq + kTile);
                lds_dma4_s(args.rowvals + 2 * ((int64_t)head * Trv + base + r0), 4u * lane, lrv);
            } else {
                // the stage at the sequence's end: rows clamped to its last row
#pragma unroll
                for (int i = 0; i < kBPW; ++i) {
                    const int row = (wave * kBPW + i) * C::kRowsPerBlock + lane / C::kChunks;
                    const int chunk = (lane % C::kChunks) ^ swz(row);
                    const int64_t off = (base + min(r0 + row, s - 1)) * q_stride + (int64_t)head * D + chunk * 8;
                    lds_dma16(args.q + off, lq + 1024 * i);
                    lds_dma16(args.dout + off, lq + kTile + 1024 * i);
                }
                const int64_t rr = (int64_t)head * Trv + base + min(r0 + (lane >> 1), s - 1);
                lds_dma4(args.rowvals + 2 * rr + (lane & 1), lrv);
            }
        };
        // A-operand row fragments (Q rows: which = 0, dO rows: which = 1) of the stage whose
        // per-lane row addresses are ra, k-steps ks0 .. ks0 + n - 1 over D
        auto rows_addr = [&](int st, uint32_t (&ra)[4]) {
            const uint32_t b = stage_lds(st);
#pragma unroll
            for (int j = 0; j < 4; ++j) ra[j] = lds_add(b, rofs[j]);
        };
        auto read_rows = [&](const uint32_t (&ra)[4], int which, u32x4 (&f)[C::kKS], int ks0, int n) {
#pragma unroll
            for (int ks = 0; ks < C::kKS; ++ks)
                if (ks >= ks0 && ks < ks0 + n)
                    f[ks] = *(const lds_u32x4*)(uintptr_t)(ra[ks & 3] + which * kTile + 128 * (ks >> 2));
        };
        // B-operand transposed fragments: for k-step ks2 and D tile mt, lane l receives column
        // mt*32 + l%32 of rows 16 ks2 + 8 (i/4) + 4 (l/32) + i%4 (the accumulator row order)
        // (a[0], a[1] = per-lane column bases of the stage, from cols_addr; which = 1: dO, 0: Q)
        auto cols_addr = [&](int st, uint32_t (&a)[2]) {
            const uint32_t b = stage_lds(st);
            a[0] = lds_add(b, tofs[0]);
            a[1] = lds_add(b, tofs[1]);
        };
        auto read_col = [&](const uint32_t (&a)[2], int which, int ks2, int mt, bf16x8& f) {
            const uint32_t p0 = a[mt & 1] + which * kTile + 128 * (mt >> 1) + 16 * ks2 * C::kRowBytes;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)p0);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(p0 + 8 * C::kRowBytes));
            f.lo = __builtin_bit_cast(bf16x4, lo);
            f.hi = __builtin_bit_cast(bf16x4, hi);
        };
        // lse2 and delta of the lane's accumulator rows 8*j + 4*half + (0..3) (elements 4j..4j+3):
        // four (lse2, delta) pairs at rva + 64 j
        auto read_rowvals = [&](uint32_t rva, int j, f32x4& l2, f32x4& dl) {
            const f32x4 a = __builtin_bit_cast(f32x4, *(const lds_u32x4*)(uintptr_t)(rva + 64 * j));
            const f32x4 b = __builtin_bit_cast(f32x4, *(const lds_u32x4*)(uintptr_t)(rva + 64 * j + 16));
            l2 = f32x4{a[0], a[2], b[0], b[2]};
            dl = f32x4{a[1], a[3], b[1], b[3]};
        };
        // S (rows x keys) = Q K^T and dP = dO V^T of one stage from its row fragments
        auto sdp_full = [&](const u32x4 (&qr)[C::kKS], const u32x4 (&dr)[C::kKS], f32x16& S, f32x16& dP) {
            S = f32x16{};
            dP = f32x16{};
#pragma unroll
            for (int ks = 0; ks < C::kKS; ++ks) {
                S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qr[ks]), __builtin_bit_cast(bf16x8, kf[ks]), S, 0, 0, 0);
                dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, dr[ks]), __builtin_bit_cast(bf16x8, vf[ks]), dP, 0, 0, 0);
            }
        };
        // invisible (key, row) pairs of a stage get S = -inf, so P = 0 and dS = 0
        auto stage_full = [&](const StageAt& x) {
            const int r0 = x.ru * kUnit;
            return (!causal || kt * kKeyTile + kKeyTile - 1 <= r0 + dpos) && r0 + kUnit <= s &&
                   kt * kKeyTile + kKeyTile <= sk;
        };
        auto apply_mask = [&](const StageAt& x, f32x16& S) {
            const int r0 = x.ru * kUnit;
            const int lim = min(s - 1 - r0, kUnit);     // rows r0 + jr with jr <= lim exist
            // visible iff jr >= kr: the key exists and (causal) key <= row + dpos
            const int kr = key >= sk ? kUnit : (causal ? max(key - dpos - r0, -1) : -1);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int jr = 8 * (i >> 2) + 4 * half + (i & 3);
                S[i] = (jr < kr || jr > lim) ? -INFINITY : S[i];
            }
        };

        f32x16 dk[C::kMT], dv[C::kMT];
#pragma unroll
        for (int mt = 0; mt < C::kMT; ++mt) { dk[mt] = f32x16{}; dv[mt] = f32x16{}; }

        if (n_st > 0) {
            // prologue: stages 0 .. kAhead-1 loaded, stage 0 scored
#pragma unroll
            for (int p = 0; p < kAhead; ++p)
                if (p < n_st) load_stage(stage_at(p));
            StageAt ld = stage_at(kAhead);             // the next stage to load
            StageAt nx = stage_at(1);                  // the stage after the current one
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
            f32x16 SA, DA, SB, DB;
            bf16x8 PA[2], TA[2], PB[2], TB[2];       // P and dS as bf16 A operands
            bf16x8 dt[2][C::kMT], qt[2][C::kMT];
            {
                u32x4 qr[C::kKS], dr[C::kKS];
                uint32_t ra[4];
                rows_addr(0, ra);
                read_rows(ra, 0, qr, 0, C::kKS);
                read_rows(ra, 1, dr, 0, C::kKS);
                sdp_full(qr, dr, SA, DA);
            }
            if (!stage_full(stage_at(0))) apply_mask(stage_at(0), SA);
#pragma unroll
            for (int j = 0; j < 2; ++j) { PA[j] = bf16x8{}; TA[j] = bf16x8{}; }
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
                for (int mt = 0; mt < C::kMT; ++mt) { dt[ks2][mt] = bf16x8{}; qt[ks2][mt] = bf16x8{}; }

            // step st: dV/dK of st-1 (operands Pp, Tp, dt, qt), S/dP of st+1 into Sn/Dn, the
            // elementwise part of st from Sc/Dc into Pc/Tc.  ph = st mod kSyncEvery.
            int ph = 0;
            auto step = [&](int st, f32x16& Sc, f32x16& Dc, f32x16& Sn, f32x16& Dn,
                            const bf16x8 (&Pp)[2], const bf16x8 (&Tp)[2], bf16x8 (&Pc)[2], bf16x8 (&Tc)[2]) {
                __builtin_amdgcn_sched_barrier(0);          // steps stay apart in the schedule
                if (st > 0 && ph == 0) {
                    if (st - 1 + kAhead < n_st) __builtin_amdgcn_s_waitcnt(0x0F70 | kLoadsPerStage);
                    else __builtin_amdgcn_s_waitcnt(0x0F70);
                    __syncthreads();
                }
                ph = ph == kSyncEvery - 1 ? 0 : ph + 1;
                if (st + kAhead < n_st) load_stage(ld);
                advance(ld);
                u32x4 qr[C::kKS], dr[C::kKS];
                const int sn = min(st + 1, n_st - 1);     // past the end: harmless re-read
                constexpr int kH = C::kKS / 2;             // second half read mid-way
                {
                    uint32_t ra[4];
                    rows_addr(sn, ra);
                    read_rows(ra, 0, qr, 0, kH);
                    read_rows(ra, 1, dr, 0, kH);
                }
                __builtin_amdgcn_sched_barrier(0);
                uint32_t pw[8], tw[8];
                float pe = 0.f, te = 0.f;
                f32x4 l2[2], dl[2];                        // rows of element groups j, j+1
                const uint32_t rva = lds_add(stage_lds(st) + kRvOfs, 32u * half);
                read_rowvals(rva, 0, l2[0], dl[0]);
                // t = P (dP - delta) and the bf16 packing of element e
                auto finish = [&](int e, float p, float d) {
                    const float t = p * d;
                    if (e & 1) {
                        pw[e >> 1] = pack_bf16x2(pe, p);
                        tw[e >> 1] = pack_bf16x2(te, t);
                        asm volatile("" : "+v"(pw[e >> 1]), "+v"(tw[e >> 1]));
                    } else {
                        pe = p;
                        te = t;
                    }
                };
                constexpr int kDV = 2 * C::kMT;            // dV MFMAs (and as many dK MFMAs)
                constexpr int kSlots = 4 * kDV > 32 ? 4 * kDV : 32;
                static_assert(2 * kDV <= 2 * C::kKS, "one transposed fragment per S/dP slot");
                uint32_t ca[2];
#pragma unroll
                for (int k = 0; k < kSlots; ++k) {
                    if (k == kDV) {
                        uint32_t ra[4];
                        rows_addr(sn, ra);
                        read_rows(ra, 0, qr, kH, kH);
                        read_rows(ra, 1, dr, kH, kH);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (k >= 2 * kDV && k < 4 * kDV) {
                        // dt/qt of st-1 consumed: stage st's transposed fragments for st+1, one
                        // per S/dP slot in the order the next step's dV/dK products use them
                        const int j = k - 2 * kDV, f = j >> 1, ks2 = f / C::kMT, mt = f % C::kMT;
                        if (j == 0) cols_addr(st, ca);
                        if (j & 1) read_col(ca, 0, ks2, mt, qt[ks2][mt]);
                        else read_col(ca, 1, ks2, mt, dt[ks2][mt]);
                    }
                    if (k < 2 * kDV) {
                        const int j = k >> 1, ks2 = j / C::kMT, mt = j % C::kMT;
                        if ((k & 1) == 0) dv[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Pp[ks2], dt[ks2][mt], dv[mt], 0, 0, 0);
                        else dk[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Tp[ks2], qt[ks2][mt], dk[mt], 0, 0, 0);
                    } else if (k < 2 * kDV + 2 * C::kKS) {
                        const int j = k - 2 * kDV, ks = j >> 1;
                        if (j == 0) Sn = f32x16{};      // the accumulators start here (zero C operand)
                        if (j == 1) Dn = f32x16{};
                        if ((j & 1) == 0) Sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qr[ks]), __builtin_bit_cast(bf16x8, kf[ks]), Sn, 0, 0, 0);
                        else Dn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, dr[ks]), __builtin_bit_cast(bf16x8, vf[ks]), Dn, 0, 0, 0);
                    }
                    if (k < 16 && (k & 3) == 0 && k + 4 < 16) read_rowvals(rva, (k >> 2) + 1, l2[((k >> 2) + 1) & 1], dl[((k >> 2) + 1) & 1]);
                    if (k < 16) {
                        const int i = k, jb = (i >> 2) & 1;
                        const float d = Dc[i] - dl[jb][i & 3];
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(Sc[i], c2, -l2[jb][i & 3]));
                        finish(i, p, d);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    Pc[h] = __builtin_bit_cast(bf16x8, u32x4{pw[4 * h], pw[4 * h + 1], pw[4 * h + 2], pw[4 * h + 3]});
                    Tc[h] = __builtin_bit_cast(bf16x8, u32x4{tw[4 * h], tw[4 * h + 1], tw[4 * h + 2], tw[4 * h + 3]});
                }
                if (st + 1 < n_st && !stage_full(nx)) apply_mask(nx, Sn);
                advance(nx);
            };
            int st = 0;
            for (; st + 1 < n_st; st += 2) {
                step(st, SA, DA, SB, DB, PA, TA, PB, TB);
                step(st + 1, SB, DB, SA, DA, PB, TB, PA, TA);
            }
            // the dV/dK products of the last stage (its dt/qt were read in its step)
            const bf16x8 (&PL)[2] = (st < n_st) ? PB : PA;
            const bf16x8 (&TL)[2] = (st < n_st) ? TB : TA;
            if (st < n_st) step(st, SA, DA, SB, DB, PA, TA, PB, TB);
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
                for (int mt = 0; mt < C::kMT; ++mt) {
                    dv[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(PL[ks2], dt[ks2][mt], dv[mt], 0, 0, 0);
                    dk[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(TL[ks2], qt[ks2][mt], dk[mt], 0, 0, 0);
                }
        }

        // the next item is taken when this workgroup is about to be free (taking it earlier
        // would hand out large items before it is known which workgroup finishes first)
        if (wave == 0) k_next = pop();
        // dK = scale * dk, dV = dv; accumulator element i of D tile mt is key
        // kj0 + 8*(i/4) + 4*half + (i%4), column mt*32 + l32.
        __syncthreads();
        if (MODE == 1) {
            // add to the fp32 accumulators: 32 lanes cover 128 contiguous bytes of a key row
            if (n_st > 0) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kr = kj0 + 8 * (i >> 2) + 4 * half + (i & 3);
                    if (kr < sk) {
                        float* kp = args.dk_acc + ((int64_t)kr * Hkv + g) * D + l32;
                        float* vp = args.dv_acc + ((int64_t)kr * Hkv + g) * D + l32;
#pragma unroll
                        for (int mt = 0; mt < C::kMT; ++mt) {
                            kp[mt * 32] += dk[mt][i] * args.scale;
                            vp[mt * 32] += dv[mt][i];
                        }
                    }
                }
            }
        } else {
            // out through this wave's share of the ring (after every wave left the loop): rows
            // of 32 keys, then 16-byte stores
            unsigned char* tk = ring[wave].q;           // 32 keys x D bf16 each
            unsigned char* tv = ring[wave].d;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kr = 8 * (i >> 2) + 4 * half + (i & 3);
#pragma unroll
                for (int mt = 0; mt < C::kMT; ++mt) {
                    const int col = mt * 32 + l32;
                    const int off = kr * C::kRowBytes + (((col >> 3) ^ swz(kr)) << 4) + (col & 7) * 2;
                    *(__bf16*)(tk + off) = (__bf16)(dk[mt][i] * args.scale);
                    *(__bf16*)(tv + off) = (__bf16)dv[mt][i];
                }
            }
            constexpr int kRowsPerRead = 64 / C::kChunks;
#pragma unroll
            for (int rr = 0; rr < kUnit; rr += kRowsPerRead) {
                const int kr = rr + lane / C::kChunks, ch = lane % C::kChunks;
                const int off = kr * C::kRowBytes + ((ch ^ swz(kr)) << 4);
                const u32x4 wk = *(const u32x4*)(tk + off);
                const u32x4 wv = *(const u32x4*)(tv + off);
                if (kj0 + kr < sk) {
                    const int64_t o = ((base + kj0 + kr) * Hkv + g) * D + ch * 8;
                    *(u32x4*)(args.dk + o) = wk;
                    *(u32x4*)(args.dv + o) = wv;
                }
            }
        }
        if (wave == 0) publish(__builtin_amdgcn_readfirstlane(k_next), slot ^ 1);
        __syncthreads();
    }
}

// =============================================================================================
// Row values and the combined kernel
// =============================================================================================
// lse in log2 units and delta = rowsum(dO * O) of every (row, head), as adjacent pairs in the
// head-major [H][rows][2] workspace, so that the 32 rows of a dK/dV stage are 256 contiguous
// bytes (one 4-byte direct load per lane).  Sixteen lanes per (row,
// head): lane c takes the 8 elements of 16-byte chunk c (consecutive lanes read consecutive
// chunks, so a wave's loads are contiguous), then a butterfly over the 16 lanes sums them.
template <int D, int MODE>
__global__ __launch_bounds__(256) void bwd_rowvals_kernel(BwdArgs args) {
    constexpr int kLanes = 16;                       // lanes per (row, head)
    constexpr int kPerLane = D / kLanes;             // elements per lane: 8 (D = 128) or 4 (D = 64)
    const int H = args.H;
    const int rows = MODE == 0 ? args.T : args.Lq;
    const int64_t n = (int64_t)rows * H;
    const int c = threadIdx.x % kLanes;
    for (int64_t t = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kLanes; t < n;
         t += (int64_t)gridDim.x * blockDim.x / kLanes) {
        const uint16_t* dp = args.dout + t * D + c * kPerLane;
        const uint16_t* op = args.out + t * D + c * kPerLane;
        float part = 0.f;
        if constexpr (kPerLane == 8) {
            const u32x4 dv = *(const u32x4*)dp;
            const u32x4 ov = *(const u32x4*)op;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                part = __builtin_fmaf(bf16_lo(dv[e]), bf16_lo(ov[e]), part);
                part = __builtin_fmaf(bf16_hi(dv[e]), bf16_hi(ov[e]), part);
            }
        } else {
            const u32x2 dv = *(const u32x2*)dp;
            const u32x2 ov = *(const u32x2*)op;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                part = __builtin_fmaf(bf16_lo(dv[e]), bf16_lo(ov[e]), part);
                part = __builtin_fmaf(bf16_hi(dv[e]), bf16_hi(ov[e]), part);
            }
        }
#pragma unroll
        for (int m = kLanes / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, kLanes);
        if (c == 0) {
            const int64_t row = t / H;
            const int head = (int)(t - row * H);
            // a row that saw no key at all (lse = -inf) gets +inf, so that every P of it is 0
            const float l = args.lse[t];
            const f32x2 w = {l == -INFINITY ? INFINITY : l * kLog2e, part};
            *(f32x2*)(args.rowvals + 2 * ((int64_t)head * rows + row)) = w;
        }
    }
}

// One persistent launch drains the dK/dV queue and then the dQ queue.  The dK/dV items (a key
// tile with every row below its diagonal) are the larger ones, and on a skewed pack a few of
// them outlast the rest of that queue; the workgroups that run out of dK/dV items start on dQ
// items meanwhile, instead of idling until the next launch.
template <int D, int MODE>
__global__ __launch_bounds__(kThreads, 1) void bwd_kernel(BwdArgs args) {
    constexpr int kLds = dkdv_lds_bytes<D>() > dq_lds_bytes<D>() ? dkdv_lds_bytes<D>() : dq_lds_bytes<D>();
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kLds];
    // workgroup timeline (measurement only): start, leaving the dK/dV queue, end
    long long* const tr = (args.trace != nullptr && threadIdx.x == 0) ? args.trace + (int64_t)blockIdx.x * kTraceWords : nullptr;
    if (tr != nullptr) tr[0] = (long long)__builtin_amdgcn_s_memrealtime();
    dkdv_body<D, MODE>(args, lds, args.counters);
    if (tr != nullptr) tr[1] = (long long)__builtin_amdgcn_s_memrealtime();
    __syncthreads();
    dq_body<D, MODE>(args, lds, args.counters + kCounterSetInts);
    if (tr != nullptr) {
        tr[2] = (long long)__builtin_amdgcn_s_memrealtime();
        tr[3] = 0;
    }
    if (threadIdx.x == 0) queue_finish(args.counters);
}

template <int D, int MODE>
hipError_t launch_bwd_t(const BwdArgs& a, int grid, hipStream_t s) {
    const int64_t n = (int64_t)(MODE == 0 ? a.T : a.Lq) * a.H;
    const int blocks = (int)std::min<int64_t>((n * 16 + 255) / 256, 8192);
    hipLaunchKernelGGL((bwd_rowvals_kernel<D, MODE>), dim3(blocks), dim3(256), 0, s, a);
    hipLaunchKernelGGL((bwd_kernel<D, MODE>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int D, int grid, hipStream_t s) {
    return D == 128 ? launch_bwd_t<128, 0>(a, grid, s) : launch_bwd_t<64, 0>(a, grid, s);
}

hipError_t launch_bwd_chunk(const BwdArgs& a, int D, int grid, hipStream_t s) {
    return D == 128 ? launch_bwd_t<128, 1>(a, grid, s) : launch_bwd_t<64, 1>(a, grid, s);
}

}  // namespace hdp
