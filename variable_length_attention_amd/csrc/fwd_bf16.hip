// Forward attention on gfx950 (CDNA4): bf16 MFMA, fp32 accumulation, online softmax.
//
// One kernel serves both forms of a rank's work (research digest "ByteScale: Communication-
// Efficient Scaling of LLM Training with a 2048K Context Length on 16384 GPUs"):
//   * varlen: many short sequences packed back to back, each attending only to itself under a
//     causal mask (digest §3.1-§3.2, §4);
//   * chunk: one slice of a long sequence against one key/value chunk of a ring step, with
//     global positions (digest §3.2); the output is the normalised fp32 partial plus its lse;
//   * chunk-merge: the same ring step, its partial merged by log-sum-exp into the running
//     result in the epilogue instead of being written out for a separate merge pass.
//
// Layout of the work.  A workgroup of 4 waves takes one item = (sequence, head block, query
// tile group).  With 4 or more query heads per key/value head, the 4 waves are 4 query heads
// that share one key/value head, so every K/V tile staged in LDS feeds 4 heads.  Each wave owns
// 64 query rows of one head, held as the B operand of v_mfma_f32_32x32x16_bf16:
//     S^T (keys x rows) = K (keys x D) * Q^T (D x rows)
//     O^T (D x rows)   += V^T (D x keys) * P^T (keys x rows)
// In this orientation every lane holds whole query rows, so the row max and row sum are
// in-lane reductions plus one swap between the two half-waves, and the softmax output P^T is
// already in the B-operand layout of the second product.  Holding 64 rows per wave lets each
// K or V fragment read from LDS feed two MFMAs, which keeps LDS traffic at half the rate the
// matrix cores consume.  V^T is read from row-major LDS with the gfx950 transposing read
// ds_read_b64_tr_b16.
//
// Pipeline.  Keys are processed in units of 32.  Iteration u issues the value product of unit
// u-1 and the score product of unit u+1 on the matrix cores and runs the softmax of unit u on
// the vector ALUs; the three are independent.  K/V arrive in stages of 64 keys through direct
// global->LDS loads (global_load_lds_dwordx4, no registers), three stages deep, one workgroup
// barrier per stage.  LDS rows are unpadded and their 16-byte slots are XOR-swizzled by the
// row index (swz), so neither fragment read kind hits a bank twice in one cycle.
//
// Softmax uses exp2 with scale*log2(e) folded into one FMA and a lazy reference instead of an
// exact running max (exact arithmetic is unchanged because numerator and denominator share the
// reference).  The common path computes no max at all: P = exp2(S c2 - m) is summed in fp32
// and goes straight to bf16.  The reference starts at the row max of an item's first unit,
// taken before its exponentials.  Only when a lane's sum over a unit exceeds 2^8 (so possibly
// some P > 2^8), or on the first visible unit of a row whose first unit is wholly masked, does a
// branch take the row max, raise the reference and rescale the accumulator.
//
// Scheduling.  The kernel is persistent (one workgroup per CU).  Items are popped from a queue
// in order of decreasing cost, where the cost of a query tile is the number of key tiles it
// visits (the tile form of the O(s^2) cost of hdp_seq_flops): longest-processing-time first, so
// short items fill the gaps at the end instead of idling CUs.  With 8 head blocks there is one
// queue per XCD and head block b is served by the XCD b mod 8, so each K/V head's tiles stay in
// one XCD's L2, until that XCD's queue is empty: its workgroups then help with the other
// queues.  The order is decoded on the device from cu_seqlens, without a planning launch.  When
// a launch has at least 8 items per workgroup, a workgroup holds one item in reserve, so that the
// next item's first loads go out under the current item's output stores; with fewer, each item
// is taken when its workgroup is about to be free (taking items early would unbalance the CUs).
#include "device_common.h"

namespace hdp {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 64;      // two 32-row MFMA column tiles
constexpr int kNT = 2;
constexpr int kItemRowHeads = 256;    // query (row, head) pairs per item
constexpr int kUnit = 32;             // keys per pipeline step
constexpr int kStage = 64;            // keys per LDS stage
constexpr int kStages = 3;            // LDS ring depth
constexpr int kStageRowBytes = 256;   // output staging tile row
constexpr float kLazySum = 256.0f;    // rescale when a lane's unit sum of P exceeds 2^8
constexpr int kReserveItems = 8;      // items per workgroup from which one is held in reserve

template <int D>
struct Cfg {
    static constexpr int kRowBytes = D * 2;                       // unpadded bf16 row
    static constexpr int kTileBytes = kStage * kRowBytes;         // one K or V stage
    static constexpr int kChunks = D / 8;                         // 16-byte chunks per row
    static constexpr int kRowsPerBlock = 64 / kChunks;            // rows per 1 KB wave load
    static constexpr int kBlocksPerWave = kStage / kRowsPerBlock / kWaves;
    static constexpr int kKS = D / 16;                            // k-steps, score product
    static constexpr int kMT = D / 32;                            // D tiles, value product
};

template <int D, int MODE>
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(FwdArgs args) {
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages][2][C::kTileBytes];
    const uint32_t ring0 = lds_addr(smem);                 // LDS byte address of ring buffer 0
    __shared__ __attribute__((aligned(1024))) unsigned char obuf[kWaves][32 * kStageRowBytes];
    // Q staging of waves 2-3 (waves 0-1 stage theirs in ring buffer 2): with its own buffer, the
    // next item's Q can arrive while this item's output goes out through the output tiles
    __shared__ __attribute__((aligned(1024))) unsigned char qbuf[2][kRowsPerWave * C::kRowBytes];
    static_assert(kRowsPerWave * C::kRowBytes <= C::kTileBytes, "Q staging");
    // item records (4 ints each): at the start two, later one, in wave 0's output tile, which is
    // free from the end of its output stores until the next item's stores (all waves read the
    // record at the start of that item)
    int* const mbox = (int*)obuf[0];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    if (args.trace != nullptr && tid == 0) args.trace[(int64_t)blockIdx.x * kTraceWords] = (long long)__builtin_amdgcn_s_memrealtime();

    const int H = args.H, Hkv = args.Hkv;
    const int G = H / Hkv;
    const int hpw = args.hpw;
    const int W = kItemRowHeads / hpw;         // query rows per item
    const int nhb = H / hpw;
    const int nq_queues = args.nqueues;
    const int queue = blockIdx.x % nq_queues;
    const int nhbq = nhb / nq_queues;          // head blocks per queue
    const int64_t q_stride = (int64_t)H * D;
    const int64_t kv_stride = (int64_t)Hkv * D;
    const float c2 = args.scale_log2;

    // ---- per-launch queue plan (wave 0 only) ----
    QueuePlan plan{0, 0, 0, 0, 0, 0, 0, 0};
    if (wave == 0) {
        if (MODE == 0) plan = queue_plan(args.cu, args.n_seq, W, nhbq, lane);
        else plan.total = ((args.Lq + W - 1) / W) * nhbq;
    }

    // per-lane constants of the fragment reads
    const int gidx = lane >> 4;                                   // 16-lane group (V^T reads)
    const int tr_row = 4 * (gidx >> 1) + ((lane & 15) >> 2);
    const int tr_col = 16 * (gidx & 1) + 4 * (lane & 3);          // bf16 column within 32
    const int tr_sub = (lane & 1) * 8;                            // byte offset within a slot
    // Byte offsets of this lane's fragment reads within a 32-row unit of a tile.  Rows 8 apart
    // share the swizzle, so the XOR only mixes the low slot bits: a read's slot is a per-lane
    // part (XOR of a few compile-time bits) plus a compile-time part, which becomes the
    // instruction's immediate offset.  K: slot of k-step ks = (2 ks + half) ^ swz(row).
    int kofs[4];
    {
        const int t = half ^ swz(l32);
#pragma unroll
        for (int j = 0; j < 4; ++j) kofs[j] = l32 * C::kRowBytes + 16 * ((2 * j) ^ t);
    }
    // Stage loads: byte offset of this lane's 16-byte chunk in each of its 1 KB blocks, relative
    // to the stage's first key row of the head (the LDS slot of a chunk is fixed by the lane).
    uint32_t gofs[C::kBlocksPerWave];
#pragma unroll
    for (int i = 0; i < C::kBlocksPerWave; ++i) {
        const int row = (wave * C::kBlocksPerWave + i) * C::kRowsPerBlock + lane / C::kChunks;
        const int chunk = (lane % C::kChunks) ^ swz(row);
        // minus the block's LDS offset, which the load instruction's immediate adds back to
        // both addresses (row >= 4 i for D = 128, >= 8 i for D = 64, so this stays >= 0)
        gofs[i] = (uint32_t)((row * kv_stride + chunk * 8) * 2) - 1024u * i;
    }
    // V^T: slot of D tile mt = (4 mt + c) ^ swz(tr_row), c = column / 8 within the tile
    int vofs[2];
    {
        const int t = (tr_col >> 3) ^ swz(tr_row);
#pragma unroll
        for (int j = 0; j < 2; ++j) vofs[j] = tr_row * C::kRowBytes + 16 * ((4 * j) ^ t) + tr_sub;
    }

    // ---- item queue (wave 0) ----
    // Item k of queue src_q -> record slot of the mailbox.  Items are taken at the end of an
    // item, just before its output stores (which hide the atomic's latency), and decoded once
    // the stores are issued.  When the queue holds many items per workgroup, a workgroup knows
    // one item ahead: it takes two items at the start and then, at the end of an item, the one
    // after the next, so that the next item's first loads go out before this item's output
    // stores and their latency passes under the stores.  With few items per workgroup, taking
    // items early would unbalance the CUs (the longest-first order decides less), so each item
    // is taken when the workgroup is about to be free and its loads go out at its start.
    // Every queue holds the same items (for its own head blocks).  A workgroup whose queue is
    // empty takes the remaining items of the other XCDs' queues in turn: the XCDs do not all
    // run at the same speed, and otherwise the launch waits for the slowest one's queue.  It
    // first reads all the queues it has not tried at once, so that at the end of a launch, when
    // they are all dry, it stops after one round trip instead of one per queue.
    int src_q = queue;
    int stolen = 0;
    // the atomic's result is in lane 0; callers take it with readfirstlane, so the decode that
    // follows is scalar code (a lane shuffle would leave it in a vector register)
    auto pop = [&]() {
        int k = 0;
        if (lane == 0) k = atomicAdd(&args.counters[src_q * kQueueStride], 1);
        return k;
    };
    auto publish = [&](int k, int slot) {
        if (k >= plan.total && stolen < nq_queues - 1) {
            // this queue is dry: read every queue not yet tried at once (lane j: the j-th next
            // queue, an atomic add of 0 that takes nothing, waited in the same block) and skip
            // those already dry (a counter only grows)
            const int left = nq_queues - 1 - stolen;
            int seen = plan.total;
            if (lane < left) {
                const int* cq = &args.counters[((queue + stolen + 1 + lane) % nq_queues) * kQueueStride];
                asm volatile("global_atomic_add %0, %1, %2, off sc0\n\ts_waitcnt vmcnt(0)"
                             : "=v"(seen) : "v"(cq), "v"(0) : "memory");
            }
            const unsigned long long open = __ballot(lane < left && seen < plan.total);
            stolen = open == 0 ? nq_queues - 1 : stolen + (int)__builtin_ctzll(open);
        }
        while (k >= plan.total && stolen < nq_queues - 1) {
            ++stolen;
            src_q = (queue + stolen) % nq_queues;
            k = __builtin_amdgcn_readfirstlane(pop());
        }
        int a = 0, len = 0, hbq = 0, c = 0;
        bool ok = k < plan.total;
        if (ok) {
            if (MODE == 0) {
                ok = queue_decode(args.cu, args.n_seq, plan, W, nhbq, k, lane, a, len, hbq, c);
            } else {
                a = 0;
                len = args.Lq;
                hbq = k % nhbq;
                c = ((args.Lq + W - 1) / W) - k / nhbq;
            }
        }
        if (lane == 0) {
            mbox[4 * slot + 0] = ok ? a : -1;
            mbox[4 * slot + 1] = len;
            mbox[4 * slot + 2] = src_q + nq_queues * hbq;
            mbox[4 * slot + 3] = c - 1;                   // query tile group: cost grows with it
        }
    };
    // query position minus key position of (row 0, key 0)
    const int delta = MODE == 0 ? 0 : args.delta;
    const bool causal = MODE == 0 ? true : (args.causal != 0);
    // an item's record (uniform: scalar registers) and what follows from it
    struct Item { int a, s_rows, hb, tg; };
    auto read_rec = [&](int slot) {
        return Item{__builtin_amdgcn_readfirstlane(mbox[4 * slot + 0]), __builtin_amdgcn_readfirstlane(mbox[4 * slot + 1]),
                    __builtin_amdgcn_readfirstlane(mbox[4 * slot + 2]), __builtin_amdgcn_readfirstlane(mbox[4 * slot + 3])};
    };
    struct Geo { int64_t qbase, kbase; int s_rows, sk, head, g, r_lo, n_units, n_stages; };
    auto geo = [&](const Item& x) {
        Geo e;
        e.qbase = x.a;
        e.kbase = MODE == 0 ? e.qbase : 0;
        e.s_rows = x.s_rows;
        e.sk = MODE == 0 ? x.s_rows : args.Lk;
        e.head = x.hb * hpw + (wave % hpw);
        e.g = (x.hb * hpw) / G;
        e.r_lo = x.tg * W + (wave / hpw) * kRowsPerWave;        // this wave's first row
        // keys the workgroup visits
        const int wg_rmax = min(x.s_rows, (x.tg + 1) * W) - 1;
        int jmax = e.sk - 1;
        if (causal) jmax = min(jmax, delta + wg_rmax);
        e.n_units = (wg_rmax < 0 || jmax < 0) ? 0 : (int)(jmax / kUnit) + 1;
        e.n_stages = (e.n_units + 1) / 2;
        return e;
    };

    // ---- direct global -> LDS stage loads (K and V of 64 keys) into ring buffer B ----
    // A whole stage inside the sequence takes a scalar base plus the per-lane offsets; the
    // last stage clamps its rows to the sequence's last key.
    auto load_stage_at = [&](int64_t kbase, int g, int sk, int st, int B) {
        const int j0 = st * kStage;
        // uniform base of the stage's first key row (scalar registers) + per-lane offsets
        const int64_t sofs = (kbase + j0) * kv_stride + (int64_t)g * D;
        const uint32_t lk = lds_addr(smem[B][0] + wave * C::kBlocksPerWave * 1024);
        const uint32_t lv = lds_addr(smem[B][1] + wave * C::kBlocksPerWave * 1024);
        if (j0 + kStage <= sk) {
            lds_dma16_tiles<C::kBlocksPerWave>(args.k + sofs, args.v + sofs, gofs, lk, lv);
        } else {
            uint32_t voff[C::kBlocksPerWave];
#pragma unroll
            for (int i = 0; i < C::kBlocksPerWave; ++i) {
                const int row = (wave * C::kBlocksPerWave + i) * C::kRowsPerBlock + lane / C::kChunks;
                const int chunk = (lane % C::kChunks) ^ swz(row);
                const int j = min(j0 + row, sk - 1) - j0;
                voff[i] = (uint32_t)((j * kv_stride + chunk * 8) * 2);
            }
            lds_dma16_pairs<C::kBlocksPerWave>(args.k + sofs, args.v + sofs, voff, lk, lv);
        }
    };
    // ---- Q^T fragments in registers, loaded through LDS ----
    // The wave's 64 query rows arrive by direct loads (16 lanes per row, so every load reads
    // whole 256-byte rows) into a staging tile laid out like a K stage, and the fragments are
    // then read as the K fragments are: loading the fragments straight from memory, where each
    // lane reads its own row, takes ≈2K cycles longer per item.  The staging tiles are ring
    // buffer 2 (waves 0-1), which the first stage turn refills, and qbuf (waves 2-3).  Rows past
    // the sequence's end repeat its last row (their results are never stored).
    unsigned char* const qstage = wave < 2 ? smem[2][wave] : qbuf[wave - 2];
    auto load_q_at = [&](int64_t qbase, int head, int r_lo, int s_rows) {
#pragma unroll
        for (int i = 0; i < kRowsPerWave / C::kRowsPerBlock; ++i) {
            const int row = i * C::kRowsPerBlock + lane / C::kChunks;
            const int chunk = (lane % C::kChunks) ^ swz(row);
            const int r = min(r_lo + row, s_rows - 1);
            lds_dma16(args.q + (qbase + r) * q_stride + (int64_t)head * D + chunk * 8, lds_addr(qstage + i * 1024));
        }
    };
    // an item's first loads: stages 0 and 1 into ring buffers 0 and 1, and its query rows
    auto issue_prologue = [&](const Item& x) {
        const Geo e = geo(x);
        if (e.n_units > 0) {
            load_stage_at(e.kbase, e.g, e.sk, 0, 0);
            if (e.n_stages > 1) load_stage_at(e.kbase, e.g, e.sk, 1, 1);
            load_q_at(e.qbase, e.head, e.r_lo, e.s_rows);
        }
    };

    if (wave == 0) {
        // reserve an item when the queue holds at least kReserveItems per workgroup
        const int wg_per_queue = max(1, (int)gridDim.x / nq_queues);
        const bool ahead = plan.total >= kReserveItems * wg_per_queue;
        publish(__builtin_amdgcn_readfirstlane(pop()), 0);
        if (ahead) publish(__builtin_amdgcn_readfirstlane(pop()), 1);
        else if (lane == 0) mbox[4] = -1;
        if (lane == 0) mbox[8] = ahead ? 1 : 0;
    }
    __syncthreads();
    const bool ahead = __builtin_amdgcn_readfirstlane(mbox[8]) != 0;
    Item cur = read_rec(0), nxt = read_rec(1);
    if (cur.a >= 0) issue_prologue(cur);

    int it = 0;                                  // items processed
    for (;; ++it) {
        if (cur.a < 0) break;
        int k_next = 0;
        // per-item timeline (measurement only): one record per item of the first item_slots
        long long* const itr = (args.item_trace != nullptr && tid == 0 && it < args.item_slots)
            ? args.item_trace + ((int64_t)blockIdx.x * args.item_slots + it) * kItemTraceWords : nullptr;
        if (itr != nullptr) itr[0] = (long long)__builtin_amdgcn_s_memrealtime();
        const Geo e = geo(cur);
        const int64_t qbase = e.qbase;
        const int64_t kbase = e.kbase;
        const int s_rows = e.s_rows;
        const int sk = e.sk;
        const int head = e.head;
        const int g = e.g;
        const int r_lo = e.r_lo;
        const int n_units = e.n_units;
        const int n_stages = e.n_stages;

        u32x4 qf[kNT][C::kKS];
        // The fragments go to accumulation registers (AGPRs), which the score product reads as
        // its B operand, through one assembly block that also waits for the reads; left to
        // itself the register allocator moves other operands there and adds copies to every
        // step.
        auto read_q = [&]() {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                const uint32_t b = (uint32_t)__builtin_amdgcn_readfirstlane((int)(lds_addr(qstage) + nt * 32 * C::kRowBytes));
                uint32_t a[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) a[j] = lds_add(b, kofs[j]);
                if constexpr (C::kKS == 8) {
                    asm volatile(
                        "ds_read_b128 %0, %8\n\t"
                        "ds_read_b128 %1, %9\n\t"
                        "ds_read_b128 %2, %10\n\t"
                        "ds_read_b128 %3, %11\n\t"
                        "ds_read_b128 %4, %8 offset:128\n\t"
                        "ds_read_b128 %5, %9 offset:128\n\t"
                        "ds_read_b128 %6, %10 offset:128\n\t"
                        "ds_read_b128 %7, %11 offset:128\n\t"
                        "s_waitcnt lgkmcnt(0)"
                        : "=a"(qf[nt][0]), "=a"(qf[nt][1]), "=a"(qf[nt][2]), "=a"(qf[nt][3]),
                          "=a"(qf[nt][4]), "=a"(qf[nt][5]), "=a"(qf[nt][6]), "=a"(qf[nt][7])
                        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                        : "memory");
                } else {
                    asm volatile(
                        "ds_read_b128 %0, %4\n\t"
                        "ds_read_b128 %1, %5\n\t"
                        "ds_read_b128 %2, %6\n\t"
                        "ds_read_b128 %3, %7\n\t"
                        "s_waitcnt lgkmcnt(0)"
                        : "=a"(qf[nt][0]), "=a"(qf[nt][1]), "=a"(qf[nt][2]), "=a"(qf[nt][3])
                        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                        : "memory");
                }
            }
        };

        // Per-row visibility limit: key j (relative to key 0) is visible to this lane's row of
        // column tile nt iff j <= lim0[nt] (causal) and j < sk.
        int lim0[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
            lim0[nt] = causal ? delta + r_lo + nt * 32 + l32 : sk - 1;

        auto load_stage = [&](int st, int B) { load_stage_at(kbase, g, sk, st, B); };

        // LDS base of a unit's 32 rows: half h of the K (kv = 0) or V (kv = 1) tile of ring
        // buffer buf (uniform)
        auto unit_base = [&](int buf, int h, int kv) {
            return ring0 + (uint32_t)buf * (2 * C::kTileBytes) + (uint32_t)kv * C::kTileBytes +
                   (uint32_t)h * (32 * C::kRowBytes);
        };
        // ring buffers of the current unit's stage and of the next stage load (stage st lives
        // in buffer st mod kStages), advanced by the steps instead of divided
        int cbuf = 0, lbuf = 2;
        // K fragments of the unit in half h of buffer buf (A operand of the score product): 4
        // lane addresses, the k-steps differ by immediate offsets
        auto k_addr = [&](int buf, int h, uint32_t (&a)[4]) {
            const uint32_t kb = unit_base(buf, h, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) a[j] = lds_add(kb, kofs[j]);
        };
        auto read_k = [&](int buf, int h, u32x4 (&kf)[C::kKS]) {
            uint32_t a[4];
            k_addr(buf, h, a);
#pragma unroll
            for (int ks = 0; ks < C::kKS; ++ks)
                kf[ks] = *(const lds_u32x4*)(uintptr_t)(a[ks & 3] + 128 * (ks >> 2));
        };
        // V^T fragments of unit u (A operand of the value product), transposing LDS reads: for
        // k-step ks2 and D tile mt, lane l receives 8 values of column mt*32 + l%32 from the
        // unit's rows 16 ks2 + 8 (i/4) + 4 (l/32) + i%4 (the accumulator row order)
        // (v_addr: the two per-lane column bases of the unit; read_vh: half hi of fragment
        // (ks2, mt); read_v: every fragment)
        auto v_addr = [&](int buf, int h, uint32_t (&a)[2]) {
            const uint32_t vb = unit_base(buf, h, 1);
            a[0] = lds_add(vb, vofs[0]);
            a[1] = lds_add(vb, vofs[1]);
        };
        auto read_vh = [&](const uint32_t (&a)[2], int ks2, int mt, int hi, bf16x8& f) {
            const uint32_t p0 = a[mt & 1] + 128 * (mt >> 1) + 16 * ks2 * C::kRowBytes + hi * 8 * C::kRowBytes;
            const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)p0);
            if (hi) f.hi = __builtin_bit_cast(bf16x4, x);
            else f.lo = __builtin_bit_cast(bf16x4, x);
        };
        auto read_v = [&](int buf, int h, bf16x8 (&vf)[2][C::kMT]) {
            uint32_t a[2];
            v_addr(buf, h, a);
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
                for (int mt = 0; mt < C::kMT; ++mt) {
                    read_vh(a, ks2, mt, 0, vf[ks2][mt]);
                    read_vh(a, ks2, mt, 1, vf[ks2][mt]);
                }
        };
        // S^T (32 keys x 64 rows) = K Q^T
        auto score = [&](const u32x4 (&kf)[C::kKS], f32x16 (&S)[kNT]) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) S[nt] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < C::kKS; ++ks)
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt)
                    S[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, kf[ks]), __builtin_bit_cast(bf16x8, qf[nt][ks]), S[nt], 0, 0, 0);
        };
        // O^T += V^T P^T
        auto value = [&](f32x16 (&oo)[C::kMT][kNT], const bf16x8 (&vf)[2][C::kMT], const bf16x8 (&P)[kNT][2]) {
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
                for (int mt = 0; mt < C::kMT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < kNT; ++nt)
                        oo[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks2][mt], P[nt][ks2], oo[mt][nt], 0, 0, 0);
        };
        // mask of unit u (only units that reach past the diagonal or the last key)
        // Key 8*(i/4) + 4*half + (i%4) of the unit is visible iff it is <= the row's limit; the
        // half-wave term moves into the limit so the comparisons are against constants.
        auto apply_mask = [&](int u, f32x16 (&S)[kNT]) {
            const int j0 = u * kUnit;
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                const int lim = min(lim0[nt], sk - 1) - j0;
                const int li = max(-1, min(lim, kUnit)) - 4 * half;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    S[nt][i] = (8 * (i >> 2) + (i & 3)) > li ? -INFINITY : S[nt][i];
            }
        };
        auto unit_full = [&](int u) {
            const int j0 = u * kUnit;
            return (j0 + kUnit - 1 < sk) && (!causal || j0 + kUnit - 1 <= delta + r_lo);
        };
        // row max of a unit in log2 units (both half-waves); rescale branch only
        auto row_max = [&](const f32x16 (&S)[kNT], float (&tmax)[kNT]) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                float mx = S[nt][0];
#pragma unroll
                for (int i = 1; i < 16; ++i) mx = fmaxf(mx, S[nt][i]);
                tmax[nt] = xhalf_max(mx) * c2;
            }
        };
        // P^T = exp2(S c2 - mr) as bf16 B operands, row sums (fp32, before rounding) into ll
        auto exponentials = [&](const f32x16 (&S)[kNT], const float (&mr)[kNT], float (&ll)[kNT], bf16x8 (&P)[kNT][2]) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                const float mb = mr[nt];
                float ls = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[nt][i], c2, -mb));
                    ls += p;
                    P[nt][i >> 3][i & 7] = (__bf16)p;
                }
                ll[nt] += ls;
            }
        };
        // stage ring (called at odd u only): stage (u+3)/2 goes into the buffer of stage (u-3)/2 (last read
        // in iteration u-1 or earlier); stage (u+1)/2, issued at u-2, must have landed.  A whole
        // stage's loads are not issued here but spread over the value-product slots of step u
        // (spread_k / spread_v / spread_lk / spread_lv): issued back to back right after the
        // barrier, the four waves' loads queue up at once and hold each wave for hundreds of
        // cycles.  The last stage of an item (rows clamped) is loaded here.
        bool spread = false;
        const uint16_t* spread_k = args.k;
        const uint16_t* spread_v = args.v;
        uint32_t spread_lk = 0, spread_lv = 0;
        auto stage_turn = [&](int u) {
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
            __syncthreads();
            const int st = (u + 3) >> 1;
            spread = st < n_stages && st * kStage + kStage <= sk;
            if (spread) {
                const int64_t sofs = (kbase + st * kStage) * kv_stride + (int64_t)g * D;
                spread_k = args.k + sofs;
                spread_v = args.v + sofs;
                spread_lk = ring0 + (uint32_t)lbuf * (2 * C::kTileBytes) + wave * C::kBlocksPerWave * 1024;
                spread_lv = spread_lk + C::kTileBytes;
            } else if (st < n_stages) {
                load_stage(st, lbuf);
            }
            lbuf = lbuf == kStages - 1 ? 0 : lbuf + 1;
        };
        // block i of the spread stage's K tile (i < kBlocksPerWave) or V tile, with the M0
        // handling around the first and last load
        uint32_t spread_m0 = 0;
        auto spread_load = [&](int i) {
            constexpr int NB = C::kBlocksPerWave;
            if (i == 0) spread_m0 = dma_tile_begin(spread_lk);
            if (i == NB) dma_tile_switch(spread_lv);
            const uint16_t* base = i < NB ? spread_k : spread_v;
            switch (i % NB) {
                case 0: dma_tile_load<0>(base, gofs[0]); break;
                case 1: dma_tile_load<1>(base, gofs[1]); break;
                case 2: if constexpr (NB > 2) dma_tile_load<2>(base, gofs[NB > 2 ? 2 : 0]); break;
                default: if constexpr (NB > 3) dma_tile_load<3>(base, gofs[NB > 3 ? 3 : 0]); break;
            }
            if (i == 2 * NB - 1) dma_tile_end(spread_m0);
        };
        // this item's first stages and query rows went out at the end of the previous item (or
        // before the first): wait for them and for the previous item's stores
        auto stage_prologue = [&]() {
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
        };
        // Normalise and write this wave's rows.  The accumulator holds each row split over two
        // lanes in 4-element pieces, so it goes out through a per-wave LDS tile: written there in
        // fragment order, read back so that consecutive lanes cover whole output rows, and stored
        // with 16-byte stores that fill complete cache lines.  A tile is 32 rows x 256 bytes (the
        // output row, or half of it for fp32 at D = 128), slots XOR-swizzled by the row.
        auto store_rows = [&](const f32x16 (&oo)[C::kMT][kNT], const float (&mm)[kNT], const float (&ll)[kNT]) {
            constexpr int kE = MODE == 0 ? 2 : 4;                  // output element bytes
            constexpr int kOutRow = D * kE;
            constexpr int kWb = kOutRow < kStageRowBytes ? kOutRow : kStageRowBytes;
            constexpr int kNB = kOutRow / kWb;                     // column blocks per row
            constexpr int kSlots = kWb / 16;                       // 16-byte slots per tile row
            constexpr int kRowsPerRead = 64 / kSlots;
            unsigned char* tile = obuf[wave];
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                const float lt = xhalf_sum(ll[nt]);
                const float inv = lt > 0.f ? 1.f / lt : 0.f;
                const float mb = (mm[nt] == -INFINITY) ? 0.f : mm[nt];
                const float lse = lt > 0.f ? (mb + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
                const int row0 = r_lo + nt * 32;                   // first row of this tile
                // rows row0 .. row0 + nrows - 1 of this tile exist (none past the sequence's end)
                const int nrows = max(0, min(32, s_rows - row0));
                float fs = inv;                                    // factor on the accumulator
                float lout = lse;
                float a1s = 0.f;                                   // merge: weight on o_acc of row l32
                if constexpr (MODE == 2) {
                    // Merge into the running result by log-sum-exp: with w = exp(lse - m) over
                    // m = max(lse_acc, lse), o = (w_acc o_acc + w o) / (w_acc + w) and
                    // lse = m + ln(w_acc + w).  A row whose lse_acc is -inf has seen no key yet:
                    // its o_acc is ignored; a partial with lse = -inf leaves the row as it was.
                    const int r = row0 + l32;
                    const float la = r < s_rows ? args.lse[(qbase + r) * (int64_t)H + head] : -INFINITY;
                    float a1 = 0.f, a2 = 0.f;
                    if (lse == -INFINITY) {
                        a1 = la == -INFINITY ? 0.f : 1.f;
                        lout = la;
                    } else if (la == -INFINITY) {
                        a2 = 1.f;
                    } else {
                        const float m = fmaxf(la, lse);
                        const float w1 = __builtin_amdgcn_exp2f((la - m) * kLog2e);
                        const float w2 = __builtin_amdgcn_exp2f((lse - m) * kLog2e);
                        const float iw = 1.f / (w1 + w2);
                        a1 = w1 * iw;
                        a2 = w2 * iw;
                        lout = m + __builtin_amdgcn_logf(w1 + w2) * kLn2;
                    }
                    fs = inv * a2;
                    a1s = a1;                                      // (both halves: the row's value)
                }
                buf_store_b32(args.lse + (qbase + row0) * (int64_t)H + head, nrows > 0 ? (uint32_t)((nrows - 1) * H * 4 + 4) : 0u,
                              half == 0 ? (uint32_t)(l32 * H * 4) : kDropOffset, lout);
#pragma unroll
                for (int b = 0; b < kNB; ++b) {
                    // fragment -> tile: lane (row l32, half) holds d = mt*32 + 8*a4 + 4*half + 0..3
#pragma unroll
                    for (int mt = 0; mt < C::kMT; ++mt) {
                        if (mt * 32 * kE < b * kWb || mt * 32 * kE >= (b + 1) * kWb) continue;
#pragma unroll
                        for (int a4 = 0; a4 < 4; ++a4) {
                            const int byte = (mt * 32 + 8 * a4 + 4 * half) * kE - b * kWb;
                            unsigned char* dst = tile + l32 * kWb + (((byte >> 4) ^ (l32 % kSlots)) << 4) + (byte & 15);
                            const float x0 = oo[mt][nt][4 * a4 + 0] * fs, x1 = oo[mt][nt][4 * a4 + 1] * fs;
                            const float x2 = oo[mt][nt][4 * a4 + 2] * fs, x3 = oo[mt][nt][4 * a4 + 3] * fs;
                            if (MODE == 0) {
                                u32x2 w;
                                w[0] = pack_bf16x2(x0, x1);
                                w[1] = pack_bf16x2(x2, x3);
                                *(u32x2*)dst = w;
                            } else {
                                *(float4*)dst = make_float4(x0, x1, x2, x3);
                            }
                        }
                    }
                    // tile -> global: lane i covers slot i % kSlots of tile row i / kSlots (+ step)
                    // (all reads first, so that their latencies overlap)
                    constexpr int kReads = 32 / kRowsPerRead;
                    u32x4 vals[kReads];
#pragma unroll
                    for (int i = 0; i < kReads; ++i) {
                        const int tr = i * kRowsPerRead + lane / kSlots, slot = lane % kSlots;
                        vals[i] = *(const u32x4*)(tile + tr * kWb + ((slot ^ (tr % kSlots)) << 4));
                    }
                    unsigned char* gb = (unsigned char*)args.out + ((qbase + row0) * (int64_t)H + head) * kOutRow + b * kWb;
                    const uint32_t bytes = nrows > 0 ? (uint32_t)((nrows - 1) * H * kOutRow + kWb) : 0u;
                    if constexpr (MODE == 2) {
                        // o = a1 o_acc + (the tile, already scaled by a2); o_acc read where it is
                        // written (rows past the slice's end read 0 and are not stored)
                        u32x4 acc[kReads];
#pragma unroll
                        for (int i = 0; i < kReads; ++i) {
                            const int tr = i * kRowsPerRead + lane / kSlots, slot = lane % kSlots;
                            acc[i] = buf_load_b128(gb, bytes, (uint32_t)(tr * H * kOutRow + slot * 16));
                        }
#pragma unroll
                        for (int i = 0; i < kReads; ++i) {
                            const int tr = i * kRowsPerRead + lane / kSlots;
                            const float a1 = __shfl(a1s, tr);      // from a lane of row tr
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float t = __uint_as_float(vals[i][e]);
                                vals[i][e] = __float_as_uint(a1 != 0.f ? __builtin_fmaf(a1, __uint_as_float(acc[i][e]), t) : t);
                            }
                        }
                    }
#pragma unroll
                    for (int i = 0; i < kReads; ++i) {
                        const int tr = i * kRowsPerRead + lane / kSlots, slot = lane % kSlots;
                        buf_store_b128(gb, bytes, (uint32_t)(tr * H * kOutRow + slot * 16), vals[i]);
                    }
                    if (MODE == 2 && args.out_bf16 != nullptr) {
                        // the merged result also as bf16 (half the byte offsets)
                        unsigned char* gh = (unsigned char*)args.out_bf16 + ((qbase + row0) * (int64_t)H + head) * (kOutRow / 2) + b * (kWb / 2);
                        const uint32_t hbytes = bytes / 2;
#pragma unroll
                        for (int i = 0; i < kReads; ++i) {
                            const int tr = i * kRowsPerRead + lane / kSlots, slot = lane % kSlots;
                            u32x2 w;
                            w[0] = pack_bf16x2(__uint_as_float(vals[i][0]), __uint_as_float(vals[i][1]));
                            w[1] = pack_bf16x2(__uint_as_float(vals[i][2]), __uint_as_float(vals[i][3]));
                            buf_store_b64(gh, hbytes, (uint32_t)(tr * H * (kOutRow / 2) + slot * 8), w);
                        }
                    }
                }
            }
        };

        // ---- software-pipelined units with a lazily rescaled running max ----
        // Step u issues the value product of unit u-1 and the score product of unit u+1 and
        // runs the softmax of unit u; the three are independent.  The running max m is a
        // reference, not necessarily the max: numerator and denominator share it, so the result
        // is exact whatever reference is used as long as no P overflows or all underflow.  It
        // starts at the first unit's row max and is raised (and the accumulator rescaled) only
        // when a lane's sum of P over a unit exceeds 2^8, which keeps every P <= 2^8, and on the
        // first visible unit of a row that saw no key before.
        stage_prologue();
        if (itr != nullptr) {
            itr[1] = (long long)__builtin_amdgcn_s_memrealtime();
            itr[3] = n_units;
        }
        // the item after this one, published by wave 0 at the end of the previous item
        if (ahead && it > 0) nxt = read_rec(0);
        f32x16 o[C::kMT][kNT];
#pragma unroll
        for (int mt = 0; mt < C::kMT; ++mt)
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) o[mt][nt] = f32x16{};
        // m: the reference (-inf before a row's first visible key); mref: the value subtracted
        // in the exponentials (0 while m is -inf), kept beside m so the steps need not derive it
        float m[kNT], mref[kNT], l[kNT], thr[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) { m[nt] = -INFINITY; mref[nt] = 0.f; l[nt] = 0.f; thr[nt] = -1.f; }

        // Runs when some lane's unit sum ls passed its threshold: raises the reference to the
        // row max (in log2 units), rescales what was accumulated before this unit (its sum lb)
        // and recomputes this unit's P and sum.  Rare: a branch after the step.
        auto fix_rescale = [&](f32x16 (&S)[kNT], bf16x8 (&P)[kNT][2], const float (&ls)[kNT],
                               const float (&lb)[kNT]) {
            bool need = false;
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) need |= ls[nt] > thr[nt];
            if (__ballot(need)) {
                float tmax[kNT];
                row_max(S, tmax);
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) {
                    const float mn = fmaxf(m[nt], tmax[nt]);
                    const float alpha = (m[nt] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[nt] - mn);
                    m[nt] = mn;
                    mref[nt] = (mn == -INFINITY) ? 0.f : mn;
                    l[nt] = lb[nt] * alpha;
                    thr[nt] = (mn == -INFINITY) ? -1.f : kLazySum;
#pragma unroll
                    for (int mt = 0; mt < C::kMT; ++mt) o[mt][nt] *= alpha;
                }
                exponentials(S, mref, l, P);
            }
        };

        // Every step has the same shape: step u runs the value product of unit u-1 (P of unit -1
        // is zero), the score product of unit u+1 (discarded after the last unit) and the
        // softmax of unit u, as one straight-line block whose MFMAs the scheduling barriers
        // interleave with the softmax VALU work.  The V^T fragments of unit u are read from LDS
        // in the middle of step u, once the value product of unit u-1 has been issued, so they
        // are in registers when step u+1 starts.  The rare branches come after the block: the
        // rescale of unit u, and the mask of unit u+1 (masked units only reach past the
        // diagonal or the last key, i.e. at the end of an item).  Steps go in pairs that swap
        // the roles of two score and two probability buffers, so no registers are copied
        // between steps.
        // row sum and bf16 packing of score element e (P value pe, the previous element's pp)
        auto sum_pack = [&](int e, float pp, float pe, float (&ls)[kNT], uint32_t (&pw)[kNT][8]) {
            const int nt = e / 16, i = e % 16;
            ls[nt] = i == 0 ? pe : ls[nt] + pe;
            if (i & 1) {
                // the empty asm anchors the conversion in this slot (otherwise it drifts to the
                // end of the step, or into the rare branch)
                pw[nt][i >> 1] = pack_bf16x2(pp, pe);
                asm volatile("" : "+v"(pw[nt][i >> 1]));
            }
        };
        bf16x8 vf[2][C::kMT];
        auto step = [&](int u, bool odd, f32x16 (&Sc)[kNT], f32x16 (&Sn)[kNT], const bf16x8 (&Pp)[kNT][2],
                        bf16x8 (&Pc)[kNT][2]) {
            if (odd) stage_turn(u);
            u32x4 kf[C::kKS];
            // unit u + 1: the second half of this stage (u even) or the first of the next (u odd)
            const int nbuf = cbuf == kStages - 1 ? 0 : cbuf + 1;
            uint32_t ka[4];
            k_addr(odd ? nbuf : cbuf, odd ? 0 : 1, ka);
            __builtin_amdgcn_sched_barrier(0);
            // 32 slots: one MFMA (value-product MFMAs, then score-product MFMAs) and the softmax
            // work of one score element (against the current reference: no dependency on this
            // unit's max), in this order; sched_barrier keeps the order.
            constexpr int kPV = 2 * C::kMT * kNT;
            constexpr int kQK = C::kKS * kNT;
            constexpr int kElems = 16 * kNT;                       // score elements per lane
            constexpr int kSlots = (kPV + kQK) > kElems ? (kPV + kQK) : kElems;
            float ls[kNT], lb[kNT], p1 = 0.f, p2 = 0.f;       // P of the two previous elements
            const float (&mb)[kNT] = mref;
            uint32_t pw[kNT][8];                                   // P as bf16 pairs
            uint32_t va[2];
            constexpr int kVR = 4 * C::kMT;                        // transposing V reads per unit
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                ls[nt] = 0.f;
                lb[nt] = l[nt];
                Sn[nt] = f32x16{};
            }
#pragma unroll
            for (int k = 0; k < kSlots; ++k) {
                if (k >= kPV && k < kPV + kVR) {
                    // V^T of unit u for the next step (its value products of u - 1 are issued),
                    // one read per score-product slot in the order the next step uses them
                    const int j = k - kPV, f = j >> 1;
                    if (j == 0) v_addr(cbuf, odd ? 1 : 0, va);
                    read_vh(va, f / C::kMT, f % C::kMT, j & 1, vf[f / C::kMT][f % C::kMT]);
                }
                if (k < kPV && (k % (kPV / C::kKS)) == 0) {
                    // K of unit u + 1, spread over the value-product slots
                    const int ks = k / (kPV / C::kKS);
                    kf[ks] = *(const lds_u32x4*)(uintptr_t)(ka[ks & 3] + 128 * (ks >> 2));
                }
                if (odd && (k & 1) == 0 && k / 2 < 2 * C::kBlocksPerWave && spread) spread_load(k / 2);
                if (k >= kPV + kQK) {
                    // (D = 64: more score elements than MFMAs)
                } else if (k < kPV) {
                    const int ks2 = k / (C::kMT * kNT), mt = (k / kNT) % C::kMT, nt = k % kNT;
                    o[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks2][mt], Pp[nt][ks2], o[mt][nt], 0, 0, 0);
                } else {
                    const int ks = (k - kPV) / kNT, nt = (k - kPV) % kNT;
                    Sn[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, kf[ks]), __builtin_bit_cast(bf16x8, qf[nt][ks]), Sn[nt], 0, 0, 0);
                }
                // score element e = k of this unit: its exponential here, its sum and bf16
                // packing one slot later, so that no instruction right after v_exp reads its
                // result (a transcendental result needs a wait state before a VALU reads it)
                if (k < kElems) {
                    const int nt = k / 16, i = k % 16;
                    const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(Sc[nt][i], c2, -mb[nt]));
                    if (k > 0) sum_pack(k - 1, p2, p1, ls, pw);
                    p2 = p1;
                    p1 = pv;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            sum_pack(kElems - 1, p2, p1, ls, pw);
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                l[nt] += ls[nt];
                asm volatile("" : "+v"(l[nt]));
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    Pc[nt][h] = __builtin_bit_cast(bf16x8, u32x4{pw[nt][4 * h], pw[nt][4 * h + 1], pw[nt][4 * h + 2],
                                                                 pw[nt][4 * h + 3]});
            }
            fix_rescale(Sc, Pc, ls, lb);
            if (u + 1 < n_units && !unit_full(u + 1)) apply_mask(u + 1, Sn);
            if (odd) cbuf = nbuf;
        };
        if (n_units > 0) {
            f32x16 SA[kNT], SB[kNT];
            bf16x8 PA[kNT][2], PB[kNT][2];
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                PA[nt][0] = bf16x8{};
                PA[nt][1] = bf16x8{};
            }
            read_q();
            {
                u32x4 kf[C::kKS];
                read_k(0, 0, kf);
                score(kf, SA);
            }
            read_v(0, 0, vf);   // multiplied by the zero P of unit -1
            if (!unit_full(0)) apply_mask(0, SA);
            // the reference starts at the first unit's row max, so the first step takes no
            // rescale branch (a row whose first unit is wholly masked keeps -inf and takes it)
            {
                float tmax[kNT];
                row_max(SA, tmax);
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) {
                    const bool none = tmax[nt] == -INFINITY;
                    m[nt] = tmax[nt];
                    mref[nt] = none ? 0.f : tmax[nt];
                    thr[nt] = none ? -1.f : kLazySum;
                }
            }
            int u = 0;
            for (; u + 1 < n_units; u += 2) {
                step(u, false, SA, SB, PA, PB);
                step(u + 1, true, SB, SA, PB, PA);
            }
            // vf holds unit n-1 after its step
            if (u < n_units) {
                step(u, false, SA, SB, PA, PB);
                value(o, vf, PB);
            } else {
                value(o, vf, PA);
            }
        }
        if (itr != nullptr) itr[2] = (long long)__builtin_amdgcn_s_memrealtime();
        if (ahead) {
            // Every wave is done with the ring and the Q staging: the item after the next is
            // taken and the next item's first loads go out, both under the output stores.
            __syncthreads();
            if (wave == 0 && nxt.a >= 0) k_next = pop();
            if (nxt.a >= 0) issue_prologue(nxt);
            store_rows(o, m, l);
            if (wave == 0 && nxt.a >= 0) publish(__builtin_amdgcn_readfirstlane(k_next), 0);
            cur = nxt;
        } else {
            // The next item is taken only now, when this workgroup is about to be free.  Its
            // record is in the mailbox after the barrier, and its first loads go out then.
            if (wave == 0) k_next = pop();
            store_rows(o, m, l);
            if (wave == 0) publish(__builtin_amdgcn_readfirstlane(k_next), 0);
            __syncthreads();
            cur = read_rec(0);
            if (cur.a >= 0) issue_prologue(cur);
        }
    }

    if (tid == 0) {
        if (args.trace != nullptr) {
            long long* t = args.trace + (int64_t)blockIdx.x * kTraceWords;
            t[1] = (long long)__builtin_amdgcn_s_memrealtime();
            t[2] = it;
            t[3] = 0;
        }
        queue_finish(args.counters);
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

hipError_t launch_fwd_chunk_merge(const FwdArgs& a, int D, int grid, hipStream_t s) {
    if (D == 128) hipLaunchKernelGGL((fwd_kernel<128, 2>), dim3(grid), dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((fwd_kernel<64, 2>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace hdp
