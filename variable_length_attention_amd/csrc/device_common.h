// Device helpers shared by the attention kernels: vector types, wave reductions, bf16 packing
// and the longest-first work queue over (sequence, head block, tile) items.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

#include "hdp_internal.h"

namespace hdp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// LDS byte address of a pointer into a __shared__ array
__device__ inline uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_void*)p;
}
// base + off behind an optimisation barrier: the optimiser cannot re-associate the sum with
// the immediates added later, so those stay instruction offsets of the LDS reads
__device__ inline uint32_t lds_add(uint32_t base, uint32_t off) {
    uint32_t r = base + off;
    asm volatile("" : "+v"(r));
    return r;
}

// Direct global->LDS loads (the CDNA LDS DMA): every lane reads 16 (or 4) bytes at its own
// global address and the wave writes them to LDS at lds + 16 * lane (or 4 * lane), without
// passing through registers.  lds is wave-uniform and goes to M0, which is saved and restored
// around the load.  The loads are issued from inline assembly on purpose: the compiler cannot
// tell which LDS bytes a DMA writes, so for the builtin it waits for every outstanding global
// load before the next LDS read of any buffer, which exposes the full memory latency once per
// stage.  Callers order the loads against LDS reads themselves: s_waitcnt vmcnt and a workgroup
// barrier before any wave reads a buffer that a load wrote.
__device__ inline void lds_dma16(const void* g, uint32_t lds) {
    uint32_t m0_saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0_saved) : "v"(g), "s"(lds) : "memory");
}
__device__ inline void lds_dma4(const void* g, uint32_t lds) {
    uint32_t m0_saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, off\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0_saved) : "v"(g), "s"(lds) : "memory");
}

// Groups of direct global->LDS loads of 16 bytes per lane in the scalar-base form: lane l reads
// at sbase + voff[i] (a uniform 64-bit base in SGPRs plus a 32-bit per-lane byte offset, so no
// 64-bit vector address arithmetic per load) and the wave writes LDS at lds[i] + 16 * l.  Two
// streams (two bases, e.g. K and V, or Q and dO) share the per-lane offsets: load i of stream s
// goes to lds_s + 1024 * i.  M0 is saved once, set before each load with one wait state on
// either side of the load, and restored once.  Ordering against LDS reads is the caller's, as
// for lds_dma16.
template <int N>
__device__ inline void lds_dma16_pairs(const void* sbase0, const void* sbase1, const uint32_t (&voff)[N],
                                       uint32_t lds0, uint32_t lds1) {
    static_assert(N == 1 || N == 2 || N == 4, "groups of 1, 2 or 4 loads per stream");
    uint32_t m0_saved;
    if constexpr (N == 1) {
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %4\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %2\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %5\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %3\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(m0_saved)
            : "v"(voff[0]), "s"(sbase0), "s"(sbase1), "s"(lds0 + 0u), "s"(lds1 + 0u)
            : "memory");
    } else if constexpr (N == 2) {
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %5\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %3\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %6\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %2, %3\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %7\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %4\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %8\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %2, %4\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(m0_saved)
            : "v"(voff[0]), "v"(voff[1]), "s"(sbase0), "s"(sbase1), "s"(lds0 + 0u), "s"(lds0 + 1024u), "s"(lds1 + 0u), "s"(lds1 + 1024u)
            : "memory");
    } else {
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %7\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %5\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %8\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %2, %5\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %9\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %3, %5\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %10\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %4, %5\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %11\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %6\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %12\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %2, %6\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %13\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %3, %6\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %14\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %4, %6\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(m0_saved)
            : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(sbase0), "s"(sbase1), "s"(lds0 + 0u), "s"(lds0 + 1024u), "s"(lds0 + 2048u), "s"(lds0 + 3072u), "s"(lds1 + 0u), "s"(lds1 + 1024u), "s"(lds1 + 2048u), "s"(lds1 + 3072u)
            : "memory");
    }
}
// Two tiles of N direct global->LDS loads of 16 bytes per lane in the scalar-base form, with
// one M0 write per tile: the instruction's immediate offset moves the global and the LDS address
// alike, so load i of stream s reads sbase_s + voffb[i] + 1024 i and writes lds_s + 1024 i +
// 16 * lane.  voffb[i] is therefore the lane's byte offset of block i minus 1024 i (it must not
// be negative: the per-lane offset is unsigned).  One wait state separates each M0 write from
// the loads that read it.  Ordering against LDS reads is the caller's, as for lds_dma16.
template <int N>
__device__ inline void lds_dma16_tiles(const void* sbase0, const void* sbase1, const uint32_t (&voffb)[N],
                                       uint32_t lds0, uint32_t lds1) {
    static_assert(N == 2 || N == 4, "tiles of 2 or 4 loads");
    uint32_t m0_saved;
    if constexpr (N == 2) {
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %5\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %3\n\t"
            "global_load_lds_dwordx4 %2, %3 offset:1024\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %6\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %4\n\t"
            "global_load_lds_dwordx4 %2, %4 offset:1024\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(m0_saved)
            : "v"(voffb[0]), "v"(voffb[1]), "s"(sbase0), "s"(sbase1), "s"(lds0), "s"(lds1)
            : "memory");
    } else {
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %7\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %5\n\t"
            "global_load_lds_dwordx4 %2, %5 offset:1024\n\t"
            "global_load_lds_dwordx4 %3, %5 offset:2048\n\t"
            "global_load_lds_dwordx4 %4, %5 offset:3072\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %8\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %6\n\t"
            "global_load_lds_dwordx4 %2, %6 offset:1024\n\t"
            "global_load_lds_dwordx4 %3, %6 offset:2048\n\t"
            "global_load_lds_dwordx4 %4, %6 offset:3072\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(m0_saved)
            : "v"(voffb[0]), "v"(voffb[1]), "v"(voffb[2]), "v"(voffb[3]), "s"(sbase0), "s"(sbase1), "s"(lds0), "s"(lds1)
            : "memory");
    }
}
// The pieces of lds_dma16_tiles issued one at a time, so that a stage's loads can be spread
// between other instructions: dma_tile_begin saves M0 and points it at a tile's LDS base,
// dma_tile_load issues block I of the tile (global sbase + voffb + 1024 I, LDS M0 + 1024 I +
// 16 * lane; voffb as for lds_dma16_tiles), dma_tile_switch points M0 at the next tile and
// dma_tile_end restores M0.  Between begin and end nothing else may write M0 (the callers' code
// there uses no instruction that does: checked in the generated code).
__device__ inline uint32_t dma_tile_begin(uint32_t lds) {
    uint32_t m0_saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0" : "=&s"(m0_saved) : "s"(lds) : "memory");
    return m0_saved;
}
__device__ inline void dma_tile_switch(uint32_t lds) {
    asm volatile("s_nop 0\n\ts_mov_b32 m0, %0\n\ts_nop 0" :: "s"(lds) : "memory");
}
template <int I>
__device__ inline void dma_tile_load(const void* sbase, uint32_t voffb) {
    asm volatile("global_load_lds_dwordx4 %0, %1 offset:%2" :: "v"(voffb), "s"(sbase), "n"(1024 * I) : "memory");
}
__device__ inline void dma_tile_end(uint32_t m0_saved) {
    asm volatile("s_nop 0\n\ts_mov_b32 m0, %0" :: "s"(m0_saved) : "memory");
}
// One direct load of 4 bytes per lane in the scalar-base form (sbase + voff -> lds + 4 * lane).
__device__ inline void lds_dma4_s(const void* sbase, uint32_t voff, uint32_t lds) {
    uint32_t m0_saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0_saved) : "v"(voff), "s"(sbase), "s"(lds) : "memory");
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.693147180559945309f;

// Max / sum of a value over lanes l and l^32 (the two half-waves), result in every lane.
__device__ inline float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Whole-wave integer reductions, returned as a uniform value: DPP moves reduce each row of 16
// lanes (swap neighbours, swap pairs, mirror halves, mirror the row), then the four row results
// are read out as scalars.  No LDS round trips.
__device__ inline int row16_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
    x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
    x += __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);   // row_half_mirror
    x += __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);   // row_mirror
    return x;
}
__device__ inline int row16_max(int x) {
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false));
    return x;
}
__device__ inline int wave_sum(int x) {
    x = row16_sum(x);
    return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) +
           __builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48);
}
__device__ inline int wave_max(int x) {
    x = row16_max(x);
    return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
               max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
// Stores through a raw buffer resource that covers `bytes` from `base`: a lane whose offset
// lies outside is dropped by the hardware, so every lane of a wave issues the same store
// instructions whatever rows exist.  That keeps the count of the wave's outstanding vector
// memory operations fixed, so a later wait for an older operation (the queue pop) can leave
// the stores in flight.  base and bytes are the same in every lane; reading them from the
// first lane tells the compiler so.
__device__ inline __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
    const int n = __builtin_amdgcn_readfirstlane((int)bytes);
    // 0x00020000: 32-bit data format, the raw (untyped) buffer setting of this GPU family
    return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0, n, 0x00020000);
}
__device__ inline void buf_store_b128(void* base, uint32_t bytes, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, uniform_rsrc(base, bytes), off, 0, 0);
}
__device__ inline void buf_store_b32(void* base, uint32_t bytes, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), uniform_rsrc(base, bytes), off, 0, 0);
}
__device__ inline void buf_store_b64(void* base, uint32_t bytes, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, uniform_rsrc(base, bytes), off, 0, 0);
}
// Loads through the same kind of resource: a lane whose offset lies outside reads zeros.
__device__ inline u32x4 buf_load_b128(const void* base, uint32_t bytes, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(uniform_rsrc(base, bytes), off, 0, 0);
}
// Beyond every resource the kernels build: the largest covers 32 rows of H <= 65535 heads of
// 512-byte rows, under 2^30 bytes.
constexpr uint32_t kDropOffset = 0x80000000u;

// Two floats to two bf16 (round to nearest even) in one dword, first in the low half.
__device__ inline uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// LDS slot swizzle of a row: the 16-byte slot holding chunk c of row r is c ^ swz(r).  swz maps
// any 8 consecutive rows to 8 different values (score-operand reads: 32 rows, one chunk) and
// any 4 rows 4k..4k+3 to values whose pairwise XOR is neither 0 nor 1 (transposing reads: 4
// rows x 2 adjacent chunks), so neither read kind hits a bank twice in one LDS cycle.
__device__ inline int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

// Sequence i clamped to [0, Tc]: start and length.  Malformed cu_seqlens give empty sequences.
__device__ inline void seq_span(const int32_t* cu, int i, int Tc, int& a, int& len) {
    int s0 = min(max(cu[i], 0), Tc);
    int s1 = min(max(cu[i + 1], s0), Tc);
    a = s0;
    len = s1 - s0;
}

// ---------------------------------------------------------------------------------------------
// Longest-first queue.  Sequence i contributes ntiles_i = ceil(len_i / W) tiles for each of the
// queue's head blocks; a tile's cost level c runs from 1 to ntiles_i (the caller maps c to a
// tile so that cost grows with c).  Items are handed out level by level from the top, which is
// longest-processing-time-first order; within a level any order is equivalent.  Everything is
// derived from cu_seqlens on the device by one wave.
// ---------------------------------------------------------------------------------------------
struct QueuePlan {
    int total;   // items in this queue
    int maxc;    // highest level
    int Tc;      // clamped token count
    int nt0;     // tile count of sequence `lane` (0 past n_seq): the first 64 sequences stay in
                 // registers, so decoding touches memory only for sequences 64 and up
    int st0;     // start and length of sequence `lane` (clamped)
    int ln0;
    int la;      // with at most 64 sequences and 64 levels (fast): items above level lane + 1,
    int fast;    // per head block, so decoding is a wave vote instead of a search
};

__device__ inline int seq_tiles(const int32_t* cu, int i, int Tc, int W) {
    int a, len;
    seq_span(cu, i, Tc, a, len);
    return (len + W - 1) / W;
}

// sum_i max(0, ntiles_i - c)
__device__ inline int levels_above(const int32_t* cu, int n_seq, const QueuePlan& p, int W, int c, int lane) {
    int acc = max(0, p.nt0 - c);
    for (int i = lane + 64; i < n_seq; i += 64) acc += max(0, seq_tiles(cu, i, p.Tc, W) - c);
    return wave_sum(acc);
}

// Tbound caps the token count (the caller's row count when it is known).
__device__ inline QueuePlan queue_plan(const int32_t* cu, int n_seq, int W, int nhbq, int lane,
                                       int Tbound = 0x7fffffff) {
    QueuePlan p;
    p.Tc = min(max(cu[n_seq], 0), Tbound);
    p.st0 = 0;
    p.ln0 = 0;
    if (lane < n_seq) seq_span(cu, lane, p.Tc, p.st0, p.ln0);
    p.nt0 = (p.ln0 + W - 1) / W;
    int sum = p.nt0, mx = p.nt0;
    for (int i = lane + 64; i < n_seq; i += 64) {
        const int nt = seq_tiles(cu, i, p.Tc, W);
        sum += nt;
        mx = max(mx, nt);
    }
    p.total = wave_sum(sum) * nhbq;
    p.maxc = wave_max(mx);
    p.la = 0;
    p.fast = n_seq <= 64 && p.maxc <= 64;
    if (p.fast) {
        for (int i = 0; i < n_seq; ++i) p.la += max(0, __builtin_amdgcn_readlane(p.nt0, i) - (lane + 1));
    }
    return p;
}

// Item k (< total) of the queue -> sequence (a, len), head block index within the queue, level.
// Returns false only if the plan does not match cu_seqlens (never for k < total).
__device__ inline bool queue_decode(const int32_t* cu, int n_seq, const QueuePlan& p, int W, int nhbq,
                                    int k, int lane, int& a, int& len, int& hbq, int& c) {
    int j;
    if (p.fast) {
        // levels_above falls with the level: the smallest level c with levels_above(c) * nhbq
        // <= k is the lowest lane that votes yes (lane c - 1 holds level c)
        const uint64_t m = __ballot(lane < p.maxc && p.la * nhbq <= k);
        c = (int)__builtin_ctzll(m) + 1;
        j = k - __builtin_amdgcn_readlane(p.la, c - 1) * nhbq;
    } else {
        int lo = 1, hi = p.maxc;   // smallest level with levels_above(level) * nhbq <= k
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (levels_above(cu, n_seq, p, W, mid, lane) * nhbq <= k) hi = mid;
            else lo = mid + 1;
        }
        c = lo;
        j = k - levels_above(cu, n_seq, p, W, c, lane) * nhbq;
    }
    int r = j / nhbq;
    hbq = j % nhbq;
    int seq = -1;
    for (int i0 = 0; i0 < n_seq && seq < 0; i0 += 64) {
        const int i = i0 + lane;
        bool ok = false;
        if (i < n_seq) ok = (i0 == 0 ? p.nt0 : seq_tiles(cu, i, p.Tc, W)) >= c;
        const uint64_t m = __ballot(ok);
        const int cnt = __popcll(m);
        if (r < cnt) {
            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            const uint64_t hit = __ballot(ok && below == r);
            seq = i0 + (int)__builtin_ctzll(hit);
        } else {
            r -= cnt;
        }
    }
    if (seq < 0) return false;
    if (seq < 64) {
        a = __builtin_amdgcn_readlane(p.st0, seq);
        len = __builtin_amdgcn_readlane(p.ln0, seq);
    } else {
        seq_span(cu, seq, p.Tc, a, len);
    }
    return true;
}

// Called by thread 0 of every workgroup after its last pop: the last one out resets the
// queue counters of both sets, so they are zero again for the next launch on the stream.
__device__ inline void queue_finish(int* counters) {
    __threadfence();
    int* done = &counters[kMaxQueues * kQueueStride];
    if (atomicAdd(done, 1) == (int)gridDim.x - 1) {
        for (int set = 0; set < 2; ++set)
            for (int qi = 0; qi < kMaxQueues; ++qi) atomicExch(&counters[set * kCounterSetInts + qi * kQueueStride], 0);
        atomicExch(done, 0);
        __threadfence();
    }
}

}  // namespace hdp
