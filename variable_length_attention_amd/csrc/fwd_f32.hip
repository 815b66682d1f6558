// Packed variable-length causal attention, forward, fp32 throughout.
//
// The small fp32 form of the rank's packed slice (research digest "ByteScale: Communication-
// Efficient Scaling of LLM Training with a 2048K Context Length on 16384 GPUs", §3.1-§3.2:
// packed sequences, each attending only to itself; §4: causal).  Fp32 has no dense MFMA
// advantage worth the layout work at the sizes this form is used for, so it runs on the vector
// ALUs.  A workgroup takes 16 consecutive query rows of one (sequence, head); each wave holds 4
// of them, one per group of 16 lanes (lane i of a group holds elements 4i .. 4i+3 of each 64-wide
// slice of the row), so a K or V row is one coalesced 256-byte read per slice, a dot product is
// an in-lane sum plus four DPP steps within the group, and the wave's four rows advance together.
// The keys the 16 rows see are staged in LDS in chunks (128 KB of K and V) by direct global->LDS
// loads, all in flight together, so the key loop reads LDS rather than waiting on memory; the
// online softmax runs in ascending key order, four keys at a time.  Grid: (sequence, head, 8
// row-block strides).
#include <type_traits>

#include "device_common.h"

namespace hdp {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBlocks = 8;                    // grid z: a workgroup takes row blocks z, z + 8, ...
constexpr int kBlockRows = 16;                   // rows per workgroup pass: 4 waves x 4 groups
constexpr float kLn2 = 0.693147180559945309f;

// Sum over the 16 lanes of a DPP row, the same value in every lane of the row: swap neighbours,
// swap pairs, mirror the half-rows, mirror the row.
template <int CTRL>
__device__ inline float dpp_add(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ inline float row16_sum(float x) {
    x = dpp_add<0xB1>(x);    // quad_perm [1,0,3,2]
    x = dpp_add<0x4E>(x);    // quad_perm [2,3,0,1]
    x = dpp_add<0x141>(x);   // row_half_mirror
    return dpp_add<0x140>(x);   // row_mirror
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void fwd_f32_kernel(F32Args a) {
    constexpr int kS = D / 64;                   // 64-wide slices of a row: float4 per lane each
    constexpr int kChunk = 128 * 128 / D;        // keys per LDS chunk: 128 (D = 128) or 256 (D = 64)
    __shared__ float4 kl[kChunk * D / 4];
    __shared__ float4 vl[kChunk * D / 4];
    const int seq = blockIdx.x;
    const int head = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar LDS bases
    const int grp = lane >> 4;                   // this lane's row within the wave
    const int li = lane & 15;
    const int G = a.H / a.Hkv;
    const int g = head / G;
    const int Tc = max(a.cu[a.n_seq], 0);
    const int s0 = min(max(a.cu[seq], 0), Tc);
    const int s1 = min(max(a.cu[seq + 1], s0), Tc);
    const int len = s1 - s0;
    const int64_t qs = (int64_t)a.H * D, ks = (int64_t)a.Hkv * D;
    for (int rb = blockIdx.z; rb * kBlockRows < len; rb += gridDim.z) {
        const int r = rb * kBlockRows + wave * 4 + grp;     // this group's row
        const int rr = min(r, len - 1);                    // rows past the end repeat the last
        const int kmax = min(rb * kBlockRows + kBlockRows - 1, len - 1);   // last key of the block
        const int wmax = min(rb * kBlockRows + wave * 4 + 3, len - 1);     // last key of the wave
        const float* qr = a.q + (int64_t)(s0 + rr) * qs + (int64_t)head * D + 4 * li;
        float4 q[kS], acc[kS];
#pragma unroll
        for (int v = 0; v < kS; ++v) {
            q[v] = *(const float4*)(qr + 64 * v);
            acc[v] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float m = -INFINITY, l = 0.f;
        for (int c0 = 0; c0 <= kmax; c0 += kChunk) {
            const int nk = min(kChunk, kmax + 1 - c0);
            __syncthreads();                             // the previous chunk's reads are done
            // 1 KB blocks (64 lanes x 16 bytes, kRowsPer rows) of the chunk, the waves in turn;
            // rows past the chunk's last key repeat it (not read)
            constexpr int kRowsPer = 1024 / (D * 4);
            const int nblk = (nk + kRowsPer - 1) / kRowsPer;
            for (int b = wave; b < nblk; b += kThreads / 64) {
                const int key = min(b * kRowsPer + lane / (D / 4), nk - 1);
                const int64_t off = (int64_t)(s0 + c0 + key) * ks + (int64_t)g * D + 4 * (lane % (D / 4));
                lds_dma16(a.k + off, lds_addr(&kl[b * 64]));
                lds_dma16(a.v + off, lds_addr(&vl[b * 64]));
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): the block's loads (and q) landed
            __syncthreads();
            // keys c0 .. c0 + jend - 1 are visible to this group's row; the wave runs to its
            // longest row's end, the other groups see -inf there
            const int jend = min(nk, rr + 1 - c0);
            const int jw = min(nk, wmax + 1 - c0);
            for (int j = 0; j < jw; j += 4) {
                float x[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int kk = min(j + u, nk - 1);
                    float dot = 0.f;
#pragma unroll
                    for (int v = 0; v < kS; ++v) {
                        const float4 kv = kl[kk * (D / 4) + 16 * v + li];
                        dot = __builtin_fmaf(q[v].x, kv.x, dot);
                        dot = __builtin_fmaf(q[v].y, kv.y, dot);
                        dot = __builtin_fmaf(q[v].z, kv.z, dot);
                        dot = __builtin_fmaf(q[v].w, kv.w, dot);
                    }
                    x[u] = dot;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) x[u] = row16_sum(x[u]);
                float mx = m;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    x[u] = j + u < jend ? x[u] * a.scale_log2 : -INFINITY;
                    mx = fmaxf(mx, x[u]);
                }
                if (mx > m) {
                    const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mx);
                    l *= alpha;
#pragma unroll
                    for (int v = 0; v < kS; ++v) {
                        acc[v].x *= alpha;
                        acc[v].y *= alpha;
                        acc[v].z *= alpha;
                        acc[v].w *= alpha;
                    }
                    m = mx;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    // an invisible key (x = -inf) adds nothing; m is finite from key 0 on
                    const float p = x[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x[u] - m);
                    l += p;
                    const int kk = min(j + u, nk - 1);
#pragma unroll
                    for (int v = 0; v < kS; ++v) {
                        const float4 vv = vl[kk * (D / 4) + 16 * v + li];
                        acc[v].x = __builtin_fmaf(p, vv.x, acc[v].x);
                        acc[v].y = __builtin_fmaf(p, vv.y, acc[v].y);
                        acc[v].z = __builtin_fmaf(p, vv.z, acc[v].z);
                        acc[v].w = __builtin_fmaf(p, vv.w, acc[v].w);
                    }
                }
            }
        }
        if (r < len) {
            const float inv = 1.f / l;
            float* orow = a.out + (int64_t)(s0 + r) * qs + (int64_t)head * D + 4 * li;
#pragma unroll
            for (int v = 0; v < kS; ++v)
                *(float4*)(orow + 64 * v) = make_float4(acc[v].x * inv, acc[v].y * inv, acc[v].z * inv, acc[v].w * inv);
            if (li == 0) a.lse[(int64_t)(s0 + r) * a.H + head] = (m + __builtin_amdgcn_logf(l)) * kLn2;
        }
    }
}

}  // namespace

hipError_t launch_fwd_f32(const F32Args& a, hipStream_t s) {
    dim3 grid(a.n_seq, a.H, kRowBlocks);
    if (a.D == 128) hipLaunchKernelGGL((fwd_f32_kernel<128>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((fwd_f32_kernel<64>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace hdp
