// Packed variable-length causal attention, forward, fp32 throughout.
//
// The small fp32 form of the rank's packed slice (research digest "ByteScale: Communication-
// Efficient Scaling of LLM Training with a 2048K Context Length on 16384 GPUs", §3.1-§3.2:
// packed sequences, each attending only to itself; §4: causal).  Fp32 has no dense MFMA
// advantage worth the layout work at the sizes this form is used for, so it runs on the vector
// ALUs: one wave per query row at a time, its lanes over the head dimension (lane d holds
// elements d, d + 64, ...), so each key's K and V rows are single coalesced loads and the dot
// product is a cross-lane sum.  Keys go four at a time (four independent sums in flight) through
// an online softmax in ascending key order.  Grid: (sequence, head, 8 row groups) of 4 waves,
// each wave taking every 32nd row of its sequence.
#include <type_traits>

#include "hdp_internal.h"

namespace hdp {
namespace {

constexpr int kThreads = 256;
constexpr int kRowGroups = 8;                    // grid z: waves per (sequence, head) = 8 x 4
constexpr float kLn2 = 0.693147180559945309f;

// Sum over the 64 lanes of a wave, the same value in every lane: DPP sums within each row of 16
// lanes (swap neighbours, swap pairs, mirror halves, mirror the row), then the four row sums are
// read out and added in a fixed order.
template <int CTRL>
__device__ inline float dpp_add(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int N>
__device__ inline void wave_sums(float (&x)[N]) {
#pragma unroll
    for (int u = 0; u < N; ++u) x[u] = dpp_add<0xB1>(x[u]);    // quad_perm [1,0,3,2]
#pragma unroll
    for (int u = 0; u < N; ++u) x[u] = dpp_add<0x4E>(x[u]);    // quad_perm [2,3,0,1]
#pragma unroll
    for (int u = 0; u < N; ++u) x[u] = dpp_add<0x141>(x[u]);   // row_half_mirror
#pragma unroll
    for (int u = 0; u < N; ++u) x[u] = dpp_add<0x140>(x[u]);   // row_mirror
#pragma unroll
    for (int u = 0; u < N; ++u) {
        const int b = __builtin_bit_cast(int, x[u]);
        x[u] = (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
                __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
               (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
                __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(F32Args a) {
    constexpr int kE = D / 64;                   // elements per lane
    const int seq = blockIdx.x;
    const int head = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wid = (int)blockIdx.z * (kThreads / 64) + (int)(threadIdx.x >> 6);
    const int nw = (int)gridDim.z * (kThreads / 64);
    const int G = a.H / a.Hkv;
    const int g = head / G;
    const int Tc = max(a.cu[a.n_seq], 0);
    const int s0 = min(max(a.cu[seq], 0), Tc);
    const int s1 = min(max(a.cu[seq + 1], s0), Tc);
    const int len = s1 - s0;
    const int64_t qs = (int64_t)a.H * D, ks = (int64_t)a.Hkv * D;
    const float* kb = a.k + (int64_t)s0 * ks + (int64_t)g * D + lane;
    const float* vb = a.v + (int64_t)s0 * ks + (int64_t)g * D + lane;
    for (int r = wid; r < len; r += nw) {
        const float* qr = a.q + (int64_t)(s0 + r) * qs + (int64_t)head * D + lane;
        float q[kE], acc[kE];
#pragma unroll
        for (int e = 0; e < kE; ++e) { q[e] = qr[64 * e]; acc[e] = 0.f; }
        float m = -INFINITY, l = 0.f;
        // keys j .. j + n - 1 (n = 4, or 1 for the last few), all visible to row r
        auto block = [&](int j, auto nkeys) {
            constexpr int n = decltype(nkeys)::value;
            float x[n], vv[n][kE];
#pragma unroll
            for (int u = 0; u < n; ++u) {
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < kE; ++e) {
                    dot = __builtin_fmaf(q[e], kb[(int64_t)(j + u) * ks + 64 * e], dot);
                    vv[u][e] = vb[(int64_t)(j + u) * ks + 64 * e];
                }
                x[u] = dot;
            }
            wave_sums(x);
            float mx = m;
#pragma unroll
            for (int u = 0; u < n; ++u) {
                x[u] *= a.scale_log2;
                mx = fmaxf(mx, x[u]);
            }
            if (mx > m) {                        // uniform: every lane holds the same sums
                const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mx);
                l *= alpha;
#pragma unroll
                for (int e = 0; e < kE; ++e) acc[e] *= alpha;
                m = mx;
            }
#pragma unroll
            for (int u = 0; u < n; ++u) {
                const float p = __builtin_amdgcn_exp2f(x[u] - m);
                l += p;
#pragma unroll
                for (int e = 0; e < kE; ++e) acc[e] = __builtin_fmaf(p, vv[u][e], acc[e]);
            }
        };
        int j = 0;
        for (; j + 4 <= r + 1; j += 4) block(j, std::integral_constant<int, 4>{});
        for (; j <= r; ++j) block(j, std::integral_constant<int, 1>{});
        const float inv = 1.f / l;
        float* orow = a.out + (int64_t)(s0 + r) * qs + (int64_t)head * D + lane;
#pragma unroll
        for (int e = 0; e < kE; ++e) orow[64 * e] = acc[e] * inv;
        if (lane == 0) a.lse[(int64_t)(s0 + r) * a.H + head] = (m + __builtin_amdgcn_logf(l)) * kLn2;
    }
}

}  // namespace

hipError_t launch_fwd_f32(const F32Args& a, hipStream_t s) {
    dim3 grid(a.n_seq, a.H, kRowGroups);
    if (a.D == 128) hipLaunchKernelGGL((fwd_f32_kernel<128>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((fwd_f32_kernel<64>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace hdp
