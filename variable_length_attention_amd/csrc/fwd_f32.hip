// Packed variable-length causal attention, forward, fp32 throughout.
//
// The small fp32 form of the rank's packed slice (research digest "ByteScale: Communication-
// Efficient Scaling of LLM Training with a 2048K Context Length on 16384 GPUs", §3.1-§3.2:
// packed sequences, each attending only to itself; §4: causal).  Fp32 has no dense MFMA
// advantage worth the layout work at the sizes this form is used for, so it runs on the vector
// ALUs: one workgroup per (sequence, head), one lane per query row, an online softmax over the
// row's keys in ascending order, K/V rows read through the caches.
#include "hdp_internal.h"

namespace hdp {
namespace {

constexpr int kThreads = 256;
constexpr float kLn2 = 0.693147180559945309f;

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(F32Args a) {
    const int seq = blockIdx.x;
    const int head = blockIdx.y;
    const int G = a.H / a.Hkv;
    const int g = head / G;
    const int Tc = max(a.cu[a.n_seq], 0);
    const int s0 = min(max(a.cu[seq], 0), Tc);
    const int s1 = min(max(a.cu[seq + 1], s0), Tc);
    const int len = s1 - s0;
    const int64_t qs = (int64_t)a.H * D, ks = (int64_t)a.Hkv * D;
    for (int r = threadIdx.x; r < len; r += kThreads) {
        const float* qr = a.q + (int64_t)(s0 + r) * qs + (int64_t)head * D;
        float q[D], acc[D];
#pragma unroll
        for (int d = 0; d < D; ++d) { q[d] = qr[d]; acc[d] = 0.f; }
        float m = -INFINITY, l = 0.f;
        for (int j = 0; j <= r; ++j) {
            const float* kr = a.k + (int64_t)(s0 + j) * ks + (int64_t)g * D;
            const float* vr = a.v + (int64_t)(s0 + j) * ks + (int64_t)g * D;
            float dot = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) dot = __builtin_fmaf(q[d], kr[d], dot);
            const float x = dot * a.scale_log2;
            if (x > m) {
                const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - x);
                l *= alpha;
#pragma unroll
                for (int d = 0; d < D; ++d) acc[d] *= alpha;
                m = x;
            }
            const float p = __builtin_amdgcn_exp2f(x - m);
            l += p;
#pragma unroll
            for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(p, vr[d], acc[d]);
        }
        const float inv = 1.f / l;
        float* orow = a.out + (int64_t)(s0 + r) * qs + (int64_t)head * D;
#pragma unroll
        for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv;
        a.lse[(int64_t)(s0 + r) * a.H + head] = (m + __builtin_amdgcn_logf(l)) * kLn2;
    }
}

}  // namespace

hipError_t launch_fwd_f32(const F32Args& a, hipStream_t s) {
    dim3 grid(a.n_seq, a.H);
    if (a.D == 128) hipLaunchKernelGGL((fwd_f32_kernel<128>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((fwd_f32_kernel<64>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace hdp
