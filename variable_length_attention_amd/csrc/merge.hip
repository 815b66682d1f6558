// Log-sum-exp merge of two ring-step partials, in place (research digest "ByteScale:
// Communication-Efficient Scaling of LLM Training with a 2048K Context Length on 16384 GPUs",
// §3.2: each ring step computes on one K/V slice and the steps' results are combined).
//
// Bound by HBM: per (token, head) row it reads o_acc, o_part (4D bytes each) and two lse
// values and writes o_acc and lse (plus 2D bytes when the bf16 copy is requested).  Each lane
// moves 16 bytes per tensor (float4), D/4 consecutive lanes cover one row, so every wavefront
// touches whole contiguous rows.
#include "hdp_internal.h"

namespace hdp {
namespace {

constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
    constexpr int kTpr = D / 4;                    // lanes per row
    constexpr int kRowsPerBlock = kThreads / kTpr;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kTpr;
    const int c = threadIdx.x % kTpr;
    if (row >= a.rows) return;
    const float l1 = a.lse_acc[row];
    const float l2 = a.lse_part[row];
    float4* op = (float4*)a.o_acc + row * kTpr + c;
    const float4 o1 = *op;
    const float4 o2 = ((const float4*)a.o_part)[row * kTpr + c];
    float4 r;
    float lr;
    if (l2 == -INFINITY) {
        r = o1;
        lr = l1;
    } else if (l1 == -INFINITY) {
        r = o2;
        lr = l2;
    } else {
        const float m = fmaxf(l1, l2);
        const float w1 = __expf(l1 - m), w2 = __expf(l2 - m);
        const float inv = 1.f / (w1 + w2);
        const float a1 = w1 * inv, a2 = w2 * inv;
        r = make_float4(a1 * o1.x + a2 * o2.x, a1 * o1.y + a2 * o2.y, a1 * o1.z + a2 * o2.z,
                        a1 * o1.w + a2 * o2.w);
        lr = m + __logf(w1 + w2);
    }
    *op = r;
    if (c == 0) a.lse_acc[row] = lr;
    if (a.out_bf16 != nullptr) {
        __bf16 b0 = (__bf16)r.x, b1 = (__bf16)r.y, b2 = (__bf16)r.z, b3 = (__bf16)r.w;
        uint2 w;
        w.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        w.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        *((uint2*)a.out_bf16 + row * kTpr + c) = w;
    }
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(int* p, int n) {
    for (int i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads) p[i] = 0;
}

}  // namespace

hipError_t launch_fill_zero(int* p, int n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int blocks = (n + kThreads - 1) / kThreads < 64 ? (n + kThreads - 1) / kThreads : 64;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(kThreads), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t s) {
    const int tpr = a.D / 4;
    const int rows_per_block = kThreads / tpr;
    const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    if (a.D == 128) hipLaunchKernelGGL((merge_kernel<128>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<64>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace hdp
