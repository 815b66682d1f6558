// The packed backward for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving or training loops, harnesses that forbid allocation): the same kernels
// as hdp_attn_varlen_bwd, with their scratch memory (work-queue counters and the per-row lse /
// delta values) in one fixed device array of this library instead of a workspace it allocates.
#include <mutex>

#include "hdp_attn.h"
#include "hdp_internal.h"

namespace {

constexpr size_t kCounterBytes = 4096;                    // queue counters, cleared every call
constexpr size_t kScratchBytes = HDP_NOALLOC_SCRATCH_BYTES;
static_assert(sizeof(int) * hdp::kCounterInts <= kCounterBytes, "counter area");
static_assert(kScratchBytes > kCounterBytes, "scratch size");

// One copy per GPU, alive until the process ends.  In host code `scratch` names a host-side
// stand-in, not the device memory: the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};   // device address of `scratch`, per device
int g_cus[kMaxDevices] = {};

// Device address of this device's scratch and its CU count, looked up once per device (with
// that device current).  No allocation.
int scratch_of_current_device(unsigned char** ptr, int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HDP_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return HDP_ERR_HIP;
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return HDP_ERR_HIP;
        g_cus[dev] = n;
        g_ptr[dev] = p;
    }
    *ptr = (unsigned char*)g_ptr[dev];
    *cus = g_cus[dev];
    return HDP_OK;
}

}  // namespace

extern "C" int hdp_attn_varlen_bwd_noalloc(const void* q, const void* k, const void* v, const void* out,
                                           const float* lse, const void* dout, const int32_t* cu_seqlens,
                                           int32_t n_seq, int32_t T, int32_t H, int32_t Hkv, int32_t D,
                                           float scale, void* dq, void* dk, void* dv, hipStream_t stream) {
    if (int rc = hdp::check_varlen_bwd(q, k, v, out, lse, dout, cu_seqlens, n_seq, T, H, Hkv, D, scale, dq, dk, dv))
        return rc;
    if (n_seq == 0 || T == 0) return HDP_OK;
    if (kCounterBytes + 2 * sizeof(float) * (size_t)T * (size_t)H > kScratchBytes) return HDP_ERR_SCRATCH_LIMIT;
    unsigned char* base = nullptr;
    int cus = 0;
    if (int rc = scratch_of_current_device(&base, &cus)) return rc;
    int* counters = (int*)base;
    // the counters must start at zero: a fill kernel, not a memset node, so that the call can
    // be captured into a graph and replayed
    if (hdp::launch_fill_zero(counters, hdp::kCounterInts, stream) != hipSuccess) return HDP_ERR_HIP;
    return hdp::launch_varlen_bwd(q, k, v, out, lse, dout, cu_seqlens, n_seq, T, H, Hkv, D, scale, dq, dk, dv,
                                  counters, (float*)(base + kCounterBytes), cus, stream);
}
