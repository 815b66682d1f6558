// Host-side planning of a rank's work (no device code): front/back chunk pairing of a long
// sequence over a ring, HDP sharding of a global batch over a pool of ranks, and the balance
// scheduler.  Research digest "ByteScale: Communication-Efficient Scaling of LLM Training with
// a 2048K Context Length on 16384 GPUs": §3.1 and Figure 2 (HDP pool, ceil(s/C) ranks per long
// sequence, best-fit packing of the short ones), §3.4 and Figure 4 (balance scheduler), §4
// (2N chunks handed out in front/back pairs).
#include <algorithm>
#include <cstdint>
#include <numeric>
#include <vector>

#include "hdp_attn.h"

extern "C" {

int hdp_pair_chunks(int64_t s, int32_t n_ranks, int32_t rank, int64_t* offsets, int64_t* lengths) {
    if (s < 0 || n_ranks <= 0 || rank < 0 || rank >= n_ranks || !offsets || !lengths)
        return HDP_ERR_INVALID_ARG;
    if (s > (INT64_MAX >> 21)) return HDP_ERR_OVERFLOW;    // c * s below fits in int64
    const int64_t n2 = 2 * (int64_t)n_ranks;
    auto bound = [&](int64_t c) { return c * s / n2; };    // chunk c = [bound(c), bound(c+1))
    const int64_t c[2] = {rank, n2 - 1 - rank};
    for (int i = 0; i < 2; ++i) {
        offsets[i] = bound(c[i]);
        lengths[i] = bound(c[i] + 1) - offsets[i];
    }
    return HDP_OK;
}

}  // extern "C"
