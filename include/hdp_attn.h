/*
 * hdp_attn.h -- C ABI of the per-rank attention library for Hybrid Data Parallelism on
 * MI355X (gfx950).  Library: variable_length_attention_amd/libhdpattn.so.
 *
 * What is computed.  Under Hybrid Data Parallelism every rank holds a slice of at most C
 * tokens.  Sequences no longer than C sit whole on one rank, packed back to back, and send
 * nothing; a longer sequence spans ceil(s/C) ranks that pass key/value slices around their own
 * ring (research digest "ByteScale: Communication-Efficient Scaling of LLM Training with a
 * 2048K Context Length on 16384 GPUs", §3.1 and Figure 2).  A query attends only to its own
 * sequence, and a ring step computes on the K/V slice in hand while the next one arrives
 * (same digest, §3.2).  The mask is causal (same digest, §4).  Attention work grows with the
 * square of each sequence's length (same digest, §2), which is what hdp_seq_flops counts.
 *
 * The pages print no formula; the library computes textbook scaled-dot-product attention:
 * for query row r and the keys j it may see,
 *     out_r = sum_j softmax_j(scale * <q_r, k_j>) v_j,   lse_r = ln sum_j exp(scale * <q_r, k_j>).
 * Query head h reads key/value head h / (H / Hkv) (contiguous groups).
 *
 * Conventions for every call.
 *   - Tensor pointers are DEVICE memory owned by the caller; the library keeps no reference
 *     after the call returns and frees nothing it did not allocate.
 *   - bf16 tensors are stored as uint16_t bit patterns; outputs are rounded to nearest even.
 *   - Layouts are token-major and dense: q/out/dq [T][H][D], k/v/dk/dv [T][Hkv][D],
 *     lse [T][H] fp32.  Within one token all heads are contiguous.
 *   - Every call is asynchronous on `stream` (0 = the null stream) and never synchronises the
 *     host.  Device faults surface at the caller's next synchronisation.
 *   - Arguments are checked on the host before any HIP call.  Errors return a status and
 *     launch nothing.  n_seq == 0 or Lq == 0 is a no-op returning HDP_OK.
 *   - cu_seqlens is device memory (int32, n_seq + 1 entries, cu[0] = 0, non-decreasing,
 *     T = cu[n_seq]).  Its contents are not checked on the host; the kernels clamp every
 *     sequence to [0, cu[n_seq]], so malformed entries give empty sequences, never an access
 *     outside rows 0 .. cu[n_seq]-1.  Rows outside [cu[0], cu[n_seq]) are left untouched.
 *   - Supported head dims: D = 64 and D = 128 (else HDP_ERR_UNSUPPORTED); head counts
 *     H <= 65535 (else HDP_ERR_OVERFLOW).
 *   - The library owns a small state per (device, stream): work-queue counters and, for the
 *     backward, every row's lse and delta as fp32 (2 x rows x H), grown on demand.  It is
 *     allocated stream-ordered (hipMallocAsync / hipFreeAsync on the call's stream, no
 *     device-wide synchronisation), so calls on different streams never share it and may run
 *     concurrently; calls on one stream are ordered by the stream.  The state is keyed by the
 *     stream handle: destroy a stream only after its calls have completed.
 *     hdp_release_workspace() frees the current device's state (it synchronises the device).
 *     For tests of the error path, a set environment variable HDP_TEST_FAIL_ALLOC makes every
 *     growth of the backward workspace fail (HDP_ERR_HIP, nothing launched).
 *   - With the environment variable HDP_VALIDATE set, the calls that take cu_seqlens copy it to
 *     the host first (synchronising the stream) and return HDP_ERR_INVALID_ARG unless cu[0] = 0,
 *     the entries do not decrease and (backward) cu[n_seq] <= T.  A debugging aid, off by
 *     default: the hot path never waits on the host.
 */
#ifndef HDP_ATTN_H
#define HDP_ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HDP_OK = 0,
    HDP_ERR_INVALID_ARG = 1, /* null pointer with work to do, bad sizes, H % Hkv != 0, ... */
    HDP_ERR_UNSUPPORTED = 2, /* head dim other than 64 / 128 */
    HDP_ERR_HIP = 3,         /* a HIP launch or allocation failed */
    HDP_ERR_OVERFLOW = 4,    /* a size product does not fit the index types */
    HDP_ERR_SCRATCH_LIMIT = 5 /* larger than the fixed scratch of hdp_attn_varlen_bwd_noalloc */
} hdp_status_t;

enum { HDP_PASS_FWD = 0, HDP_PASS_BWD = 1, HDP_PASS_FWD_BWD = 2 };

/*
 * Packed variable-length causal attention, forward, bf16 in / bf16 out, fp32 accumulation.
 * Sequence i owns packed rows cu[i] .. cu[i+1]-1; row r of it sees rows cu[i] .. cu[i]+r of
 * the same sequence and nothing else (digest §3.1-§3.2: a query attends only to its own
 * sequence; packed short sequences need no partner).
 *   q [T][H][D], k, v [T][Hkv][D] bf16; out [T][H][D] bf16 (written); lse [T][H] fp32, natural
 *   log of the row's sum of exp(scale * score) (written).  scale must be finite.
 * Work is split into (sequence, head group, query tile) items whose cost is the number of key
 * tiles they visit (the tile form of hdp_seq_flops); the kernel pops them longest first.
 */
int hdp_attn_varlen_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                        int32_t n_seq, int32_t H, int32_t Hkv, int32_t D, float scale,
                        void* out, float* lse, hipStream_t stream);

/* Same as hdp_attn_varlen_fwd with fp32 q, k, v and fp32 out (fp32 arithmetic throughout). */
int hdp_attn_varlen_fwd_f32(const float* q, const float* k, const float* v,
                            const int32_t* cu_seqlens, int32_t n_seq, int32_t H, int32_t Hkv,
                            int32_t D, float scale, float* out, float* lse, hipStream_t stream);

/*
 * One ring step (digest §3.2): a slice of Lq query tokens of one long sequence, at global
 * positions q_offset + r, against one key/value chunk of Lk tokens at global positions
 * kv_offset + j.  With causal != 0, key j is visible to row r iff kv_offset + j <= q_offset + r;
 * with causal == 0 every key is visible.
 *   q_slice [Lq][H][D], k_chunk, v_chunk [Lk][Hkv][D] bf16.
 *   o_partial [Lq][H][D] fp32 (written): the softmax average over this chunk's visible keys.
 *   lse [Lq][H] fp32 (written).  A row with no visible key gets o = 0 and lse = -inf.
 * Combine the steps with hdp_lse_merge.  Offsets must be >= 0.
 */
int hdp_attn_chunk_partial(const void* q_slice, int32_t Lq, const void* k_chunk,
                           const void* v_chunk, int32_t Lk, int64_t q_offset, int64_t kv_offset,
                           int32_t causal, int32_t H, int32_t Hkv, int32_t D, float scale,
                           float* o_partial, float* lse, hipStream_t stream);

/*
 * One ring step with its merge fused (digest §3.2: each step computes on the chunk in hand and
 * the steps' results are combined): the same attention of the slice against the chunk as
 * hdp_attn_chunk_partial, merged by log-sum-exp into the running result in place, as
 * hdp_lse_merge would do with that partial, without writing the partial out:
 *   o_acc [Lq][H][D], lse_acc [Lq][H] fp32: read and overwritten.  A row whose lse_acc is -inf
 *   has seen no key yet: its o_acc is ignored (it may hold anything).  A row that sees no key of
 *   this chunk keeps its values (and keeps o_acc = 0 if it has seen none at all).
 *   out_bf16: NULL, or [Lq][H][D] bf16 that receives the merged o_acc rounded to bf16.
 * Start a ring with lse_acc = -inf (any o_acc) or with the first step's hdp_attn_chunk_partial.
 * HBM traffic of the merge: 1,032 bytes per (row, head) at D = 128 against 2,064 for a partial
 * written out and merged by hdp_lse_merge.  Other arguments as hdp_attn_chunk_partial.
 */
int hdp_attn_chunk_merge(const void* q_slice, int32_t Lq, const void* k_chunk, const void* v_chunk,
                         int32_t Lk, int64_t q_offset, int64_t kv_offset, int32_t causal, int32_t H,
                         int32_t Hkv, int32_t D, float scale, float* o_acc, float* lse_acc,
                         void* out_bf16, hipStream_t stream);

/*
 * Log-sum-exp merge of two partials over disjoint key sets, in place (the ring's per-step
 * combination, digest §3.2).  For each of the L*H (token, head) rows:
 *     m = max(l_acc, l_part); w = exp(l - m); o_acc = (w_acc o_acc + w_part o_part)/(w_acc + w_part);
 *     l_acc = m + ln(w_acc + w_part).
 * A partial with lse = -inf is the identity (two empty partials stay 0 / -inf, never NaN).
 *   o_acc [L][H][D], lse_acc [L][H] fp32: read and overwritten.
 *   o_part [L][H][D], lse_part [L][H] fp32: read only.
 *   out_bf16: NULL, or [L][H][D] bf16 that receives the merged o_acc rounded to bf16.
 */
int hdp_lse_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                  int32_t L, int32_t H, int32_t D, void* out_bf16, hipStream_t stream);

/*
 * Backward of hdp_attn_varlen_fwd (the pages show forward and backward time per step but give
 * no formulas; this is the chain rule of the forward above).  With P = exp(scale*S - lse):
 *     dV = P^T dO,  dS = P * (dO V^T - rowsum(dO * out)),  dQ = scale dS K,  dK = scale dS^T Q,
 * dK and dV summed over the H/Hkv query heads of each key/value head.
 *   q, k, v, out, dout bf16 as in the forward; lse fp32 [T][H] from the forward.
 *   T: total packed tokens (the caller's row count, = cu[n_seq]).  Not in the forward's list:
 *   the backward needs it on the host, without reading cu_seqlens from the device, to size its
 *   fp32 workspace before the launch; the kernels also clamp every sequence to rows 0 .. T-1.
 *   dq [T][H][D], dk, dv [T][Hkv][D] bf16 (written).
 */
int hdp_attn_varlen_bwd(const void* q, const void* k, const void* v, const void* out,
                        const float* lse, const void* dout, const int32_t* cu_seqlens,
                        int32_t n_seq, int32_t T, int32_t H, int32_t Hkv, int32_t D,
                        float scale, void* dq, void* dk, void* dv, hipStream_t stream);

/*
 * hdp_attn_varlen_bwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving or training loops, harnesses that forbid allocation.  Same arguments,
 * kernels and results (bit for bit) as hdp_attn_varlen_bwd, but the library allocates nothing:
 * its scratch (work-queue counters and 2 x T x H fp32 row values) lives in one fixed device array
 * of HDP_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends.  Sizes need
 * 4096 + 8 * T * H <= HDP_NOALLOC_SCRATCH_BYTES (T * H <= 2,096,640, e.g. T <= 65,520 at H = 32),
 * else HDP_ERR_SCRATCH_LIMIT and nothing is launched.  The counters are cleared by a kernel at
 * the start of every call.  Every call on one GPU shares that GPU's array: calls that overlap in
 * time on one GPU (two streams, two host threads) race and give wrong results; serialise them.
 * HDP_VALIDATE is not honoured here (it would copy to the host).
 */
#define HDP_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u)
int hdp_attn_varlen_bwd_noalloc(const void* q, const void* k, const void* v, const void* out,
                                const float* lse, const void* dout, const int32_t* cu_seqlens,
                                int32_t n_seq, int32_t T, int32_t H, int32_t Hkv, int32_t D,
                                float scale, void* dq, void* dk, void* dv, hipStream_t stream);

/*
 * Backward of one ring step (the counterpart of hdp_attn_chunk_partial): the slice's rows
 * against one key/value chunk, at the same global offsets and with the same visibility.  With
 * the slice's final output and lse (over all of its keys, e.g. the merged ring result) it adds
 * this chunk's share of the gradients:
 *     dq_acc += scale dS K,   dk_acc += scale dS^T Q,   dv_acc += P^T dO,
 * P = exp(scale*S - lse) and dS = P * (dO V^T - rowsum(dO * out)) on the visible pairs, dK and
 * dV summed over the H/Hkv query heads of each key/value head.  Summed over a ring's chunks
 * (dq) and slices (dk, dv) this is the backward of the whole sequence (digest §3.2 ring steps).
 *   q_slice, out, dout bf16 [Lq][H][D]; lse fp32 [Lq][H]; k_chunk, v_chunk bf16 [Lk][Hkv][D].
 *   dq_acc fp32 [Lq][H][D]; dk_acc, dv_acc fp32 [Lk][Hkv][D]: read and updated in place
 *   (zero them before the first step).  Offsets must be >= 0.  Uses a [2][H][Lq] fp32
 *   workspace of the library.
 */
int hdp_attn_chunk_bwd(const void* q_slice, int32_t Lq, const void* k_chunk, const void* v_chunk,
                       int32_t Lk, int64_t q_offset, int64_t kv_offset, int32_t causal,
                       int32_t H, int32_t Hkv, int32_t D, float scale, const void* out,
                       const float* lse, const void* dout, float* dq_acc, float* dk_acc,
                       float* dv_acc, hipStream_t stream);

/*
 * Exact attention FLOPs of one sequence of s tokens attending to itself: visible pairs
 * P = s(s+1)/2 (causal) or s^2, times H, times 4D (forward: score and value contractions),
 * 10D (backward: five contractions) or 14D (both).  The O(s^2) cost that drives data-aware
 * sharding and the balance scheduler (digest §2, §3.4).  Returns 0 for s <= 0, H <= 0 or
 * D <= 0, and UINT64_MAX on overflow or an unknown pass.
 */
uint64_t hdp_seq_flops(int64_t s, int32_t H, int32_t D, int32_t causal, int32_t pass);

/* FLOPs of one ring step (as hdp_attn_chunk_partial counts visible pairs), same units. */
uint64_t hdp_chunk_flops(int32_t Lq, int32_t Lk, int64_t q_offset, int64_t kv_offset,
                         int32_t causal, int32_t H, int32_t D, int32_t pass);

/*
 * Front/back chunk pairing of one sequence over a ring of n_ranks ranks (digest §4: each packed
 * subsequence is cut into 2N chunks handed out in front/back pairs, which balances the causal
 * mask).  Chunk c covers tokens [floor(c s / 2N), floor((c+1) s / 2N)); rank k holds chunks k
 * and 2N-1-k.  Writes their global offsets and lengths to offsets[0..1], lengths[0..1] (front
 * chunk first).  When 2N divides s every rank's causal pairs, summed over all chunks of the
 * ring, are equal.  Host only.  s >= 0, 0 <= rank < n_ranks.
 */
int hdp_pair_chunks(int64_t s, int32_t n_ranks, int32_t rank, int64_t* offsets, int64_t* lengths);

/*
 * HDP sharding of one global batch over a pool of ranks of capacity C tokens (digest §3.1 and
 * Figure 2), host only.  A sequence longer than C gets a ring of ceil(s/C) units (one unit per
 * rank: near-equal contiguous slices, or with pair != 0 the front/back chunk pairs of
 * hdp_pair_chunks); shorter sequences are packed by best fit (decreasing length) into units of
 * at most C tokens.  Units list the rings by decreasing length, then the packed units.
 *   lens [n_seq] (>= 0; zero-length sequences are dropped).  Outputs (caller-owned):
 *   unit_first_piece [n_units + 1] (pieces of unit j are unit_first_piece[j] ..
 *   unit_first_piece[j+1] - 1), unit_ring [n_units] (the sequence index of a ring unit, -1 for
 *   a packed unit), piece_seq / piece_off / piece_len [n_pieces] (sequence, first token within
 *   it, token count).  *n_units and *n_pieces always receive the sizes needed; if they exceed
 *   max_units or max_pieces nothing else is written and HDP_ERR_OVERFLOW is returned.
 */
int hdp_plan_shard(const int64_t* lens, int32_t n_seq, int64_t C, int32_t pair, int32_t max_units,
                   int32_t max_pieces, int32_t* n_units, int32_t* n_pieces, int32_t* unit_first_piece,
                   int32_t* unit_ring, int32_t* piece_seq, int64_t* piece_off, int64_t* piece_len);

/*
 * Attention FLOPs of every unit of a plan from hdp_plan_shard (pass as in hdp_seq_flops): a
 * packed unit costs the hdp_seq_flops of its sequences; a ring unit its query pieces against
 * every piece of its ring (hdp_chunk_flops, causal).  cost [n_units] (written).  Host only.
 */
int hdp_plan_unit_flops(const int64_t* lens, int32_t n_seq, int32_t n_units,
                        const int32_t* unit_first_piece, const int32_t* unit_ring,
                        const int32_t* piece_seq, const int64_t* piece_off, const int64_t* piece_len,
                        int32_t H, int32_t D, int32_t pass, uint64_t* cost);

/*
 * Balance scheduler, DP-Balance (digest §3.4, Figure 4), host only: assigns units of equal
 * tokens but unequal cost to n_ranks ranks so that their summed costs meet; ranks may run
 * different numbers of units.  Items are packed units and whole rings (the consecutive units
 * of one ring run on distinct ranks), sorted by per-rank cost and cut into n_ranks buckets of
 * about equal FLOPs; every rank that trails the most loaded one by more than delta (all ranks
 * when none does) takes, least loaded first, the next item of the first non-empty bucket.
 *   cost, unit_ring [n_units] as from hdp_plan_unit_flops / hdp_plan_shard.  Outputs:
 *   unit_rank [n_units], rank_load [n_ranks].  A ring wider than the pool is invalid.
 */
int hdp_plan_balance(const uint64_t* cost, const int32_t* unit_ring, int32_t n_units,
                     int32_t n_ranks, uint64_t delta, int32_t* unit_rank, uint64_t* rank_load);

/*
 * Measurement helper, not part of the attention path: the shader clock (MHz) the current device
 * sustains while every CU issues back-to-back bf16 MFMAs for `iters` iterations (shader-clock
 * counter cycles over the constant 100 MHz real-time counter's elapsed time).  Roofline
 * fractions are quoted against the nominal 2.4 GHz and against this clock.  Allocates a few
 * bytes stream-ordered and synchronises `stream` to read the result into *mhz.
 */
int hdp_probe_clock(int32_t iters, double* mhz, hipStream_t stream);

/*
 * Measurement helper, not part of the attention path: per-workgroup trace of the forward
 * kernel (hdp_attn_varlen_fwd, hdp_attn_chunk_partial).  With trace != NULL (device memory of
 * 4 x capacity int64) every later forward launch whose persistent grid (one workgroup per CU)
 * fits the capacity writes, for workgroup w: trace[4w] = the real-time counter (100 MHz) when
 * it started, trace[4w+1] = when it finished its last item, trace[4w+2] = items it processed,
 * trace[4w+3] = 0.  The buffer is overwritten by each such launch.  capacity 0 turns it off.
 * Backward launches (hdp_attn_varlen_bwd, hdp_attn_chunk_bwd) write, for workgroup w:
 * trace[4w] = when it started, trace[4w+1] = when it left the dK/dV work queue (it then takes
 * dQ items), trace[4w+2] = when it finished, trace[4w+3] = 0.
 * This is how the FLOP-ordered scheduling's balance across CUs is measured.
 */
int hdp_set_trace(long long* trace, int32_t capacity);

/*
 * Measurement helper, not part of the attention path: per-item timeline of the same forward
 * launches.  With items != NULL (device memory of 4 x slots x capacity int64, slots > 0) every
 * later forward launch whose persistent grid fits the capacity writes, for the i-th item
 * (i < slots) that workgroup w processes, at items[4 (w slots + i) + 0..3]: the real-time counter
 * (100 MHz) when the item started, when its first key/value stages and query rows had landed in
 * LDS, when its last step was done (the output stores and the next item's pop follow), and the
 * number of 32-key units it ran.  Records past the items a workgroup processed are left as they
 * were.  capacity 0 turns it off; HDP_ERR_INVALID_ARG for a negative capacity or slots, or for
 * capacity > 0 with a NULL buffer or slots = 0.  With hdp_set_trace this splits each workgroup's
 * time into waiting for first loads, steps and item transitions.
 */
int hdp_set_item_trace(long long* items, int32_t capacity, int32_t slots);

/* Static text for a status code. */
const char* hdp_status_string(int status);

/* Frees the calling thread's current device's workspace (synchronises that device). */
int hdp_release_workspace(void);

#ifdef __cplusplus
}
#endif

#endif /* HDP_ATTN_H */
