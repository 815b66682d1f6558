/*
 * hdp_oracle.c -- plain, slow, fp64 CPU oracle for per-rank variable-length causal attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this file:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It shares no
 * source, header, table or helper with the HIP library, and it includes nothing from it.
 *
 * Sources.  "Digest" below is the research-digest page titled "ByteScale: Communication-Efficient
 * Scaling of LLM Training with a 2048K Context Length on 16384 GPUs" (SIGCOMM'25 primer).
 *   - Each rank holds a slice of at most C tokens; shorter sequences are packed onto one rank
 *     and send nothing (Digest §1, §3.1 and Figure 2).
 *   - A query attends only to its own sequence; a long sequence's slices pass K/V around a ring
 *     and combine per-step partial results (Digest §3.2, ring model).
 *   - The causal mask (Digest §4, front/back chunk pairing "balances the causal mask").
 *   - Attention time O(s^2), memory O(s) in the FlashAttention style (Digest §1, §2).
 * The pages never print the attention formula; this oracle writes out the textbook definition
 * of scaled-dot-product attention with a block-diagonal causal mask, row by row:
 *     x_j   = scale * <q_r, k_j>               for the visible keys j of row r
 *     m     = max_j x_j
 *     l     = sum_j exp(x_j - m)
 *     out_r = sum_j exp(x_j - m) v_j / l
 *     lse_r = m + ln l                          (natural log, unshifted)
 * Grouped heads: query head h reads key/value head floor(h / (H / Hkv)).
 * A row with no visible key has out = 0 and lse = -inf.
 *
 * All arithmetic is fp64; every sum runs in ascending index order, so results do not depend on
 * the thread count.  Layouts: q/out [T][H][D], k/v [T][Hkv][D], lse [T][H], row-major;
 * cu_seqlens has n_seq + 1 entries, cu[0] = 0, non-decreasing.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_BAD_ARG 1
#define ORC_NO_MEM 2

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Index of the sequence that owns packed token t (cu[i] <= t < cu[i+1]); -1 if none. */
static int64_t owner_seq(const int32_t* cu, int64_t n_seq, int64_t t) {
    for (int64_t i = 0; i < n_seq; ++i)
        if (t >= cu[i] && t < cu[i + 1]) return i;
    return -1;
}

static int check_cu(const int32_t* cu, int64_t n_seq) {
    if (n_seq < 0) return ORC_BAD_ARG;
    if (n_seq > 0 && cu[0] != 0) return ORC_BAD_ARG;
    for (int64_t i = 0; i < n_seq; ++i)
        if (cu[i + 1] < cu[i]) return ORC_BAD_ARG;
    return ORC_OK;
}

/*
 * Softmax-weighted average of the value rows v[key0 + j] over the visible keys j of one query
 * row, for one head.  visible[j] != 0 marks key j.  Writes D outputs and returns the lse.
 * x is caller scratch of n_keys doubles.
 */
static double attend_row(const double* qrow, const double* kbase, const double* vbase,
                         int64_t kv_stride, int64_t n_keys, const unsigned char* visible,
                         int D, double scale, double* x, double* orow) {
    double m = -INFINITY;
    int any = 0;
    for (int64_t j = 0; j < n_keys; ++j) {
        if (!visible[j]) continue;
        const double* krow = kbase + j * kv_stride;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qrow[d] * krow[d];
        x[j] = scale * dot;
        if (!any || x[j] > m) m = x[j];
        any = 1;
    }
    for (int d = 0; d < D; ++d) orow[d] = 0.0;
    if (!any) return -INFINITY;
    double l = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        if (!visible[j]) continue;
        double p = exp(x[j] - m);
        l += p;
        const double* vrow = vbase + j * kv_stride;
        for (int d = 0; d < D; ++d) orow[d] += p * vrow[d];
    }
    for (int d = 0; d < D; ++d) orow[d] /= l;
    return m + log(l);
}

/*
 * Packed variable-length causal attention, forward.  Row r of sequence i (tokens
 * cu[i] .. cu[i+1]-1) sees keys 0..r of the same sequence and nothing else.
 * rows: the packed token indices to evaluate (NULL = all T = cu[n_seq] tokens);
 * out [n_rows][H][D], lse [n_rows][H] follow the order of rows.
 */
int orc_varlen_fwd(const double* q, const double* k, const double* v, const int32_t* cu,
                   int64_t n_seq, int H, int Hkv, int D, double scale, const int64_t* rows,
                   int64_t n_rows, double* out, double* lse, int nthreads) {
    if (H <= 0 || Hkv <= 0 || D <= 0 || H % Hkv != 0) return ORC_BAD_ARG;
    if (check_cu(cu, n_seq) != ORC_OK) return ORC_BAD_ARG;
    const int64_t T = n_seq > 0 ? cu[n_seq] : 0;
    if (rows == NULL) n_rows = T;
    int64_t max_len = 0;
    for (int64_t i = 0; i < n_seq; ++i)
        if (cu[i + 1] - cu[i] > max_len) max_len = cu[i + 1] - cu[i];
    const int G = H / Hkv;
    int status = ORC_OK;
    set_threads(nthreads);
#pragma omp parallel
    {
        double* x = (double*)malloc(sizeof(double) * (size_t)(max_len + 1));
        unsigned char* vis = (unsigned char*)malloc((size_t)(max_len + 1));
        if (x == NULL || vis == NULL) {
#pragma omp atomic write
            status = ORC_NO_MEM;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t n = 0; n < n_rows; ++n) {
                const int64_t t = rows ? rows[n] : n;
                const int64_t s = owner_seq(cu, n_seq, t);
                if (s < 0) {
                    for (int h = 0; h < H; ++h) {
                        lse[n * H + h] = NAN;
                        for (int d = 0; d < D; ++d) out[(n * H + h) * D + d] = NAN;
                    }
                    continue;
                }
                const int64_t a = cu[s];
                const int64_t r = t - a;
                for (int64_t j = 0; j <= r; ++j) vis[j] = 1; /* causal: keys 0..r of its own sequence */
                for (int h = 0; h < H; ++h) {
                    const int g = h / G;
                    lse[n * H + h] = attend_row(q + (t * H + h) * (int64_t)D,
                                                k + (a * Hkv + g) * (int64_t)D,
                                                v + (a * Hkv + g) * (int64_t)D,
                                                (int64_t)Hkv * D, r + 1, vis, D, scale, x,
                                                out + (n * H + h) * (int64_t)D);
                }
            }
        }
        free(x);
        free(vis);
    }
    return status;
}

/*
 * One ring step's partial: the query slice (Lq tokens at global positions q_offset + r) against
 * one key/value chunk (Lk tokens at global positions kv_offset + j).  With causal != 0, key j is
 * visible to row r iff kv_offset + j <= q_offset + r; otherwise every key is visible.  Output is
 * the normalised partial average and its lse; a row with no visible key gets 0 and -inf.
 * rows: the slice rows to evaluate (NULL = all Lq); outputs follow the order of rows.
 */
int orc_chunk_partial(const double* q, int64_t Lq, const double* k, const double* v, int64_t Lk,
                      int64_t q_offset, int64_t kv_offset, int causal, int H, int Hkv, int D,
                      double scale, const int64_t* rows, int64_t n_rows, double* o, double* lse,
                      int nthreads) {
    if (H <= 0 || Hkv <= 0 || D <= 0 || H % Hkv != 0 || Lq < 0 || Lk < 0) return ORC_BAD_ARG;
    if (rows == NULL) n_rows = Lq;
    const int G = H / Hkv;
    int status = ORC_OK;
    set_threads(nthreads);
#pragma omp parallel
    {
        double* x = (double*)malloc(sizeof(double) * (size_t)(Lk + 1));
        unsigned char* vis = (unsigned char*)malloc((size_t)(Lk + 1));
        if (x == NULL || vis == NULL) {
#pragma omp atomic write
            status = ORC_NO_MEM;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t n = 0; n < n_rows; ++n) {
                const int64_t r = rows ? rows[n] : n;
                for (int64_t j = 0; j < Lk; ++j)
                    vis[j] = (unsigned char)(!causal || kv_offset + j <= q_offset + r);
                for (int h = 0; h < H; ++h) {
                    const int g = h / G;
                    lse[n * H + h] = attend_row(q + (r * H + h) * (int64_t)D, k + (int64_t)g * D,
                                                v + (int64_t)g * D, (int64_t)Hkv * D, Lk, vis, D,
                                                scale, x, o + (n * H + h) * (int64_t)D);
                }
            }
        }
        free(x);
        free(vis);
    }
    return status;
}

/*
 * One ring step of the backward (the backward counterpart of orc_chunk_partial): the slice's
 * rows (Lq tokens at global positions q_offset + r) against one key/value chunk (Lk tokens at
 * kv_offset + j), given the slice's final output `out` and lse over the whole key range, and
 * dO.  Same visibility as orc_chunk_partial.  With P_rj = exp(scale <q_r, k_j> - lse_r) and
 * delta_r = sum_d dO_r[d] out_r[d] (the chain rule of the definition above, summed over this
 * chunk's keys only):
 *     dq_r = scale sum_j P_rj (<dO_r, v_j> - delta_r) k_j          this chunk's share of dQ
 *     dk_j = scale sum_{h in group} sum_r P_rj (<dO_r, v_j> - delta_r) q_r
 *     dv_j = sum_{h in group} sum_r P_rj dO_r
 * Summed over the chunks of a ring (and over the slices, for dk/dv) they give the full
 * backward.  qrows / krows select the slice rows of dq and the chunk rows of dk, dv to evaluate
 * (NULL = all); dq [n_q][H][D], dk and dv [n_k][Hkv][D] follow the order of the lists and are
 * overwritten.
 */
int orc_chunk_bwd(const double* q, int64_t Lq, const double* k, const double* v, int64_t Lk,
                  int64_t q_offset, int64_t kv_offset, int causal, int H, int Hkv, int D,
                  double scale, const double* out, const double* lse, const double* dout,
                  const int64_t* qrows, int64_t n_q, const int64_t* krows, int64_t n_k,
                  double* dq, double* dk, double* dv, int nthreads) {
    if (H <= 0 || Hkv <= 0 || D <= 0 || H % Hkv != 0 || Lq < 0 || Lk < 0) return ORC_BAD_ARG;
    const int G = H / Hkv;
    double* delta = (double*)malloc(sizeof(double) * (size_t)(Lq * H + 1));
    if (delta == NULL) return ORC_NO_MEM;
    set_threads(nthreads);
    for (int64_t r = 0; r < Lq; ++r)
        for (int h = 0; h < H; ++h) {
            double dl = 0.0;
            for (int d = 0; d < D; ++d)
                dl += dout[(r * H + h) * (int64_t)D + d] * out[(r * H + h) * (int64_t)D + d];
            delta[r * H + h] = dl;
        }

    if (qrows == NULL) n_q = Lq;
    if (krows == NULL) n_k = Lk;

    /* dQ rows of the slice */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t n = 0; n < n_q; ++n) {
        const int64_t r = qrows ? qrows[n] : n;
        for (int h = 0; h < H; ++h) {
            const int g = h / G;
            double* dqr = dq + (n * H + h) * (int64_t)D;
            for (int d = 0; d < D; ++d) dqr[d] = 0.0;
            const double* qr = q + (r * H + h) * (int64_t)D;
            const double* dor = dout + (r * H + h) * (int64_t)D;
            for (int64_t j = 0; j < Lk; ++j) {
                if (causal && kv_offset + j > q_offset + r) continue;
                const double* kj = k + (j * Hkv + g) * (int64_t)D;
                const double* vj = v + (j * Hkv + g) * (int64_t)D;
                double dot = 0.0, dp = 0.0;
                for (int d = 0; d < D; ++d) { dot += qr[d] * kj[d]; dp += dor[d] * vj[d]; }
                const double p = exp(scale * dot - lse[r * H + h]);
                const double ds = p * (dp - delta[r * H + h]);
                for (int d = 0; d < D; ++d) dqr[d] += scale * ds * kj[d];
            }
        }
    }

    /* dK and dV rows of the chunk */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t n = 0; n < n_k; ++n) {
        const int64_t j = krows ? krows[n] : n;
        for (int g = 0; g < Hkv; ++g) {
            double* dkj = dk + (n * Hkv + g) * (int64_t)D;
            double* dvj = dv + (n * Hkv + g) * (int64_t)D;
            for (int d = 0; d < D; ++d) { dkj[d] = 0.0; dvj[d] = 0.0; }
            const double* kj = k + (j * Hkv + g) * (int64_t)D;
            const double* vj = v + (j * Hkv + g) * (int64_t)D;
            for (int hh = 0; hh < G; ++hh) {
                const int h = g * G + hh;
                for (int64_t r = 0; r < Lq; ++r) {
                    if (causal && kv_offset + j > q_offset + r) continue;
                    const double* qr = q + (r * H + h) * (int64_t)D;
                    const double* dor = dout + (r * H + h) * (int64_t)D;
                    double dot = 0.0, dp = 0.0;
                    for (int d = 0; d < D; ++d) { dot += qr[d] * kj[d]; dp += dor[d] * vj[d]; }
                    const double p = exp(scale * dot - lse[r * H + h]);
                    const double ds = p * (dp - delta[r * H + h]);
                    for (int d = 0; d < D; ++d) {
                        dkj[d] += scale * ds * qr[d];
                        dvj[d] += p * dor[d];
                    }
                }
            }
        }
    }
    free(delta);
    return ORC_OK;
}

/*
 * Log-sum-exp merge of two normalised partials over disjoint key sets (the ring's per-step
 * combination, Digest §3.2).  In place on (o_acc, lse_acc), n rows of H heads:
 *     m = max(l1, l2), w_k = exp(l_k - m), o = (w1 o1 + w2 o2) / (w1 + w2), l = m + ln(w1 + w2).
 * A partial with lse = -inf has no keys and is the identity.
 */
int orc_lse_merge(double* o_acc, double* lse_acc, const double* o_part, const double* lse_part,
                  int64_t n, int H, int D) {
    if (n < 0 || H <= 0 || D <= 0) return ORC_BAD_ARG;
    for (int64_t i = 0; i < n * H; ++i) {
        const double l1 = lse_acc[i], l2 = lse_part[i];
        double* o1 = o_acc + i * D;
        const double* o2 = o_part + i * D;
        if (l2 == -INFINITY) continue;
        if (l1 == -INFINITY) {
            for (int d = 0; d < D; ++d) o1[d] = o2[d];
            lse_acc[i] = l2;
            continue;
        }
        const double m = l1 > l2 ? l1 : l2;
        const double w1 = exp(l1 - m), w2 = exp(l2 - m);
        for (int d = 0; d < D; ++d) o1[d] = (w1 * o1[d] + w2 * o2[d]) / (w1 + w2);
        lse_acc[i] = m + log(w1 + w2);
    }
    return ORC_OK;
}

/*
 * Backward of packed variable-length causal attention, from the chain rule on the definition
 * above, with the oracle's own fp64 out and lse:
 *     P_rj  = exp(x_rj - lse_r)                    (x_rj = scale <q_r, k_j>)
 *     delta = sum_d dO_r[d] out_r[d]
 *     dS_rj = P_rj (<dO_r, v_j> - delta_r)
 *     dQ_r  = scale sum_j dS_rj k_j
 *     dK_j  = scale sum_{h in group} sum_r dS_rj q_r
 *     dV_j  = sum_{h in group} sum_r P_rj dO_r
 * qrows selects the dq rows to evaluate, krows the dk/dv rows (NULL = all).  dq is
 * [n_q][H][D]; dk, dv are [n_k][Hkv][D], in the order of the row lists.
 */
int orc_varlen_bwd(const double* q, const double* k, const double* v, const double* dout,
                   const int32_t* cu, int64_t n_seq, int H, int Hkv, int D, double scale,
                   const int64_t* qrows, int64_t n_q, const int64_t* krows, int64_t n_k,
                   double* dq, double* dk, double* dv, int nthreads) {
    if (H <= 0 || Hkv <= 0 || D <= 0 || H % Hkv != 0) return ORC_BAD_ARG;
    if (check_cu(cu, n_seq) != ORC_OK) return ORC_BAD_ARG;
    const int64_t T = n_seq > 0 ? cu[n_seq] : 0;
    if (qrows == NULL) n_q = T;
    if (krows == NULL) n_k = T;
    const int G = H / Hkv;
    int64_t max_len = 0;
    for (int64_t i = 0; i < n_seq; ++i)
        if (cu[i + 1] - cu[i] > max_len) max_len = cu[i + 1] - cu[i];

    /* Step 1: the rows whose lse and delta the requested outputs use: each dq row itself, and
     * for a dk/dv row t every row of its sequence from t to the end (the rows that see key t). */
    unsigned char* need = (unsigned char*)calloc((size_t)(T + 1), 1);
    double* lse = (double*)malloc(sizeof(double) * (size_t)(T * H + 1));
    double* delta = (double*)malloc(sizeof(double) * (size_t)(T * H + 1));
    if (!need || !lse || !delta) {
        free(need); free(lse); free(delta);
        return ORC_NO_MEM;
    }
    for (int64_t n = 0; n < n_q; ++n) {
        const int64_t t = qrows ? qrows[n] : n;
        if (owner_seq(cu, n_seq, t) >= 0) need[t] = 1;
    }
    for (int64_t n = 0; n < n_k; ++n) {
        const int64_t t = krows ? krows[n] : n;
        const int64_t s = owner_seq(cu, n_seq, t);
        if (s >= 0)
            for (int64_t u = t; u < cu[s + 1]; ++u) need[u] = 1;
    }
    int status = ORC_OK;
    set_threads(nthreads);

    /* Step 2: lse_r and delta_r for every row of every needed sequence. */
#pragma omp parallel
    {
        double* x = (double*)malloc(sizeof(double) * (size_t)(max_len + 1));
        unsigned char* vis = (unsigned char*)malloc((size_t)(max_len + 1));
        double* orow = (double*)malloc(sizeof(double) * (size_t)D);
        if (!x || !vis || !orow) {
#pragma omp atomic write
            status = ORC_NO_MEM;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t t = 0; t < T; ++t) {
                if (!need[t]) continue;
                const int64_t s = owner_seq(cu, n_seq, t);
                if (s < 0) continue;
                const int64_t a = cu[s], r = t - a;
                for (int64_t j = 0; j <= r; ++j) vis[j] = 1;
                for (int h = 0; h < H; ++h) {
                    const int g = h / G;
                    lse[t * H + h] = attend_row(q + (t * H + h) * (int64_t)D,
                                                k + (a * Hkv + g) * (int64_t)D,
                                                v + (a * Hkv + g) * (int64_t)D, (int64_t)Hkv * D,
                                                r + 1, vis, D, scale, x, orow);
                    double dl = 0.0;
                    for (int d = 0; d < D; ++d) dl += dout[(t * H + h) * (int64_t)D + d] * orow[d];
                    delta[t * H + h] = dl;
                }
            }
        }
        free(x);
        free(vis);
        free(orow);
    }
    if (status != ORC_OK) {
        free(need); free(lse); free(delta);
        return status;
    }

    /* Step 3: dQ rows. */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t n = 0; n < n_q; ++n) {
        const int64_t t = qrows ? qrows[n] : n;
        const int64_t s = owner_seq(cu, n_seq, t);
        for (int h = 0; h < H; ++h) {
            double* dqr = dq + (n * H + h) * (int64_t)D;
            for (int d = 0; d < D; ++d) dqr[d] = s < 0 ? NAN : 0.0;
            if (s < 0) continue;
            const int64_t a = cu[s], r = t - a;
            const int g = h / G;
            const double* qr = q + (t * H + h) * (int64_t)D;
            const double* dor = dout + (t * H + h) * (int64_t)D;
            for (int64_t j = 0; j <= r; ++j) {
                const double* kj = k + ((a + j) * Hkv + g) * (int64_t)D;
                const double* vj = v + ((a + j) * Hkv + g) * (int64_t)D;
                double dot = 0.0, dp = 0.0;
                for (int d = 0; d < D; ++d) { dot += qr[d] * kj[d]; dp += dor[d] * vj[d]; }
                const double p = exp(scale * dot - lse[t * H + h]);
                const double ds = p * (dp - delta[t * H + h]);
                for (int d = 0; d < D; ++d) dqr[d] += scale * ds * kj[d];
            }
        }
    }

    /* Step 4: dK and dV rows (sum over the query heads of the group and the rows r >= j). */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t n = 0; n < n_k; ++n) {
        const int64_t t = krows ? krows[n] : n;
        const int64_t s = owner_seq(cu, n_seq, t);
        for (int g = 0; g < Hkv; ++g) {
            double* dkj = dk + (n * Hkv + g) * (int64_t)D;
            double* dvj = dv + (n * Hkv + g) * (int64_t)D;
            for (int d = 0; d < D; ++d) { dkj[d] = s < 0 ? NAN : 0.0; dvj[d] = s < 0 ? NAN : 0.0; }
            if (s < 0) continue;
            const int64_t e = cu[s + 1];
            const double* kj = k + (t * Hkv + g) * (int64_t)D;
            const double* vj = v + (t * Hkv + g) * (int64_t)D;
            for (int hh = 0; hh < G; ++hh) {
                const int h = g * G + hh;
                for (int64_t u = t; u < e; ++u) { /* rows that see key t: t <= u < end */
                    const double* qu = q + (u * H + h) * (int64_t)D;
                    const double* du = dout + (u * H + h) * (int64_t)D;
                    double dot = 0.0, dp = 0.0;
                    for (int d = 0; d < D; ++d) { dot += qu[d] * kj[d]; dp += du[d] * vj[d]; }
                    const double p = exp(scale * dot - lse[u * H + h]);
                    const double ds = p * (dp - delta[u * H + h]);
                    for (int d = 0; d < D; ++d) {
                        dkj[d] += scale * ds * qu[d];
                        dvj[d] += p * du[d];
                    }
                }
            }
        }
    }
    free(need);
    free(lse);
    free(delta);
    return ORC_OK;
}

/*
 * Number of (query, key) pairs the mask leaves visible for one query slice against one key
 * chunk, by enumeration.  Attention work is O(s^2) in these pairs (Digest §2, "attention work
 * grows as the square of each sequence's length").
 */
uint64_t orc_count_pairs(int64_t Lq, int64_t Lk, int64_t q_offset, int64_t kv_offset, int causal) {
    uint64_t n = 0;
    for (int64_t r = 0; r < Lq; ++r)
        for (int64_t j = 0; j < Lk; ++j)
            if (!causal || kv_offset + j <= q_offset + r) ++n;
    return n;
}

/*
 * FLOPs by definition: every visible pair costs, per head, one length-D dot product for the
 * score (2D: D multiplies and D adds) and one length-D multiply-add of the value row (2D) in the
 * forward; the backward's five pair-wise contractions (score recompute, dP, dV, dK, dQ) cost 2D
 * each.  pass: 0 = forward (4D), 1 = backward (10D), 2 = both (14D).
 */
uint64_t orc_attn_flops(int64_t Lq, int64_t Lk, int64_t q_offset, int64_t kv_offset, int causal,
                        int H, int D, int pass) {
    const uint64_t pairs = orc_count_pairs(Lq, Lk, q_offset, kv_offset, causal);
    uint64_t per = 0;
    if (pass == 0) per = 2ull * D + 2ull * D;
    else if (pass == 1) per = 5ull * 2ull * D;
    else if (pass == 2) per = 2ull * D + 2ull * D + 5ull * 2ull * D;
    return pairs * (uint64_t)H * per;
}
