/*
 * CPU oracle for zigzag varlen ring attention.  TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct: every value is computed from its definition
 * in double precision, one query row at a time.  Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load this library; the HIP
 * library never links, includes or calls it, and this file includes nothing
 * from the HIP side.
 *
 * What is computed, and where it comes from:
 *
 *  - Zigzag split.  ring-attention-pytorch issue #20 ("Zigzag attention
 *    support?"), the extract_local snippet: the sequence is cut into 2*W equal
 *    chunks and rank r keeps chunk r followed by chunk 2*W-1-r.  MaxText
 *    PR #1133 ("Add Context Parallelism support to cudnn Flash Attention"),
 *    review of the load-balanced flag, describes the same reordering.  For
 *    packed input the split is applied to every sequence on its own (the
 *    pages leave the packed case open) and ranks are stacked rank-major.
 *
 *  - Attention.  Causal softmax(Q K^T * scale) V with scale = 1/sqrt(head_dim)
 *    (MaxText PR #1133, the scale_factor argument of the cuDNN call), masked so
 *    that tokens of different packed sequences never see each other (EasyDeL
 *    issue #129, "Attention Mask for Packed Sequences (via Attention Bias)",
 *    opening request: -inf bias between examples).  Query head h reads key /
 *    value head h / (Hq/Hkv) (contiguous GQA groups; the pages do not fix it).
 *
 *  - Ring step.  FlagScale PR #910 ("[Train] Support custom attention with
 *    context parallel"), description: a ring driver calls a per-step forward
 *    and backward.  Step s pairs rank r's queries with shard (r - s) mod W; the
 *    step's result is the masked softmax restricted to that shard's keys,
 *    reported as a partial output and its log-sum-exp.  Rows with no visible
 *    key get output 0 and LSE = -inf.
 *
 *  - LSE merge.  Two partials over disjoint key sets combine into the softmax
 *    over their union: L = log(e^a + e^b), O = e^(a-L) O_a + e^(b-L) O_b.
 *
 *  - Backward.  The gradient of the same attention: P = exp(S - LSE),
 *    dP = dO V^T, D = rowsum(P * dP), dS = P (dP - D), dQ = scale dS K,
 *    dK = scale dS^T Q, dV = P^T dO, summed over the query heads of a group.
 *
 *  - Tile classification.  FlagScale PR #910 lists pruning of redundant work;
 *    here a tile is a BM x BN rectangle of (query, key) pairs whose grid starts
 *    at every zigzag chunk boundary, and it is classified by counting its
 *    visible pairs one by one.
 *
 * Precision: inputs are float (bf16 values are exact in float); all arithmetic
 * is double.  Build: gcc -O2 -fopenmp -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* Sequences and the zigzag permutation                                      */
/* ------------------------------------------------------------------------- */

static int64_t total_tokens(const int32_t *cu, int32_t nseq) { return cu[nseq]; }

/* Sequence that holds packed position p (cu is sorted). */
static int32_t seq_of(const int32_t *cu, int32_t nseq, int64_t p) {
    for (int32_t i = 0; i < nseq; ++i)
        if (p >= cu[i] && p < cu[i + 1]) return i;
    return -1;
}

/* Check that every sequence splits into 2*cp equal chunks. 0 = ok. */
int oracle_check_lengths(const int32_t *cu, int32_t nseq, int32_t cp) {
    if (nseq < 1 || cp < 1 || cu[0] != 0) return -1;
    for (int32_t i = 0; i < nseq; ++i) {
        int64_t L = (int64_t)cu[i + 1] - cu[i];
        if (L <= 0 || L % (2 * cp) != 0) return -1;
    }
    return 0;
}

/*
 * dst[p] = zigzag row of packed token p.  Built the way extract_local builds a
 * rank's shard: for every rank r, walk the sequences in order and append
 * chunk r and then chunk 2cp-1-r of each; ranks are laid out one after the
 * other.
 */
int oracle_zigzag_dst(const int32_t *cu, int32_t nseq, int32_t cp, int64_t *dst) {
    if (oracle_check_lengths(cu, nseq, cp)) return -1;
    int64_t row = 0;
    for (int32_t r = 0; r < cp; ++r) {
        for (int32_t i = 0; i < nseq; ++i) {
            int64_t L = (int64_t)cu[i + 1] - cu[i];
            int64_t c = L / (2 * cp);
            int32_t picks[2] = {r, 2 * cp - 1 - r};
            for (int u = 0; u < 2; ++u)
                for (int64_t o = 0; o < c; ++o) dst[cu[i] + picks[u] * c + o] = row++;
        }
    }
    return row == total_tokens(cu, nseq) ? 0 : -1;
}

/* For every zigzag row z: the packed token it holds. */
static int64_t *zigzag_src(const int32_t *cu, int32_t nseq, int32_t cp) {
    int64_t T = total_tokens(cu, nseq);
    int64_t *dst = (int64_t *)malloc(sizeof(int64_t) * T);
    int64_t *src = (int64_t *)malloc(sizeof(int64_t) * T);
    oracle_zigzag_dst(cu, nseq, cp, dst);
    for (int64_t p = 0; p < T; ++p) src[dst[p]] = p;
    free(dst);
    return src;
}

/* Is key (packed position pk) visible from query (packed position pq)? */
static int visible(const int32_t *cu, int32_t nseq, int64_t pq, int64_t pk) {
    return seq_of(cu, nseq, pq) == seq_of(cu, nseq, pk) && pk <= pq;
}

/* ------------------------------------------------------------------------- */
/* Masked softmax attention, one query row at a time                         */
/* ------------------------------------------------------------------------- */

static double dot(const float *a, const float *b, int32_t d) {
    double s = 0.0;
    for (int32_t e = 0; e < d; ++e) s += (double)a[e] * (double)b[e];
    return s;
}

/*
 * One query row against the keys listed in keys[0..nk): scores, max, sum,
 * output and LSE.  q_row and o_row have d entries; k and v are [*, hkv, d]
 * with kv head g.  Empty key list: o = 0, lse = -inf.  sbuf holds nk doubles.
 */
static void softmax_row(const float *q_row, const float *k, const float *v, int32_t hkv, int32_t g,
                        int32_t d, double scale, const int64_t *keys, int64_t nk, double *sbuf,
                        double *o_row, double *lse) {
    for (int32_t e = 0; e < d; ++e) o_row[e] = 0.0;
    if (nk == 0) { *lse = -INFINITY; return; }
    double m = -INFINITY;
    for (int64_t t = 0; t < nk; ++t) {
        sbuf[t] = scale * dot(q_row, k + ((size_t)keys[t] * hkv + g) * d, d);
        if (sbuf[t] > m) m = sbuf[t];
    }
    double l = 0.0;
    for (int64_t t = 0; t < nk; ++t) {
        double p = exp(sbuf[t] - m);
        l += p;
        const float *vr = v + ((size_t)keys[t] * hkv + g) * d;
        for (int32_t e = 0; e < d; ++e) o_row[e] += p * (double)vr[e];
    }
    for (int32_t e = 0; e < d; ++e) o_row[e] /= l;
    *lse = m + log(l);
}

static int64_t max_len(const int32_t *cu, int32_t nseq) {
    int64_t m = 0;
    for (int32_t i = 0; i < nseq; ++i)
        if (cu[i + 1] - cu[i] > m) m = cu[i + 1] - cu[i];
    return m;
}

/*
 * Full attention over packed sequences, packed layout.
 * q [T,hq,d], k/v [T,hkv,d]  ->  o [T,hq,d], lse [hq,T].
 */
void oracle_attn_fwd(const float *q, const float *k, const float *v, const int32_t *cu, int32_t nseq,
                     int32_t hq, int32_t hkv, int32_t d, double scale, double *o, double *lse) {
    int64_t T = total_tokens(cu, nseq);
    int32_t G = hq / hkv;
    int64_t Lmax = max_len(cu, nseq);
#pragma omp parallel
    {
        double *sbuf = (double *)malloc(sizeof(double) * Lmax);
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * Lmax);
#pragma omp for schedule(dynamic, 16) collapse(2)
        for (int32_t h = 0; h < hq; ++h)
            for (int64_t p = 0; p < T; ++p) {
                int32_t i = seq_of(cu, nseq, p);
                int64_t nk = 0;
                for (int64_t kp = cu[i]; kp <= p; ++kp) keys[nk++] = kp;
                softmax_row(q + ((size_t)p * hq + h) * d, k, v, hkv, h / G, d, scale, keys, nk, sbuf,
                            o + ((size_t)p * hq + h) * d, lse + (size_t)h * T + p);
            }
        free(sbuf);
        free(keys);
    }
}

/*
 * The same attention for selected (packed row, head) pairs only.
 * o [n,d], lse [n].
 */
void oracle_attn_fwd_rows(const float *q, const float *k, const float *v, const int32_t *cu,
                          int32_t nseq, int32_t hq, int32_t hkv, int32_t d, double scale,
                          const int64_t *rows, const int32_t *heads, int64_t n, double *o,
                          double *lse) {
    int32_t G = hq / hkv;
    int64_t Lmax = max_len(cu, nseq);
#pragma omp parallel
    {
        double *sbuf = (double *)malloc(sizeof(double) * Lmax);
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * Lmax);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n; ++t) {
            int64_t p = rows[t];
            int32_t h = heads[t];
            int32_t i = seq_of(cu, nseq, p);
            int64_t nk = 0;
            for (int64_t kp = cu[i]; kp <= p; ++kp) keys[nk++] = kp;
            softmax_row(q + ((size_t)p * hq + h) * d, k, v, hkv, h / G, d, scale, keys, nk, sbuf,
                        o + (size_t)t * d, lse + t);
        }
        free(sbuf);
        free(keys);
    }
}

/*
 * General masked attention: q [tq,hq,d], k/v [tk,hkv,d], mask [tq*tk] (1 =
 * visible) -> o [tq,hq,d], lse [hq,tq].  Rows with no visible key: 0, -inf.
 */
void oracle_masked_attn(const float *q, const float *k, const float *v, const uint8_t *mask,
                        int64_t tq, int64_t tk, int32_t hq, int32_t hkv, int32_t d, double scale,
                        double *o, double *lse) {
    int32_t G = hq / hkv;
#pragma omp parallel
    {
        double *sbuf = (double *)malloc(sizeof(double) * (tk ? tk : 1));
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (tk ? tk : 1));
#pragma omp for schedule(dynamic, 16) collapse(2)
        for (int32_t h = 0; h < hq; ++h)
            for (int64_t r = 0; r < tq; ++r) {
                int64_t nk = 0;
                for (int64_t c = 0; c < tk; ++c)
                    if (mask[r * tk + c]) keys[nk++] = c;
                softmax_row(q + ((size_t)r * hq + h) * d, k, v, hkv, h / G, d, scale, keys, nk, sbuf,
                            o + ((size_t)r * hq + h) * d, lse + (size_t)h * tq + r);
            }
        free(sbuf);
        free(keys);
    }
}

/* ------------------------------------------------------------------------- */
/* Ring steps                                                                */
/* ------------------------------------------------------------------------- */

/*
 * Visibility of ring step (rank, step): mask[(T/cp) x (T/cp)], row = rank's
 * zigzag row, column = key row inside shard j = (rank - step) mod cp.
 */
int oracle_step_mask(const int32_t *cu, int32_t nseq, int32_t cp, int32_t rank, int32_t step,
                     uint8_t *mask) {
    if (oracle_check_lengths(cu, nseq, cp) || rank < 0 || rank >= cp || step < 0 || step >= cp)
        return -1;
    int64_t T = total_tokens(cu, nseq), n = T / cp;
    int32_t j = ((rank - step) % cp + cp) % cp;
    int64_t *src = zigzag_src(cu, nseq, cp);
#pragma omp parallel for schedule(static)
    for (int64_t a = 0; a < n; ++a)
        for (int64_t b = 0; b < n; ++b)
            mask[a * n + b] = (uint8_t)visible(cu, nseq, src[rank * n + a], src[j * n + b]);
    free(src);
    return 0;
}

/*
 * Partial result of ring step (rank, step) on zigzag-ordered tensors:
 * q_zz [T,hq,d], k_zz/v_zz [T,hkv,d] -> o_part [T/cp,hq,d], lse_part [hq,T/cp].
 */
int oracle_ring_step_fwd(const float *q_zz, const float *k_zz, const float *v_zz, const int32_t *cu,
                         int32_t nseq, int32_t cp, int32_t rank, int32_t step, int32_t hq,
                         int32_t hkv, int32_t d, double scale, double *o_part, double *lse_part) {
    int64_t T = total_tokens(cu, nseq), n = T / cp;
    uint8_t *mask = (uint8_t *)malloc((size_t)n * n);
    if (oracle_step_mask(cu, nseq, cp, rank, step, mask)) { free(mask); return -1; }
    int32_t j = ((rank - step) % cp + cp) % cp;
    oracle_masked_attn(q_zz + (size_t)rank * n * hq * d, k_zz + (size_t)j * n * hkv * d,
                       v_zz + (size_t)j * n * hkv * d, mask, n, n, hq, hkv, d, scale, o_part,
                       lse_part);
    free(mask);
    return 0;
}

/*
 * (o_a, lse_a) <- (o_a, lse_a) merged with (o_b, lse_b).
 * o [rows,heads,d], lse [heads,rows].  (0, -inf) is the identity.
 */
void oracle_lse_merge(double *o_a, double *lse_a, const double *o_b, const double *lse_b,
                      int64_t rows, int32_t heads, int32_t d) {
    for (int32_t h = 0; h < heads; ++h)
        for (int64_t r = 0; r < rows; ++r) {
            double a = lse_a[(size_t)h * rows + r], b = lse_b[(size_t)h * rows + r];
            double m = a > b ? a : b;
            double *oa = o_a + ((size_t)r * heads + h) * d;
            const double *ob = o_b + ((size_t)r * heads + h) * d;
            if (m == -INFINITY) {
                for (int32_t e = 0; e < d; ++e) oa[e] = 0.0;
                lse_a[(size_t)h * rows + r] = -INFINITY;
                continue;
            }
            double L = m + log(exp(a - m) + exp(b - m));
            double wa = exp(a - L), wb = exp(b - L);
            for (int32_t e = 0; e < d; ++e) oa[e] = wa * oa[e] + wb * ob[e];
            lse_a[(size_t)h * rows + r] = L;
        }
}

/* ------------------------------------------------------------------------- */
/* Backward                                                                  */
/* ------------------------------------------------------------------------- */

/*
 * Per (head, packed row): the row's LSE and D = sum_k P_qk dP_qk, where
 * dP_qk = <dO_q, V_k>.  lse, dsum: [hq,T].
 */
static void bwd_row_stats(const float *q, const float *k, const float *v, const float *dout,
                          const int32_t *cu, int32_t nseq, int32_t hq, int32_t hkv, int32_t d,
                          double scale, int64_t p, int32_t h, double *sbuf, double *lse_out,
                          double *dsum_out) {
    int32_t G = hq / hkv, g = h / G;
    int32_t i = seq_of(cu, nseq, p);
    const float *qr = q + ((size_t)p * hq + h) * d;
    const float *dor = dout + ((size_t)p * hq + h) * d;
    int64_t nk = p - cu[i] + 1;
    double m = -INFINITY;
    for (int64_t t = 0; t < nk; ++t) {
        sbuf[t] = scale * dot(qr, k + ((size_t)(cu[i] + t) * hkv + g) * d, d);
        if (sbuf[t] > m) m = sbuf[t];
    }
    double l = 0.0;
    for (int64_t t = 0; t < nk; ++t) l += exp(sbuf[t] - m);
    double lse = m + log(l);
    double ds = 0.0;
    for (int64_t t = 0; t < nk; ++t) {
        double P = exp(sbuf[t] - lse);
        ds += P * dot(dor, v + ((size_t)(cu[i] + t) * hkv + g) * d, d);
    }
    *lse_out = lse;
    *dsum_out = ds;
}

/*
 * Gradients of the attention above with respect to q, k, v for upstream
 * gradient dout [T,hq,d]. dq [T,hq,d], dk/dv [T,hkv,d]; all packed layout.
 * Three plain passes: row statistics, then dK/dV per key row, then dQ per
 * query row (no shared accumulators, so the passes parallelise freely).
 */
void oracle_attn_bwd(const float *q, const float *k, const float *v, const float *dout,
                     const int32_t *cu, int32_t nseq, int32_t hq, int32_t hkv, int32_t d,
                     double scale, double *dq, double *dk, double *dv) {
    int64_t T = total_tokens(cu, nseq);
    int32_t G = hq / hkv;
    int64_t Lmax = max_len(cu, nseq);
    double *lse = (double *)malloc(sizeof(double) * T * hq);
    double *dsum = (double *)malloc(sizeof(double) * T * hq);
#pragma omp parallel
    {
        double *sbuf = (double *)malloc(sizeof(double) * Lmax);
#pragma omp for schedule(dynamic, 16) collapse(2)
        for (int32_t h = 0; h < hq; ++h)
            for (int64_t p = 0; p < T; ++p)
                bwd_row_stats(q, k, v, dout, cu, nseq, hq, hkv, d, scale, p, h, sbuf,
                              lse + (size_t)h * T + p, dsum + (size_t)h * T + p);
        free(sbuf);
    }
    /* dK, dV: key row kp of kv head g collects from every query row pq >= kp of
     * its sequence and every query head of the group. */
#pragma omp parallel for schedule(dynamic, 16) collapse(2)
    for (int32_t g = 0; g < hkv; ++g)
        for (int64_t kp = 0; kp < T; ++kp) {
            int32_t i = seq_of(cu, nseq, kp);
            const float *kr = k + ((size_t)kp * hkv + g) * d;
            const float *vr = v + ((size_t)kp * hkv + g) * d;
            double *dkr = dk + ((size_t)kp * hkv + g) * d;
            double *dvr = dv + ((size_t)kp * hkv + g) * d;
            for (int32_t e = 0; e < d; ++e) dkr[e] = dvr[e] = 0.0;
            for (int32_t h = g * G; h < (g + 1) * G; ++h)
                for (int64_t pq = kp; pq < cu[i + 1]; ++pq) {
                    const float *qr = q + ((size_t)pq * hq + h) * d;
                    const float *dor = dout + ((size_t)pq * hq + h) * d;
                    double P = exp(scale * dot(qr, kr, d) - lse[(size_t)h * T + pq]);
                    double dS = P * (dot(dor, vr, d) - dsum[(size_t)h * T + pq]);
                    for (int32_t e = 0; e < d; ++e) {
                        dvr[e] += P * (double)dor[e];
                        dkr[e] += scale * dS * (double)qr[e];
                    }
                }
        }
    /* dQ: query row pq of head h collects from keys kp <= pq of its sequence. */
#pragma omp parallel for schedule(dynamic, 16) collapse(2)
    for (int32_t h = 0; h < hq; ++h)
        for (int64_t pq = 0; pq < T; ++pq) {
            int32_t i = seq_of(cu, nseq, pq), g = h / G;
            const float *qr = q + ((size_t)pq * hq + h) * d;
            const float *dor = dout + ((size_t)pq * hq + h) * d;
            double *dqr = dq + ((size_t)pq * hq + h) * d;
            for (int32_t e = 0; e < d; ++e) dqr[e] = 0.0;
            for (int64_t kp = cu[i]; kp <= pq; ++kp) {
                const float *kr = k + ((size_t)kp * hkv + g) * d;
                const float *vr = v + ((size_t)kp * hkv + g) * d;
                double P = exp(scale * dot(qr, kr, d) - lse[(size_t)h * T + pq]);
                double dS = P * (dot(dor, vr, d) - dsum[(size_t)h * T + pq]);
                for (int32_t e = 0; e < d; ++e) dqr[e] += scale * dS * (double)kr[e];
            }
        }
    free(lse);
    free(dsum);
}

/*
 * dQ for selected (packed row, head) pairs only: dq [n,d].  Each row needs
 * only its own LSE and D, so this is exact at any size.
 */
void oracle_attn_bwd_dq_rows(const float *q, const float *k, const float *v, const float *dout,
                             const int32_t *cu, int32_t nseq, int32_t hq, int32_t hkv, int32_t d,
                             double scale, const int64_t *rows, const int32_t *heads, int64_t n,
                             double *dq) {
    int32_t G = hq / hkv;
    int64_t Lmax = max_len(cu, nseq);
#pragma omp parallel
    {
        double *sbuf = (double *)malloc(sizeof(double) * Lmax);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n; ++t) {
            int64_t pq = rows[t];
            int32_t h = heads[t], g = h / G, i = seq_of(cu, nseq, pq);
            double lse, ds;
            bwd_row_stats(q, k, v, dout, cu, nseq, hq, hkv, d, scale, pq, h, sbuf, &lse, &ds);
            const float *qr = q + ((size_t)pq * hq + h) * d;
            const float *dor = dout + ((size_t)pq * hq + h) * d;
            double *dqr = dq + (size_t)t * d;
            for (int32_t e = 0; e < d; ++e) dqr[e] = 0.0;
            for (int64_t kp = cu[i]; kp <= pq; ++kp) {
                const float *kr = k + ((size_t)kp * hkv + g) * d;
                double P = exp(scale * dot(qr, kr, d) - lse);
                double dS = P * (dot(dor, v + ((size_t)kp * hkv + g) * d, d) - ds);
                for (int32_t e = 0; e < d; ++e) dqr[e] += scale * dS * (double)kr[e];
            }
        }
        free(sbuf);
    }
}

/*
 * dK and dV for selected (packed key row, key/value head) pairs only:
 * dk, dv [n,d].  Key row kp of head g collects, from every query head h of
 * the group and every query row pq >= kp of its sequence,
 *   dV += P_qk dO_q  and  dK += scale * dS_qk Q_q,
 * with P = exp(S - LSE_q) and dS = P (dP - D_q) taken from the query row's own
 * LSE and D (bwd_row_stats, the same definitions as oracle_attn_bwd), so the
 * result is exact at any size.  head_on (int32[hq], or NULL for every head)
 * leaves out heads with head_on[h] == 0: the caller uses it only for heads
 * whose dO is identically zero, which add exactly nothing (dP = 0 and D = 0
 * give dS = 0, and P dO = 0).  The row statistics of every (head, row) the
 * selected keys need are computed once, before the sums -- unless the caller
 * passes them: lse_in and dsum_in ([hq,T], both or neither) then hold each
 * needed row's LSE and D = sum_k P_qk dP_qk = <dO_q, O_q> (O the row's
 * attention output), e.g. from oracle_attn_fwd_rows of the same inputs.
 */
void oracle_attn_bwd_dkv_rows(const float *q, const float *k, const float *v, const float *dout,
                              const int32_t *cu, int32_t nseq, int32_t hq, int32_t hkv, int32_t d,
                              double scale, const int64_t *rows, const int32_t *kv_heads, int64_t n,
                              const int32_t *head_on, const double *lse_in, const double *dsum_in,
                              double *dk, double *dv) {
    int64_t T = total_tokens(cu, nseq);
    int32_t G = hq / hkv;
    int64_t Lmax = max_len(cu, nseq);
    /* need[h*T + pq]: the statistics of query row pq of head h are used */
    uint8_t *need = (uint8_t *)calloc((size_t)hq * T, 1);
    double *lse_own = NULL, *dsum_own = NULL;
    if (!lse_in) {
        lse_own = (double *)malloc(sizeof(double) * hq * T);
        dsum_own = (double *)malloc(sizeof(double) * hq * T);
    }
    const double *lse = lse_in ? lse_in : lse_own;
    const double *dsum = lse_in ? dsum_in : dsum_own;
    for (int64_t t = 0; t < n; ++t) {
        int32_t i = seq_of(cu, nseq, rows[t]);
        for (int32_t h = kv_heads[t] * G; h < (kv_heads[t] + 1) * G; ++h) {
            if (head_on && !head_on[h]) continue;
            for (int64_t pq = rows[t]; pq < cu[i + 1]; ++pq) need[(size_t)h * T + pq] = 1;
        }
    }
    if (!lse_in) {
#pragma omp parallel
        {
            double *sbuf = (double *)malloc(sizeof(double) * Lmax);
#pragma omp for schedule(dynamic, 16) collapse(2)
            for (int32_t h = 0; h < hq; ++h)
                for (int64_t p = 0; p < T; ++p)
                    if (need[(size_t)h * T + p])
                        bwd_row_stats(q, k, v, dout, cu, nseq, hq, hkv, d, scale, p, h, sbuf,
                                      lse_own + (size_t)h * T + p, dsum_own + (size_t)h * T + p);
            free(sbuf);
        }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < n; ++t) {
        int64_t kp = rows[t];
        int32_t g = kv_heads[t], i = seq_of(cu, nseq, kp);
        const float *kr = k + ((size_t)kp * hkv + g) * d;
        const float *vr = v + ((size_t)kp * hkv + g) * d;
        double *dkr = dk + (size_t)t * d;
        double *dvr = dv + (size_t)t * d;
        for (int32_t e = 0; e < d; ++e) dkr[e] = dvr[e] = 0.0;
        for (int32_t h = g * G; h < (g + 1) * G; ++h) {
            if (head_on && !head_on[h]) continue;
            for (int64_t pq = kp; pq < cu[i + 1]; ++pq) {
                const float *qr = q + ((size_t)pq * hq + h) * d;
                const float *dor = dout + ((size_t)pq * hq + h) * d;
                double P = exp(scale * dot(qr, kr, d) - lse[(size_t)h * T + pq]);
                double dS = P * (dot(dor, vr, d) - dsum[(size_t)h * T + pq]);
                for (int32_t e = 0; e < d; ++e) {
                    dvr[e] += P * (double)dor[e];
                    dkr[e] += scale * dS * (double)qr[e];
                }
            }
        }
    }
    free(need);
    free(lse_own);
    free(dsum_own);
}

/* ------------------------------------------------------------------------- */
/* Tiles and work balance                                                    */
/* ------------------------------------------------------------------------- */

/*
 * Tile grid of one rank's rows (or one shard's keys): for every sequence, its
 * two zigzag chunks in shard order, each cut into pieces of `step` rows from
 * the chunk start (the last piece may be shorter).  Writes [start, end) pairs
 * in local row indices; returns the count.
 */
static int64_t chunk_grid(const int32_t *cu, int32_t nseq, int32_t cp, int32_t step, int64_t *se) {
    int64_t n = 0, row = 0;
    for (int32_t i = 0; i < nseq; ++i) {
        int64_t c = ((int64_t)cu[i + 1] - cu[i]) / (2 * cp);
        for (int u = 0; u < 2; ++u) {
            for (int64_t a = 0; a < c; a += step) {
                se[2 * n] = row + a;
                se[2 * n + 1] = row + (a + step < c ? a + step : c);
                ++n;
            }
            row += c;
        }
    }
    return n;
}

/*
 * Tiles of ring step (rank, step) that hold at least one visible pair, sorted
 * by (q0, k0): out[5*t..] = q0, q1, k0, k1, kind with kind 1 = every pair
 * visible, 2 = some but not all.  Local row indices (rank rows, shard keys).
 * Returns 0, or -1 on bad arguments, or -2 if cap is too small (n still set).
 */
int oracle_tiles(const int32_t *cu, int32_t nseq, int32_t cp, int32_t rank, int32_t step,
                 int32_t bm, int32_t bn, int32_t *out, int64_t cap, int64_t *n_out) {
    if (oracle_check_lengths(cu, nseq, cp) || bm < 1 || bn < 1 || rank < 0 || rank >= cp ||
        step < 0 || step >= cp)
        return -1;
    int64_t T = total_tokens(cu, nseq), n = T / cp;
    uint8_t *mask = (uint8_t *)malloc((size_t)n * n);
    oracle_step_mask(cu, nseq, cp, rank, step, mask);
    int64_t *qs = (int64_t *)malloc(sizeof(int64_t) * 2 * (n + 2 * nseq));
    int64_t *ks = (int64_t *)malloc(sizeof(int64_t) * 2 * (n + 2 * nseq));
    int64_t nq = chunk_grid(cu, nseq, cp, bm, qs), nk = chunk_grid(cu, nseq, cp, bn, ks);
    int64_t cnt = 0;
    for (int64_t a = 0; a < nq; ++a)
        for (int64_t b = 0; b < nk; ++b) {
            int64_t vis = 0, area = (qs[2 * a + 1] - qs[2 * a]) * (ks[2 * b + 1] - ks[2 * b]);
            for (int64_t x = qs[2 * a]; x < qs[2 * a + 1]; ++x)
                for (int64_t y = ks[2 * b]; y < ks[2 * b + 1]; ++y) vis += mask[x * n + y];
            if (vis == 0) continue;
            if (cnt < cap) {
                int32_t *t = out + 5 * cnt;
                t[0] = (int32_t)qs[2 * a];
                t[1] = (int32_t)qs[2 * a + 1];
                t[2] = (int32_t)ks[2 * b];
                t[3] = (int32_t)ks[2 * b + 1];
                t[4] = vis == area ? 1 : 2;
            }
            ++cnt;
        }
    free(mask);
    free(qs);
    free(ks);
    *n_out = cnt;
    return cnt <= cap ? 0 : -2;
}

/*
 * Visible (query, key) pairs per rank over all ring steps, counted one pair
 * at a time: out[cp].
 */
int oracle_rank_pairs(const int32_t *cu, int32_t nseq, int32_t cp, int64_t *out) {
    if (oracle_check_lengths(cu, nseq, cp)) return -1;
    int64_t T = total_tokens(cu, nseq), n = T / cp;
    int64_t *src = zigzag_src(cu, nseq, cp);
    for (int32_t r = 0; r < cp; ++r) {
        int64_t cnt = 0;
#pragma omp parallel for reduction(+ : cnt) schedule(dynamic, 64)
        for (int64_t a = 0; a < n; ++a)
            for (int64_t kz = 0; kz < T; ++kz) cnt += visible(cu, nseq, src[r * n + a], src[kz]);
        out[r] = cnt;
    }
    free(src);
    return 0;
}

/* Threads the oracle's parallel loops use. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
