/*
 * aba_oracle.c -- plain, slow, fp64 CPU model of the AB-Attention sparse
 * attention layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: it exists so that the HIP kernels can be checked against an
 * independent implementation.  It shares no code, header, table or constant
 * generator with the HIP library.
 *
 * Source: "AB-Attention ускорил генерацию видео до 2,23× и пропускает 92%
 * внимания" (Hamidun News), sections "Три приёма AB-Attention" (IBCS, SIP and
 * the fine-grained kernel paragraph) and the lede.  The page gives prose only:
 * every formula below is the plainest reading of that prose, and each place
 * where a reading had to be chosen is marked READING.
 *
 * Conventions
 *   q, k, v   : float32 arrays [B, H, N_pad, D] (D fastest).  bf16 inputs are
 *               passed widened to float32, which is exact.  All arithmetic is
 *               done in double.
 *   N         : valid tokens; rows >= N are padding and are ignored.
 *   blk       : tokens per query block (128: the page's query blocks).
 *               NB = ceil(N / blk).
 *   kblk      : tokens per key block: 128, or 4 for the fine-grained
 *               selection of the page's third paragraph ("Три приёма
 *               AB-Attention", the kernel paragraph: key/value blocks of 4
 *               tokens).  NBk = ceil(N / kblk).  Pooling, scoring, sampling,
 *               attention and the attention mass all work per key block of
 *               kblk tokens; clustering works per query block of blk.
 *   items     : optional list of (b, h, query-block) triples, int32[n][3], so
 *               that large layers can be checked on a sample of query blocks.
 *
 * Parity pins for every function live in tests/ (see the test files named
 * test_oracle_*.py); none of them retypes the formulas below.
 */
#define _GNU_SOURCE /* qsort_r */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define TWO32 4294967296.0

#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the OpenMP loops below use (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------- */
/* O0 -- blocks.  Query block / key block j covers tokens                  */
/* [blk*j, min(blk*j + blk, N)): the page splits queries into contiguous     */
/* 128-token blocks and computes in the original token order (IBCS          */
/* paragraph).                                                              */
/* ---------------------------------------------------------------------- */
int oracle_n_blocks(int n_valid, int blk) { return (n_valid + blk - 1) / blk; }

static int rows_in_block(int n_valid, int blk, int j)
{
    int lo = j * blk;
    int hi = lo + blk < n_valid ? lo + blk : n_valid;
    return hi > lo ? hi - lo : 0;
}

static const float *row_ptr(const float *base, int H, long n_pad, int D, int b, int h, long t)
{
    return base + (((long)b * H + h) * n_pad + t) * (long)D;
}

static int same_centroid(const double *cent, int D, int m1, int m2)
{
    for (int d = 0; d < D; ++d)
        if (cent[(long)m1 * D + d] != cent[(long)m2 * D + d]) return 0;
    return 1;
}

/* Assignment step: a[i] = argmin_m |x_i - c_m|^2, ties to the smallest m.
 * Returns the smallest relative gap (d2 - d1) / d2 over the rows, where d2 is
 * the nearest centroid that differs from the chosen one (1 if there is none).
 * Copies of the chosen centroid (a block with fewer rows than clusters starts
 * with repeated rows) tie with it exactly in any precision and so do not make
 * the assignment fragile; a different centroid at the same distance does. */
static double assign_rows(const float *x, long ld, int n, int D, int C, const double *cent, int *a)
{
    double min_gap = 1.0;
    for (int i = 0; i < n; ++i) {
        double best = INFINITY, second = INFINITY;
        int bm = 0;
        for (int m = 0; m < C; ++m) {
            double dist = 0.0;
            for (int d = 0; d < D; ++d) {
                double diff = (double)x[(long)i * ld + d] - cent[(long)m * D + d];
                dist += diff * diff;
            }
            if (dist < best) {
                second = best;
                best = dist;
                bm = m;
            } else if (dist == best && same_centroid(cent, D, m, bm)) {
                /* a copy of the chosen centroid */
            } else if (dist < second) {
                second = dist;
            }
        }
        a[i] = bm;
        if (second < INFINITY) {
            double gap = second > 0.0 ? (second - best) / second : 0.0;
            if (gap < min_gap) min_gap = gap;
        }
    }
    return min_gap;
}

/* ---------------------------------------------------------------------- */
/* O1 -- IBCS clustering of one query block.                               */
/* The page: the queries of a block are grouped into C = 8 clusters, each   */
/* with a centroid and a weight equal to the share of the block's queries   */
/* that fall in it (IBCS paragraph).                                        */
/* READING: textbook Lloyd k-means with squared Euclidean distance;         */
/* deterministic strided init c_m = x[floor(m*n/C)]; exactly T rounds of    */
/* (assign, update); ties go to the smallest m; an empty cluster keeps its  */
/* centroid; weights from the last assignment.                              */
/*                                                                          */
/* x: n rows of D floats, row stride ld.  cent: C*D, weight: C.            */
/* assign (nullable): n ints, the last assignment.                          */
/* Returns the smallest relative gap (d2 - d1) / d2 between the best and    */
/* the second-best squared distance seen in any assignment (1 if C == 1),   */
/* so callers can tell near-ties, where fp32 and fp64 may disagree.         */
/* ---------------------------------------------------------------------- */
double oracle_kmeans_block(const float *x, long ld, int n, int D, int C, int T,
                           double *cent, double *weight, int *assign)
{
    int *a = (int *)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    long *count = (long *)calloc((size_t)C, sizeof(long));
    double *sum = (double *)calloc((size_t)C * D, sizeof(double));
    double min_gap = 1.0;

    for (int m = 0; m < C; ++m) {
        long r = (long)m * n / C;
        for (int d = 0; d < D; ++d) cent[(long)m * D + d] = n > 0 ? (double)x[r * ld + d] : 0.0;
    }

    for (int it = 0; it < T; ++it) {
        double g = assign_rows(x, ld, n, D, C, cent, a);
        if (g < min_gap) min_gap = g;
        /* update step: mean of the rows assigned to each cluster */
        memset(count, 0, sizeof(long) * (size_t)C);
        memset(sum, 0, sizeof(double) * (size_t)C * D);
        for (int i = 0; i < n; ++i) {
            count[a[i]] += 1;
            for (int d = 0; d < D; ++d) sum[(long)a[i] * D + d] += (double)x[(long)i * ld + d];
        }
        for (int m = 0; m < C; ++m)
            if (count[m] > 0)
                for (int d = 0; d < D; ++d) cent[(long)m * D + d] = sum[(long)m * D + d] / (double)count[m];
    }
    if (T == 0) assign_rows(x, ld, n, D, C, cent, a); /* no rounds: weights of the initial centroids */

    /* weight = share of the block's queries in the cluster (last assignment) */
    memset(count, 0, sizeof(long) * (size_t)C);
    for (int i = 0; i < n; ++i) count[a[i]] += 1;
    for (int m = 0; m < C; ++m) weight[m] = n > 0 ? (double)count[m] / (double)n : 0.0;
    if (assign)
        for (int i = 0; i < n; ++i) assign[i] = a[i];

    free(a);
    free(count);
    free(sum);
    return min_gap;
}

/* Whole layer: cent [B,H,NB,C,D], weight [B,H,NB,C], gap (nullable) [B,H,NB]. */
void oracle_kmeans(const float *q, int B, int H, int N, int N_pad, int D, int blk, int C, int T,
                   double *cent, double *weight, double *gap)
{
    int NB = oracle_n_blocks(N, blk);
    long total = (long)B * H * NB;
#pragma omp parallel for schedule(dynamic)
    for (long it = 0; it < total; ++it) {
        int j = (int)(it % NB);
        int h = (int)((it / NB) % H);
        int b = (int)(it / ((long)NB * H));
        const float *x = row_ptr(q, H, N_pad, D, b, h, (long)j * blk);
        double g = oracle_kmeans_block(x, D, rows_in_block(N, blk, j), D, C, T,
                                       cent + it * (long)C * D, weight + it * C, NULL);
        if (gap) gap[it] = g;
    }
}

/* ---------------------------------------------------------------------- */
/* O2 -- mean-pooled keys.  Each key block is represented by the mean of    */
/* its keys (IBCS paragraph: "averaged keys").                              */
/* READING: padding rows (t >= N) are excluded; the partial last block is   */
/* the mean of its valid keys only.                                         */
/* kbar: [B,H,NB,D].                                                        */
/* ---------------------------------------------------------------------- */
void oracle_pool(const float *k, int B, int H, int N, int N_pad, int D, int blk, double *kbar)
{
    int NB = oracle_n_blocks(N, blk);
    long total = (long)B * H * NB;
#pragma omp parallel for schedule(static)
    for (long it = 0; it < total; ++it) {
        int j = (int)(it % NB);
        int h = (int)((it / NB) % H);
        int b = (int)(it / ((long)NB * H));
        int n = rows_in_block(N, blk, j);
        const float *x = row_ptr(k, H, N_pad, D, b, h, (long)j * blk);
        for (int d = 0; d < D; ++d) {
            double s = 0.0;
            for (int t = 0; t < n; ++t) s += (double)x[(long)t * D + d];
            kbar[it * D + d] = s / (double)n;
        }
    }
}

/* ---------------------------------------------------------------------- */
/* O3 -- IBCS block score.  A key block's score is the cluster-weighted     */
/* attention of the centroids to its averaged keys (IBCS paragraph).        */
/* READING: per-centroid softmax over all key blocks of the row with the    */
/* attention scale s, then the weighted sum over centroids:                 */
/*   l_mj = s * c_m . kbar_j,  a_mj = softmax_j(l_mj),  S_j = sum_m w_m a_mj */
/* so each row of S is a distribution over key blocks.                      */
/* cent [B,H,NBq,C,D], weight [B,H,NBq,C], kbar [B,H,NBk,D] -> scores        */
/* [B,H,NBq,NBk] (double).                                                  */
/* ---------------------------------------------------------------------- */
void oracle_score(const double *cent, const double *weight, const double *kbar, int B, int H,
                  int NBq, int NBk, int C, int D, double scale, double *scores)
{
    long total = (long)B * H * NBq;
#pragma omp parallel for schedule(dynamic)
    for (long it = 0; it < total; ++it) {
        long bh = it / NBq;
        const double *c = cent + it * (long)C * D;
        const double *w = weight + it * C;
        const double *kb = kbar + bh * (long)NBk * D;
        double *row = scores + it * (long)NBk;
        double *logit = (double *)malloc(sizeof(double) * (size_t)NBk);
        for (int j = 0; j < NBk; ++j) row[j] = 0.0;
        for (int m = 0; m < C; ++m) {
            double mx = -INFINITY, z = 0.0;
            for (int j = 0; j < NBk; ++j) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += c[(long)m * D + d] * kb[(long)j * D + d];
                logit[j] = scale * dot;
                if (logit[j] > mx) mx = logit[j];
            }
            for (int j = 0; j < NBk; ++j) z += exp(logit[j] - mx);
            for (int j = 0; j < NBk; ++j) row[j] += w[m] * exp(logit[j] - mx) / z;
        }
        free(logit);
    }
}

/* ---------------------------------------------------------------------- */
/* O4 -- SIP inclusion thresholds for one row of scores.                    */
/* The page: a block enters the sample with probability proportional to its */
/* score; the most important blocks are always taken; every other block     */
/* keeps a non-zero chance (SIP paragraph).                                 */
/* READING (exact integer form, so that every implementation takes the     */
/* same decisions):                                                         */
/*   sigma_j = clamp(floor(S_j * 2^32), 1, 2^32)   (S_j fp32; NaN -> 1)     */
/*   order j by (sigma desc, j asc); the first block is always kept;        */
/*   capped blocks grow while (K - t) * sigma_(t+1) >= R, where R is the    */
/*   sum of sigma over the blocks not yet capped (water-filling);           */
/*   capped: theta = 2^32; others: theta = clamp(ceil((K-t)*sigma*2^32/R),  */
/*   1, 2^32), or 1 when K - t <= 0.                                        */
/* The inclusion probability is theta / 2^32, so sum_j pi_j = K whenever   */
/* not every block caps.  Returns t, the number of always-kept blocks.     */
/* ---------------------------------------------------------------------- */
static int cmp_sigma_desc(const void *pa, const void *pb, void *arg)
{
    const uint64_t *sigma = (const uint64_t *)arg;
    int a = *(const int *)pa, b = *(const int *)pb;
    uint64_t sa = sigma[a], sb = sigma[b];
    if (sa != sb) return sa > sb ? -1 : 1;
    return a < b ? -1 : (a > b ? 1 : 0);
}

static uint64_t fixed_point_score(float s)
{
    const uint64_t one = (uint64_t)1 << 32;
    if (!(s > 0.0f)) return 1; /* zero, negative or NaN */
    double v = floor((double)s * TWO32);
    if (v >= (double)one) return one;
    uint64_t r = (uint64_t)v;
    return r < 1 ? 1 : r;
}

int oracle_thresholds(const float *scores, int NB, int K, uint64_t *theta)
{
    const uint64_t one = (uint64_t)1 << 32;
    uint64_t *sigma = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)NB);
    int *ord = (int *)malloc(sizeof(int) * (size_t)NB);
    uint64_t total = 0;
    for (int j = 0; j < NB; ++j) {
        sigma[j] = fixed_point_score(scores[j]);
        ord[j] = j;
        total += sigma[j];
    }
    qsort_r(ord, (size_t)NB, sizeof(int), cmp_sigma_desc, sigma);

    int t = 1;
    uint64_t R = total - sigma[ord[0]];
    while (t < NB && K - t > 0 && (uint64_t)(K - t) * sigma[ord[t]] >= R) {
        R -= sigma[ord[t]];
        t += 1;
    }
    for (int i = 0; i < NB; ++i) {
        int j = ord[i];
        if (i < t) {
            theta[j] = one;
        } else if (K - t <= 0) {
            theta[j] = 1;
        } else {
            unsigned __int128 num = (unsigned __int128)((uint64_t)(K - t) * sigma[j]) << 32;
            unsigned __int128 q = num / R;
            if (q * R != num) q += 1; /* ceiling */
            if (q < 1) q = 1;
            if (q > one) q = one;
            theta[j] = (uint64_t)q;
        }
    }
    free(sigma);
    free(ord);
    return t;
}

/* ---------------------------------------------------------------------- */
/* O5 -- draws.  Philox4x32-10, the counter-based generator of Salmon,     */
/* Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"     */
/* (SC'11): ten rounds of two 32x32->64 multiplies with the published       */
/* multipliers, the key bumped by the published Weyl constants between      */
/* rounds.                                                                  */
/* ---------------------------------------------------------------------- */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* The uniform 32-bit word drawn for key block j of query block qb in head h */
/* of batch b: word (j & 3) of Philox4x32-10 with key (seed_lo, seed_hi)     */
/* and counter (j >> 2, qb, h, b).                                          */
uint32_t oracle_draw(uint64_t seed, int b, int h, int qb, int j)
{
    uint32_t ctr[4] = {(uint32_t)j >> 2, (uint32_t)qb, (uint32_t)h, (uint32_t)b};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return out[j & 3];
}

/* SIP sampling plan for a whole layer.  A block is kept iff its draw is    */
/* below its threshold (so P(kept) = theta / 2^32); kept blocks are listed   */
/* in ascending order with the Horvitz-Thompson weight 1 / pi = 2^32/theta   */
/* (SIP paragraph: a block with probability 25% counts as four).            */
/* scores [B,H,NBq,NBk] fp32; idx/w [B,H,NBq,cap]; cnt [B,H,NBq].           */
/* theta_out (nullable) [B,H,NBq,NBk].                                      */
/* READING: the scores may be a slice of a larger layer, heads h0 .. h0+H-1  */
/* of batch entries b0 .. b0+B-1; the draws are addressed by those global    */
/* indices, so a slice draws exactly what the whole layer draws for it.     */
void oracle_sample(const float *scores, int B, int H, int NBq, int NBk, int K, uint64_t seed, int cap, int h0,
                   int b0, int32_t *idx, int32_t *cnt, float *w, uint64_t *theta_out)
{
    long total = (long)B * H * NBq;
#pragma omp parallel for schedule(dynamic)
    for (long it = 0; it < total; ++it) {
        int qb = (int)(it % NBq);
        int h = (int)((it / NBq) % H);
        int b = (int)(it / ((long)NBq * H));
        uint64_t *theta = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)NBk);
        oracle_thresholds(scores + it * (long)NBk, NBk, K, theta);
        int n = 0;
        for (int j = 0; j < NBk; ++j) {
            uint32_t r = oracle_draw(seed, b0 + b, h0 + h, qb, j);
            if ((uint64_t)r < theta[j]) {
                if (n < cap) {
                    idx[it * (long)cap + n] = j;
                    w[it * (long)cap + n] = (float)(TWO32 / (double)theta[j]);
                }
                ++n;
            }
        }
        cnt[it] = n;
        if (theta_out)
            for (int j = 0; j < NBk; ++j) theta_out[it * (long)NBk + j] = theta[j];
        free(theta);
    }
}

/* ---------------------------------------------------------------------- */
/* O6 -- attention over a sampling plan.  Each kept block is multiplied by   */
/* its inverse inclusion probability in both the numerator and the softmax  */
/* normaliser (Horvitz-Thompson), which is plain softmax attention with the */
/* logits of block j shifted by ln w_j (SIP paragraph); the output stays in */
/* the original token order (IBCS paragraph).                               */
/* READING: non-causal; keys >= N are masked; query rows >= N give 0.       */
/*                                                                          */
/* For one query row i with the kept list (j, w_j):                         */
/*   l_t = s * q_i . k_t,   M = shift (if given) else max over kept l_t      */
/*   num = sum_j w_j sum_{t in j} exp(l_t - M) v_t                           */
/*   den = sum_j w_j sum_{t in j} exp(l_t - M)                               */
/*   o_i = num / den                                                         */
/* ---------------------------------------------------------------------- */
static void attend_row(const float *qi, const float *kh, const float *vh, int N, int D, int kblk,
                       double scale, const int32_t *list, const float *wl, int n_list, int have_shift,
                       double shift, double *num, double *den_out, double *logit_buf)
{
    double M = -INFINITY;
    int pos = 0;
    for (int e = 0; e < n_list; ++e) {
        int j = list[e];
        int n = rows_in_block(N, kblk, j);
        for (int t = 0; t < n; ++t) {
            const float *kt = kh + ((long)j * kblk + t) * D;
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += (double)qi[d] * (double)kt[d];
            logit_buf[pos] = scale * dot;
            if (logit_buf[pos] > M) M = logit_buf[pos];
            ++pos;
        }
    }
    if (have_shift) M = shift;
    double den = 0.0;
    for (int d = 0; d < D; ++d) num[d] = 0.0;
    pos = 0;
    for (int e = 0; e < n_list; ++e) {
        int j = list[e];
        double wj = (double)wl[e];
        int n = rows_in_block(N, kblk, j);
        for (int t = 0; t < n; ++t) {
            const float *vt = vh + ((long)j * kblk + t) * D;
            double p = wj * exp(logit_buf[pos] - M);
            den += p;
            for (int d = 0; d < D; ++d) num[d] += p * (double)vt[d];
            ++pos;
        }
    }
    *den_out = den;
}

/* items: int32 [n_items][3] = (b, h, query block).  idx/w: [B,H,NBq,cap]    */
/* (entries are key blocks of kblk tokens), cnt: [B,H,NBq].                  */
/* out: [n_items, blk, D] double.  shift (nullable):                         */
/* [n_items, blk]; when given, num [n_items,blk,D] and den [n_items,blk] are */
/* written too and out = num / den.                                          */
void oracle_attend(const float *q, const float *k, const float *v, int B, int H, int N, int N_pad,
                   int D, int blk, int kblk, double scale, const int32_t *idx, const int32_t *cnt, const float *w,
                   int cap, const int32_t *items, int n_items, const double *shift, double *out,
                   double *num_out, double *den_out)
{
    int NB = oracle_n_blocks(N, blk);
    (void)B;
#pragma omp parallel for schedule(dynamic)
    for (int it = 0; it < n_items; ++it) {
        int b = items[3 * it], h = items[3 * it + 1], qb = items[3 * it + 2];
        long row = ((long)b * H + h) * NB + qb;
        const int32_t *list = idx + row * cap;
        const float *wl = w + row * cap;
        int n_list = cnt[row] < cap ? cnt[row] : cap;
        const float *kh = row_ptr(k, H, N_pad, D, b, h, 0);
        const float *vh = row_ptr(v, H, N_pad, D, b, h, 0);
        double *logit_buf = (double *)malloc(sizeof(double) * ((size_t)n_list * kblk + 1));
        double *num = (double *)malloc(sizeof(double) * (size_t)D);
        int nq = rows_in_block(N, blk, qb);
        for (int r = 0; r < blk; ++r) {
            double *o = out + ((long)it * blk + r) * D;
            if (r >= nq) {
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                if (shift) {
                    for (int d = 0; d < D; ++d) num_out[((long)it * blk + r) * D + d] = 0.0;
                    den_out[(long)it * blk + r] = 0.0;
                }
                continue;
            }
            const float *qi = row_ptr(q, H, N_pad, D, b, h, (long)qb * blk + r);
            double den;
            attend_row(qi, kh, vh, N, D, kblk, scale, list, wl, n_list, shift != NULL,
                       shift ? shift[(long)it * blk + r] : 0.0, num, &den, logit_buf);
            for (int d = 0; d < D; ++d) o[d] = num[d] / den;
            if (shift) {
                for (int d = 0; d < D; ++d) num_out[((long)it * blk + r) * D + d] = num[d];
                den_out[(long)it * blk + r] = den;
            }
        }
        free(logit_buf);
        free(num);
    }
}

/* ---------------------------------------------------------------------- */
/* Dense softmax attention (the full-attention reference the page measures  */
/* against, "Как мерили и что вышло"): every valid query attends to every   */
/* valid key, written independently of the block-list code above.          */
/* items as in oracle_attend; out [n_items, blk, D].                        */
/* ---------------------------------------------------------------------- */
void oracle_attend_full(const float *q, const float *k, const float *v, int B, int H, int N, int N_pad,
                        int D, int blk, double scale, const int32_t *items, int n_items, double *out)
{
    (void)B;
#pragma omp parallel for schedule(dynamic)
    for (int it = 0; it < n_items; ++it) {
        int b = items[3 * it], h = items[3 * it + 1], qb = items[3 * it + 2];
        double *logit = (double *)malloc(sizeof(double) * (size_t)N);
        int nq = rows_in_block(N, blk, qb);
        for (int r = 0; r < blk; ++r) {
            double *o = out + ((long)it * blk + r) * D;
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            if (r >= nq) continue;
            const float *qi = row_ptr(q, H, N_pad, D, b, h, (long)qb * blk + r);
            double mx = -INFINITY, z = 0.0;
            for (int t = 0; t < N; ++t) {
                const float *kt = row_ptr(k, H, N_pad, D, b, h, t);
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += (double)qi[d] * (double)kt[d];
                logit[t] = scale * dot;
                if (logit[t] > mx) mx = logit[t];
            }
            for (int t = 0; t < N; ++t) {
                const float *vt = row_ptr(v, H, N_pad, D, b, h, t);
                double p = exp(logit[t] - mx);
                z += p;
                for (int d = 0; d < D; ++d) o[d] += p * (double)vt[d];
            }
            for (int d = 0; d < D; ++d) o[d] /= z;
        }
        free(logit);
    }
}

/* ---------------------------------------------------------------------- */
/* Attention mass per key block, for the top-k retention diagnostic (the    */
/* page's "share of attention mass kept by ideal top-k", section "Где       */
/* ломаются прежние разреженные схемы"): mass[it][j] = mean over the valid  */
/* queries i of query block qb of sum_{t in j} P_it, with P the dense       */
/* softmax and j a key block of kblk tokens.  items as above (query blocks   */
/* of blk tokens); mass [n_items, NBk].                                     */
/* ---------------------------------------------------------------------- */
void oracle_block_mass(const float *q, const float *k, int B, int H, int N, int N_pad, int D, int blk,
                       int kblk, double scale, const int32_t *items, int n_items, double *mass)
{
    int NB = oracle_n_blocks(N, kblk);
    (void)B;
#pragma omp parallel for schedule(dynamic)
    for (int it = 0; it < n_items; ++it) {
        int b = items[3 * it], h = items[3 * it + 1], qb = items[3 * it + 2];
        double *logit = (double *)malloc(sizeof(double) * (size_t)N);
        double *m = mass + (long)it * NB;
        int nq = rows_in_block(N, blk, qb);
        for (int j = 0; j < NB; ++j) m[j] = 0.0;
        for (int r = 0; r < nq; ++r) {
            const float *qi = row_ptr(q, H, N_pad, D, b, h, (long)qb * blk + r);
            double mx = -INFINITY, z = 0.0;
            for (int t = 0; t < N; ++t) {
                const float *kt = row_ptr(k, H, N_pad, D, b, h, t);
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += (double)qi[d] * (double)kt[d];
                logit[t] = scale * dot;
                if (logit[t] > mx) mx = logit[t];
            }
            for (int t = 0; t < N; ++t) z += exp(logit[t] - mx);
            for (int t = 0; t < N; ++t) m[t / kblk] += exp(logit[t] - mx) / z / (double)nq;
        }
        free(logit);
    }
}

/* Largest possible attention mass kept by K blocks: the sum of the K       */
/* largest entries of one mass row (ideal top-k, same section as above).    */
double oracle_topk_mass(const double *mass_row, int NB, int K)
{
    char *taken = (char *)calloc((size_t)NB, 1);
    double total = 0.0;
    for (int r = 0; r < K && r < NB; ++r) {
        int best = -1;
        for (int j = 0; j < NB; ++j)
            if (!taken[j] && (best < 0 || mass_row[j] > mass_row[best])) best = j;
        taken[best] = 1;
        total += mass_row[best];
    }
    free(taken);
    return total;
}
