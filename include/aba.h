/*
 * aba.h -- C ABI of the MI355X (gfx950) AB-Attention sparse attention layer.
 *
 * The layer is the attention of a video diffusion transformer made sparse as
 * the AB-Attention page ("AB-Attention ускорил генерацию видео до 2,23× и
 * пропускает 92% внимания", Hamidun News) describes it in its section
 * "Три приёма AB-Attention":
 *
 *   IBCS  -- each 128-query block is clustered into 8 centroids weighted by
 *            cluster share; every key block is scored by the weighted attention
 *            of those centroids to the block's averaged keys      (aba_score)
 *   SIP   -- key blocks are sampled with probability proportional to score, the
 *            most important always kept, and each kept block is weighted by its
 *            inverse inclusion probability                        (aba_sample)
 *   kernel-- the kept blocks are computed as ordinary softmax attention with
 *            shifted logits, in the original token order, with no permutation
 *            of tokens and no extra copies                        (aba_attend)
 *
 * and the full attention the page measures quality against ("Как мерили и что
 * вышло")                                                         (aba_attend_full).
 *
 * Conventions for every entry point
 *   - Tensors are device memory owned by the caller; the library allocates,
 *     frees and synchronizes nothing.  q, k, v and out are [B, H, N_pad, D]
 *     row-major (D fastest), N_pad = 128 * ceil(N / 128); token order is the
 *     caller's (frame-major for a video latent grid) and is never permuted.
 *   - Element type of q/k/v/out is the plan's dtype: ABA_BF16 (raw bfloat16
 *     bits) or ABA_F32.  Scores, centroids, weights and pooled keys are float32.
 *   - Rows >= N of q/k/v are ignored (they may hold anything); rows >= N of
 *     out are written as 0.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream) and may be issued from several host threads.
 *   - Errors: arguments are validated before anything is launched; on a bad
 *     argument the call returns ABA_E_INVALID or ABA_E_UNSUPPORTED and launches
 *     nothing.  A failed launch returns ABA_E_HIP.  aba_last_error() gives a
 *     message for the calling thread's last failure.  Device faults surface at
 *     the caller's next synchronization.
 */
#ifndef ABA_H
#define ABA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t; /* same declaration as HIP's own */

typedef enum aba_status {
    ABA_OK = 0,
    ABA_E_INVALID = 1,     /* malformed argument (null pointer, bad size, budget < 1, ...) */
    ABA_E_UNSUPPORTED = 2, /* well-formed but outside what the kernels implement */
    ABA_E_HIP = 3          /* a HIP launch or runtime call failed */
} aba_status;

typedef enum aba_dtype { ABA_F32 = 0, ABA_BF16 = 1 } aba_dtype;

/* Query block size: the page splits queries into 128-token blocks (IBCS
 * paragraph).  Key blocks are either the same 128 tokens or, as in the page's
 * kernel paragraph, 4 tokens: the unit of selection is then smaller than the
 * compute tile, and the kept 4-token blocks are gathered by index into full
 * 128-key matrix-core tiles. */
#define ABA_BLOCK 128
#define ABA_FINE_BLOCK 4
/* Largest number of query blocks per sequence (N <= 131072 tokens), and of
 * 4-token key blocks. */
#define ABA_MAX_BLOCKS 1024
#define ABA_MAX_KEY_BLOCKS 32768
/* Largest number of clusters per query block (the page uses 8). */
#define ABA_MAX_CLUSTERS 8

/* A plan is plain data filled by aba_plan and owned by the caller; it has no
 * destroy call and may be copied freely. */
typedef struct aba_plan {
    int32_t batch;          /* B */
    int32_t heads;          /* H */
    int32_t seq_len;        /* N, valid tokens */
    int32_t head_dim;       /* D: 64 or 128 (ABA_F32: 64) */
    int32_t block;          /* ABA_BLOCK: tokens per query block */
    int32_t n_blocks;       /* NB = ceil(N / 128) query blocks */
    int32_t seq_pad;        /* N_pad = 128 * NB */
    int32_t n_clusters;     /* C, 1..8 (the page: 8) */
    int32_t kmeans_iters;   /* T, Lloyd rounds (0..64) */
    int32_t budget;         /* K >= 1: expected kept key blocks per query block */
    int32_t list_cap;       /* capacity of one sampled list = NBk */
    int32_t dtype;          /* aba_dtype of q, k, v, out */
    float softmax_scale;    /* s, 1/sqrt(D) unless given */
    int32_t key_block;      /* tokens per key block: ABA_BLOCK or ABA_FINE_BLOCK */
    int32_t n_key_blocks;   /* NBk = ceil(N / key_block) */
    int32_t reserved;
    uint64_t workspace_bytes; /* device scratch for aba_score, aba_sample, aba_attend
                                 and aba_attend_full;
                                 every call uses it from offset 0 and only while it
                                 runs, so one buffer serves all calls ordered on a
                                 stream (calls that overlap in time need their own) */
} aba_plan_t;

/* Fill *p for a layer of `batch` x `heads` sequences of `seq_len` valid tokens,
 * selecting key blocks of `key_block` tokens (ABA_BLOCK or ABA_FINE_BLOCK) with
 * an expected `budget` of them per query block (at equal attention work, a
 * 4-token budget is 32 times the 128-token one).  softmax_scale <= 0 selects
 * 1/sqrt(head_dim).  Host-only; launches nothing.
 * Returns ABA_E_INVALID for non-positive sizes, budget < 1, a key_block other
 * than 128 or 4, or a null p, and ABA_E_UNSUPPORTED for a head_dim/dtype pair
 * without kernels (4-token key blocks: bf16 with head_dim 128, or fp32 with
 * 64), more than ABA_MAX_BLOCKS query blocks, more than ABA_MAX_CLUSTERS
 * clusters, or a 4-token budget whose sorted top exceeds the LDS of a CU
 * (8 * 2^ceil(log2 K) bytes > 155648, when 1024 < NBk and K < NBk). */
aba_status aba_plan(aba_plan_t *p, int32_t batch, int32_t heads, int32_t seq_len, int32_t head_dim,
                    aba_dtype dtype, int32_t n_clusters, int32_t kmeans_iters, int32_t budget, int32_t key_block,
                    float softmax_scale);

/* IBCS block scores (IBCS paragraph): for every (b, h, query block) cluster the
 * block's valid queries into C centroids with Lloyd k-means (strided initial
 * centroids q[floor(m*n/C)], T rounds of assign + update, ties to the lowest
 * index, an empty cluster keeps its centroid), weight each centroid by its
 * share of the block's queries, mean-pool every key block (of the plan's
 * key_block tokens) over its valid keys, and score key block j by
 *     S[j] = sum_m w_m softmax_j(s * c_m . kbar_j).
 * Each row of scores sums to one.
 *   q, k       : [B,H,N_pad,D] in the plan's dtype
 *   scores     : out, float32 [B,H,NB,NBk]
 *   centroids  : out, nullable, float32 [B,H,NB,C,D]
 *   cluster_w  : out, nullable, float32 [B,H,NB,C]
 *   pooled_k   : out, nullable, float32 [B,H,NBk,D]
 *   workspace  : at least p->workspace_bytes of device memory (required: the
 *                two scoring passes keep per-chunk softmax statistics there) */
aba_status aba_score(const aba_plan_t *p, const void *q, const void *k, float *scores, float *centroids,
                     float *cluster_w, float *pooled_k, void *workspace, hipStream_t stream);

/* SIP sampling plan (SIP paragraph).  Per (b, h, query block) row of scores:
 *   sigma_j = clamp(floor(S_j * 2^32), 1, 2^32) (NaN or <= 0 -> 1);
 *   order blocks by (sigma desc, index asc); the first is always kept; more
 *   blocks are capped at probability 1 while (K - t) * sigma_(t+1) >= R, with R
 *   the sum of sigma over the blocks not yet capped (water-filling);
 *   capped: theta = 2^32; other blocks theta = clamp(ceil((K-t) sigma 2^32 / R),
 *   1, 2^32) (1 when K - t <= 0), so P(kept) = theta / 2^32 sums to K;
 *   the draw for key block j is word (j & 3) of Philox4x32-10 (Salmon et al.,
 *   SC'11) with key (seed_lo, seed_hi) and counter (j >> 2, query block,
 *   head_offset + h, batch_offset + b);
 *   block j is kept iff draw < theta_j, with weight w = float(2^32 / theta_j)
 *   (an fp64 division), the Horvitz-Thompson factor 1/pi.
 *   scores       : float32 [B,H,NB,NBk]
 *   head_offset  : global index of head 0 of this call (>= 0): a call over
 *                  heads h0 .. h0+H-1 of a larger layer passes h0
 *   batch_offset : global index of batch entry 0 of this call (>= 0)
 *   idx    : out, int32 [B,H,NB,list_cap], kept key blocks in ascending order
 *   cnt    : out, int32 [B,H,NB], number kept (>= 1)
 *   w      : out, float32 [B,H,NB,list_cap], weights of the listed blocks
 *   workspace : at least p->workspace_bytes of device memory; required when
 *               rows hold more than 8192 key blocks (4-token key blocks beyond
 *               32768 tokens) and the budget is below the row length: those
 *               rows are split into chunks whose totals, tops and counts it
 *               keeps.  May be NULL otherwise.
 * Entries at or past cnt are left unspecified.  The lists depend only on
 * (scores, budget, seed) and the global (batch, head) indices: every draw is
 * addressable by (seed, b, h, query block, key block), so a call over a slice
 * of heads draws exactly what a call over the whole layer draws for them.
 * Offsets with head_offset + H or batch_offset + B above 2^31 - 1 ->
 * ABA_E_INVALID. */
aba_status aba_sample(const aba_plan_t *p, const float *scores, uint64_t seed, int32_t head_offset,
                      int32_t batch_offset, int32_t *idx, int32_t *cnt, float *w, void *workspace,
                      hipStream_t stream);

/* Block-sparse attention over a sampling plan (SIP and kernel paragraphs).  For
 * each valid query i of query block b, with the kept list (j, w_j) of key
 * blocks of the plan's key_block tokens:
 *     o_i = sum_j w_j sum_{t in j} e^{s q_i.k_t} v_t / sum_j w_j sum_{t in j} e^{s q_i.k_t}
 * i.e. softmax attention with the logits of block j shifted by ln w_j; keys
 * >= N are masked.  List entries outside [0, NBk) or with a weight that is not
 * positive and finite are skipped; cnt is clamped to [0, list_cap]; a query
 * block with nothing to attend gets zeros.
 *   q, k, v   : [B,H,N_pad,D];  idx, cnt, w : as produced by aba_sample
 *   out       : out, [B,H,N_pad,D] in the plan's dtype
 *   workspace : at least p->workspace_bytes of device memory; required for
 *               ABA_BF16 (it holds the work order, and at head_dim 64 a
 *               transposed copy of v), may be NULL for ABA_F32.  NULL where
 *               required -> ABA_E_INVALID. */
aba_status aba_attend(const aba_plan_t *p, const void *q, const void *k, const void *v, const int32_t *idx,
                      const int32_t *cnt, const float *w, void *out, void *workspace, hipStream_t stream);

/* Dense softmax attention softmax(s q k^T) v over all valid keys, non-causal
 * (the full-attention reference of "Как мерили и что вышло").  Same layout,
 * workspace rule and output convention as aba_attend; the key block size of
 * the plan does not matter here. */
aba_status aba_attend_full(const aba_plan_t *p, const void *q, const void *k, const void *v, void *out,
                           void *workspace, hipStream_t stream);

/* aba_attend without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments (minus workspace), kernels and
 * results as aba_attend.  The work order lives in a static device array of the
 * library (1 MiB, i.e. at most 262144 = B * H * NB query blocks), one per GPU,
 * held until the process ends; it needs no clearing between calls.  Every call
 * on a GPU shares that GPU's array: calls that overlap in time on one GPU race
 * and must be ordered by the caller (one stream, or events).  Allocates
 * nothing.  Returns ABA_E_UNSUPPORTED for more query blocks than the array
 * holds, and for bf16 at head_dim 64 (which stages a transposed copy of v). */
aba_status aba_attend_noalloc(const aba_plan_t *p, const void *q, const void *k, const void *v, const int32_t *idx,
                              const int32_t *cnt, const float *w, void *out, hipStream_t stream);

/* Dense attention mass per key block (of the plan's key_block tokens), for
 * judging a block selection (IBCS paragraph and the opening of "Три приёма
 * AB-Attention": the share of the attention a selection keeps).  For each
 * listed query block b' with n valid query rows:
 *     mass[item][j] = (1/n) sum_i sum_{t in key block j, t < N} softmax_t(s q_i . k_t)
 * so each row sums to one; its K largest entries sum to the ideal top-K mass.
 * ABA_BF16 only (ABA_E_UNSUPPORTED otherwise).  A diagnostic, off the attention
 * path: it costs two dense QK^T passes per listed query block.
 *   q, k    : [B,H,N_pad,D]
 *   items   : device int32 [n_items][3] of (b, h, query block); an item outside
 *             the layer yields a row of zeros
 *   n_items : >= 0 (0 launches nothing)
 *   mass    : out, device float32 [n_items][NBk] */
aba_status aba_block_mass(const aba_plan_t *p, const void *q, const void *k, const int32_t *items, int32_t n_items,
                          float *mass, hipStream_t stream);

/* Measurement support, not a step of the layer: a loop of bf16 matrix-core
 * products with register operands and no memory traffic, on every compute unit
 * (512 workgroups of 256 threads: two wavefronts per SIMD, the occupancy of the
 * attention kernels).  Each wavefront runs iters x 16 v_mfma_f32_32x32x16_bf16,
 * so one call performs iters x 2^30 floating-point operations (512 x 4 x 16 x
 * 32768 per round).  Timed by the caller on `stream`, it gives the rate the
 * matrix cores sustain: with random != 0 on operands with random bits (the
 * power drawn, hence the shader clock the chip holds, depends on operand
 * toggling), with random == 0 on zeros.  The bf16 peak of 2.5 PFLOP/s is quoted
 * at a 2.4 GHz clock; a kernel's measured rate can be set against both.
 *   iters : 1 .. 10^6 (else ABA_E_INVALID)
 *   out   : device float32 [512 * 256], a checksum per thread (keeps the
 *           products from being discarded); contents are not meaningful */
aba_status aba_mfma_rate(int32_t iters, int32_t random, float *out, hipStream_t stream);

/* Message for the calling thread's last non-OK status ("" if none).  The
 * pointer stays valid until the thread's next aba_* call. */
const char *aba_last_error(void);

/* Library version string. */
const char *aba_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ABA_H */
