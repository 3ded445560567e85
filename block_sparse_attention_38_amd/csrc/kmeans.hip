// kmeans.hip -- IBCS intra-block clustering (gfx950).
//
// AB-Attention page, section "Три приёма AB-Attention", IBCS paragraph: the
// queries of every 128-token block are grouped into 8 clusters, each with a
// centroid and a weight equal to the cluster's share of the block's queries.
//
// One workgroup (256 threads) per (b, h, query block); the block's valid query
// rows stay in LDS for all rounds, so q is read from HBM exactly once.
// Lloyd k-means with strided initial centroids x[floor(m*n/C)], T rounds of
// (assign, update), ties to the lowest cluster index, empty clusters keeping
// their centroid; the weights come from the last assignment.
//
// Assignment uses |x - c|^2 = |x|^2 - 2 x.c + |c|^2 without the |x|^2 term
// (it does not change the argmin): thread (i, half) scores its row against
// half of the centroids, and the two halves are merged through LDS.
#include "aba_internal.h"

namespace aba {
namespace {

// Rows are kept in LDS in their input type, padded by one 16-byte chunk so that
// lanes on consecutive rows start on different banks.
template <typename T, int D> constexpr int row_stride() { return D + 16 / (int)sizeof(T); }

__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T, int D>
__global__ __launch_bounds__(256) void kmeans_kernel(const T *__restrict__ q, int N, int N_pad, int NB, int C, int T_iters,
                                                     float *__restrict__ cent_out, float *__restrict__ w_out)
{
    constexpr int kStride = row_stride<T, D>();
    constexpr int kGroups = 256 / D;                      // update step: cluster groups per dimension
    constexpr int kPerGroup = (kMaxClusters + kGroups - 1) / kGroups;
    __shared__ __align__(16) T xs[kBlock * kStride];
    __shared__ __align__(16) float cs[kMaxClusters][D];
    __shared__ float cnorm[kMaxClusters];
    __shared__ float cand_d[2][kBlock];
    __shared__ int cand_m[2][kBlock];
    __shared__ int asg[kBlock];
    __shared__ int count[kMaxClusters];

    const int row = blockIdx.x;                           // (b*H + h) * NB + query block
    const int qb = row % NB;
    const long bh = row / NB;
    const int n = min(kBlock, N - qb * kBlock);
    const int tid = threadIdx.x;
    const T *src = q + (bh * N_pad + (long)qb * kBlock) * D;

    // stage the block's valid rows in LDS (16-byte chunks)
    constexpr int kElemsPerChunk = 16 / sizeof(T);
    constexpr int kChunksPerRow = D / kElemsPerChunk;
    for (int i = tid; i < n * kChunksPerRow; i += 256) {
        const int r = i / kChunksPerRow, c = i % kChunksPerRow;
        *reinterpret_cast<uint4 *>(&xs[r * kStride + c * kElemsPerChunk]) =
            *reinterpret_cast<const uint4 *>(src + (long)r * D + c * kElemsPerChunk);
    }
    __syncthreads();

    // strided initial centroids
    for (int i = tid; i < C * D; i += 256) {
        const int m = i / D, d = i % D;
        const int r = (int)((long)m * n / C);
        cs[m][d] = to_f32(xs[r * kStride + d]);
    }

    const int rows_assign = tid & (kBlock - 1), half = tid >> 7;
    const int m_lo = half * ((C + 1) / 2), m_hi = min(C, m_lo + (C + 1) / 2);
    const int d_upd = tid % D, g_upd = tid / D;
    const int mu_lo = g_upd * kPerGroup, mu_hi = min(C, mu_lo + kPerGroup);

    const int rounds = T_iters > 0 ? T_iters : 1;
    for (int it = 0; it < rounds; ++it) {
        __syncthreads();
        if (tid < C) {
            float s = 0.f;
            for (int d = 0; d < D; ++d) s = fmaf(cs[tid][d], cs[tid][d], s);
            cnorm[tid] = s;
        }
        __syncthreads();

        // assignment: row i against clusters [m_lo, m_hi)
        const int i = rows_assign;
        if (i < n) {
            float dots[(kMaxClusters + 1) / 2];
#pragma unroll
            for (int mm = 0; mm < (kMaxClusters + 1) / 2; ++mm) dots[mm] = 0.f;
            for (int d0 = 0; d0 < D; d0 += 8) {
                float x[8];
                load8(&xs[i * kStride + d0], x);
#pragma unroll
                for (int mm = 0; mm < (kMaxClusters + 1) / 2; ++mm) {
                    const int m = m_lo + mm;
                    if (m < m_hi) {
                        const float4 c0 = *reinterpret_cast<const float4 *>(&cs[m][d0]);
                        const float4 c1 = *reinterpret_cast<const float4 *>(&cs[m][d0 + 4]);
                        float a = dots[mm];
                        a = fmaf(x[0], c0.x, a); a = fmaf(x[1], c0.y, a);
                        a = fmaf(x[2], c0.z, a); a = fmaf(x[3], c0.w, a);
                        a = fmaf(x[4], c1.x, a); a = fmaf(x[5], c1.y, a);
                        a = fmaf(x[6], c1.z, a); a = fmaf(x[7], c1.w, a);
                        dots[mm] = a;
                    }
                }
            }
            float best = INFINITY;
            int bm = m_lo;
#pragma unroll
            for (int mm = 0; mm < (kMaxClusters + 1) / 2; ++mm) {
                const int m = m_lo + mm;
                if (m < m_hi) {
                    const float dist = fmaf(-2.f, dots[mm], cnorm[m]);
                    if (dist < best) {
                        best = dist;
                        bm = m;
                    }
                }
            }
            cand_d[half][i] = best;
            cand_m[half][i] = bm;
        }
        __syncthreads();
        if (tid < n) {
            // strict comparison: on a tie the lower half (lower cluster index) wins
            asg[tid] = (cand_d[1][tid] < cand_d[0][tid]) ? cand_m[1][tid] : cand_m[0][tid];
        }
        __syncthreads();
        if (tid < C) {
            int c = 0;
            for (int r = 0; r < n; ++r) c += (asg[r] == tid);
            count[tid] = c;
        }
        if (T_iters == 0) break;   // weights of the initial centroids only

        // update: thread (d, group) sums dimension d of its clusters' rows
        float acc[kPerGroup];
#pragma unroll
        for (int mm = 0; mm < kPerGroup; ++mm) acc[mm] = 0.f;
        for (int r = 0; r < n; ++r) {
            const int a = asg[r] - mu_lo;
            const float x = to_f32(xs[r * kStride + d_upd]);
#pragma unroll
            for (int mm = 0; mm < kPerGroup; ++mm)
                if (a == mm) acc[mm] += x;
        }
        __syncthreads();
#pragma unroll
        for (int mm = 0; mm < kPerGroup; ++mm) {
            const int m = mu_lo + mm;
            if (m < mu_hi && count[m] > 0) cs[m][d_upd] = acc[mm] / (float)count[m];
        }
    }
    __syncthreads();

    float *co = cent_out + (long)row * C * D;
    for (int i2 = tid; i2 < C * D; i2 += 256) co[i2] = cs[i2 / D][i2 % D];
    if (tid < C) w_out[(long)row * C + tid] = (float)((double)count[tid] / (double)n);
}

// ---------------------------------------------------------------------------
// bf16 inputs: both halves of a Lloyd round are small contractions and run on
// bf16 MFMA (32x32x16).
//   assignment  dots^T = C_split X^T.  Query rows are exact in bf16; every fp32
//               centroid c is split into three bf16 parts hi + mid + lo (each
//               the rounding of the remainder of the previous ones), which
//               carry its 24-bit mantissa, so each product is exact and the
//               dot product has fp32 accuracy.  Accumulator rows are 8p + m
//               (part p of cluster m), so a lane holds all three parts of four
//               clusters for its query and adds them locally; the argmin needs
//               one exchange between the two lane halves.
//   update      sums = onehot^T X with X^T staged once per block in LDS; new
//               centroids are sums / counts.  The assignment writes, once per
//               round, a membership flag byte per (cluster, query) and each
//               wavefront's cluster counts (ballots) to LDS; the update turns
//               eight flags into its one-hot operand with two shifts and four
//               byte permutes; the lanes that form a centroid element also
//               write its three bf16 parts and its share of |c|^2, so a round
//               has two barriers.
// A round whose assignment equals the previous round's leaves every later
// round unchanged bit for bit (same rows, same sums), so the loop stops there:
// the result is exactly that of all T rounds.
// One workgroup of 4 wavefronts per (b, h, query block); wavefront w owns
// queries [32w, 32w + 32) in the assignment and dims [32w, 32w + 32) in the
// update.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x)
{
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Eight bf16 values from the flags of eight bytes (f0: elements 0..3, f1: 4..7):
// 4.0 (0x4080: low byte 0x80, high byte 0x40) for a set flag, else 0.  Byte
// permutes interleave each flag byte (0x80 / 0) with itself shifted right by one
// (0x40 / 0).
__device__ __forceinline__ uint4 onehot4(uint32_t f0, uint32_t f1)
{
    const uint32_t g0 = f0 >> 1, g1 = f1 >> 1;
    // selector bytes 0..3 pick bytes of the second operand, 4..7 of the first
    return make_uint4(__builtin_amdgcn_perm(g0, f0, 0x05010400u), __builtin_amdgcn_perm(g0, f0, 0x07030602u),
                      __builtin_amdgcn_perm(g1, f1, 0x05010400u), __builtin_amdgcn_perm(g1, f1, 0x07030602u));
}

// The same workgroup also pools the keys of its 128 tokens (IBCS paragraph:
// a key block is represented by its averaged keys): one 128-token key block
// (kb = 128) or 32 4-token ones (kb = 4), into kbar [B, H, NBk, D].  It does so
// first: the key loads are issued ahead of the query loads, so their latency
// overlaps the query staging, and the separate pooling pass over k disappears.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void kmeans_mfma_kernel(const uint16_t *__restrict__ q, int N, int N_pad, int NB,
                                                          int C, int T_iters, float *__restrict__ cent_out,
                                                          float *__restrict__ w_out, const uint16_t *__restrict__ k,
                                                          int kb, int NBk, float *__restrict__ kbar)
{
    constexpr int KS = D / 16;          // k-steps over the head dimension
    constexpr int DCH = D / 8;          // 16-byte chunks per row of D bf16
    // X^T: row d holds 128 queries (16 chunks of 8), chunk c stored at c ^ xt_swz(d): 16
    // consecutive rows (the update's reads) and the rows 8c + j of the 16 chunks c of
    // one transposing write both land on 16 different chunks, so neither conflicts
    __shared__ uint4 xt_s[D * 16];
    auto xt_swz = [](int d) __attribute__((always_inline)) { return (d & 15) ^ ((d >> 4) & 7); };
    // split centroids: row 8p + m holds part p of cluster m (chunk swizzle c ^
    // (row & (DCH - 1))); the three parts sum exactly to the fp32 centroid, so
    // no separate fp32 copy is kept (that keeps the block under 40 KB of LDS:
    // four workgroups per CU)
    __shared__ uint4 cs_s[24 * DCH];
    __shared__ float cn_part[4][kMaxClusters];   // per-wavefront shares of |c_m|^2
    // membership flags written by the assignment: byte q of row m is 0x80 when
    // query q is in cluster m, else 0 (rows padded to 136 bytes: the eight rows
    // an update operand read touches start on different banks); and the
    // per-wavefront cluster counts of the last assignment
    constexpr int kFlagPitch = kBlock + 8;
    __shared__ __align__(16) uint8_t flag_s[kMaxClusters * kFlagPitch];
    __shared__ int cnt_s[4][kMaxClusters];

    const int row = blockIdx.x;                           // (b*H + h) * NB + query block
    const int qb = row % NB;
    const long bh = row / NB;
    const int n = min(kBlock, N - qb * kBlock);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, half = lane >> 5;
    const uint16_t *src = q + (bh * N_pad + (long)qb * kBlock) * D;

    // ---- key pooling of this block's 128 tokens (n valid), first: the key
    // loads are issued before the query loads, so their latency overlaps the
    // query staging below instead of trailing the rounds
    const uint16_t *ksrc = k + (bh * N_pad + (long)qb * kBlock) * D;
    constexpr int G = 256 / DCH;           // 128-token key block: thread (group g, chunk c)
    constexpr int RPT = kBlock / G;        // sums rows g, g + G, .. (loads issued before the sums)
    constexpr int kFine = kBlock / kFineBlock;
    constexpr int IPT = kFine * DCH / 256; // 4-token key blocks: (block, chunk) items per thread
    static_assert(kFine * DCH % 256 == 0, "whole items per thread");
    static_assert(RPT == IPT * kFineBlock, "the same number of row loads in both cases");
    uint4 kraw[RPT];
    if (kb == kBlock) {
        const int c = tid % DCH, g = tid / DCH;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = g + G * i;
            kraw[i] = r < n ? *reinterpret_cast<const uint4 *>(ksrc + (long)r * D + 8 * c) : make_uint4(0, 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int i = tid + 256 * it, g = i / DCH, c = i % DCH;
            const int j = qb * kFine + g;
#pragma unroll
            for (int r = 0; r < kFineBlock; ++r)
                kraw[it * kFineBlock + r] =
                    (j < NBk && kFineBlock * j + r < N)
                        ? *reinterpret_cast<const uint4 *>(ksrc + (long)(kFineBlock * g + r) * D + 8 * c)
                        : make_uint4(0, 0, 0, 0);
        }
    }

    // this wavefront's 32 queries as B fragments of the assignment product
    const int my_q = wave * 32 + l32;
    const bool qv = my_q < n;
    bf16x8 xf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (qv) raw = *reinterpret_cast<const uint4 *>(src + (long)my_q * D + 16 * ks + 8 * half);
        xf[ks] = __builtin_bit_cast(bf16x8, raw);
    }

    // sum the keys (the query loads above stay in flight)
    if (kb == kBlock) {
        const int g = tid / DCH;
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            if (g + G * i >= n) break;
            const uint32_t w4[4] = {kraw[i].x, kraw[i].y, kraw[i].z, kraw[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += bf16_lo(w4[e]);
                acc[2 * e + 1] += bf16_hi(w4[e]);
            }
        }
        // the groups g of one wavefront (lanes c + DCH j) add up by shuffles, the
        // four wavefronts' sums through LDS (the X^T space, written only below)
#pragma unroll
        for (int o = DCH; o < 64; o <<= 1)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
        float *part = reinterpret_cast<float *>(xt_s);
        if (lane < DCH) {
#pragma unroll
            for (int e = 0; e < 8; ++e) part[wave * D + 8 * lane + e] = acc[e];
        }
        __syncthreads();
        if (tid < D)
            kbar[((long)bh * NBk + qb) * D + tid] =
                (((part[tid] + part[D + tid]) + part[2 * D + tid]) + part[3 * D + tid]) / (float)n;
        __syncthreads();   // the X^T writes below reuse the space
    } else {
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int i = tid + 256 * it, g = i / DCH, c = i % DCH;
            const int j = qb * kFine + g;
            if (j >= NBk) continue;
            const int nr = min(kFineBlock, N - kFineBlock * j);
            float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int r = 0; r < kFineBlock; ++r) {
                if (r >= nr) break;
                const uint4 x = kraw[it * kFineBlock + r];
                const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] += bf16_lo(w4[e]);
                    acc[2 * e + 1] += bf16_hi(w4[e]);
                }
            }
            const float fn = (float)nr;
            float4 *dst = reinterpret_cast<float4 *>(kbar + ((long)bh * NBk + j) * D + 8 * c);
            dst[0] = make_float4(acc[0] / fn, acc[1] / fn, acc[2] / fn, acc[3] / fn);
            dst[1] = make_float4(acc[4] / fn, acc[5] / fn, acc[6] / fn, acc[7] / fn);
        }
    }

    // X^T into LDS: thread (c, quad) moves queries 4quad..4quad+3 of dims 8c..8c+7
    uint2 *xt2 = reinterpret_cast<uint2 *>(xt_s);
#pragma unroll
    for (int pass = 0; pass < DCH / 8; ++pass) {
        const int c = tid % DCH, quad = tid / DCH + pass * (256 / DCH);
        uint4 rows[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int qq = 4 * quad + rr;
            rows[rr] = make_uint4(0, 0, 0, 0);
            if (qq < n) rows[rr] = *reinterpret_cast<const uint4 *>(src + (long)qq * D + 8 * c);
        }
        const uint32_t *r0 = reinterpret_cast<const uint32_t *>(&rows[0]);
        const uint32_t *r1 = reinterpret_cast<const uint32_t *>(&rows[1]);
        const uint32_t *r2 = reinterpret_cast<const uint32_t *>(&rows[2]);
        const uint32_t *r3 = reinterpret_cast<const uint32_t *>(&rows[3]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) {
                const int d = 8 * c + 2 * p + hl;
                const uint32_t a = hl ? ((r0[p] >> 16) | (r1[p] & 0xFFFF0000u)) : ((r0[p] & 0xFFFFu) | (r1[p] << 16));
                const uint32_t b = hl ? ((r2[p] >> 16) | (r3[p] & 0xFFFF0000u)) : ((r2[p] & 0xFFFFu) | (r3[p] << 16));
                xt2[d * 32 + (((quad >> 1) ^ xt_swz(d)) << 1) + (quad & 1)] = make_uint2(a, b);
            }
        }
    }

    // strided initial centroids q[floor(m n / C)]: bf16 values, so the high
    // part is the row itself and the other two are zero; clusters >= C stay
    // zero and are never chosen.  Threads (m, chunk) also form |c_m|^2.
    if (tid < kMaxClusters * DCH) {
        const int m = tid / DCH, c = tid % DCH;
        uint4 hi = make_uint4(0, 0, 0, 0);
        if (m < C) hi = *reinterpret_cast<const uint4 *>(src + (long)(m * n / C) * D + 8 * c);
        const uint32_t *h = reinterpret_cast<const uint32_t *>(&hi);
        float nrm = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x0 = bf16_lo(h[e]), x1 = bf16_hi(h[e]);
            nrm = fmaf(x0, x0, nrm);
            nrm = fmaf(x1, x1, nrm);
        }
#pragma unroll
        for (int pp = 0; pp < 3; ++pp) {
            const int r = 8 * pp + m;
            cs_s[r * DCH + (c ^ (r & (DCH - 1)))] = pp == 0 ? hi : make_uint4(0, 0, 0, 0);
        }
        // reduce |c_m|^2 over the DCH consecutive lanes of cluster m
#pragma unroll
        for (int o = 1; o < DCH; o <<= 1) nrm += __shfl_xor(nrm, o, 64);
        if (c == 0) {
            cn_part[0][m] = nrm;
            cn_part[1][m] = cn_part[2][m] = cn_part[3][m] = 0.f;
        }
    }
    __syncthreads();
    uint16_t *cs16 = reinterpret_cast<uint16_t *>(cs_s);
    // element d of cluster m's part p, and the fp32 centroid element (exact sum of the parts)
    auto part_at = [&](int p, int m, int d) __attribute__((always_inline)) -> uint16_t & {
        const int rr = 8 * p + m;
        return cs16[(rr * DCH + ((d >> 3) ^ (rr & (DCH - 1)))) * 8 + (d & 7)];
    };
    auto centroid = [&](int m, int d) __attribute__((always_inline)) {
        return (bf16_bits_to_f32(part_at(0, m, d)) + bf16_bits_to_f32(part_at(1, m, d))) +
               bf16_bits_to_f32(part_at(2, m, d));
    };

    const int rounds = T_iters > 0 ? T_iters : 1;
    int prev = -1;
    for (int it = 0; it < rounds; ++it) {
        // ---- assignment: dots^T = C_split X^T for this wavefront's 32 queries
        floatx16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            // rows 24..31 of the A operand only feed accumulator rows that are
            // never read: any stored row serves
            const int ar = l32 < 24 ? l32 : l32 - 8;
            const uint4 a = cs_s[ar * DCH + ((2 * ks + half) ^ (ar & (DCH - 1)))];
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), xf[ks], acc, 0, 0, 0);
        }
        // lane half h holds clusters 4h .. 4h+3: accumulator row 8p + m is r = 4p + (m & 3)
        float bd = INFINITY;
        int bm = 4 * half;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = 4 * half + j;
            const float dot = acc[j] + acc[4 + j] + acc[8 + j];
            const float cn2 = cn_part[0][m] + cn_part[1][m] + cn_part[2][m] + cn_part[3][m];
            const float dist = m < C ? fmaf(-2.f, dot, cn2) : INFINITY;
            if (dist < bd) {
                bd = dist;
                bm = m;
            }
        }
        const float od = __shfl_xor(bd, 32, 64);
        const int om = __shfl_xor(bm, 32, 64);
        if (od < bd || (od == bd && om < bm)) {
            bd = od;
            bm = om;
        }
        // lane half h writes the flags of its query in rows 4h .. 4h+3
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = 4 * half + j;
            flag_s[m * kFlagPitch + my_q] = (qv && bm == m) ? (uint8_t)0x80 : (uint8_t)0;
        }
#pragma unroll
        for (int m = 0; m < kMaxClusters; ++m) {
            const int c = __popcll(__ballot(half == 0 && qv && bm == m));
            if (lane == 0) cnt_s[wave][m] = c;
        }
        const int changed = (half == 0 && qv && bm != prev) ? 1 : 0;
        prev = bm;
        const int any_changed = __syncthreads_or(changed);
        if (T_iters == 0 || !any_changed) break;   // initial-centroid weights, or converged

        // ---- update: sums = onehot^T X, wavefront w owns dims [32w, 32w + 32)
        if (wave < D / 32) {
            floatx16 sum;
#pragma unroll
            for (int r = 0; r < 16; ++r) sum[r] = 0.f;
            const int d = wave * 32 + l32;
            // A operand row l32 is cluster l32 % 8 (rows >= 8 only feed accumulator
            // rows that are never read); its entries are 4.0 (bf16 0x4080) for the
            // cluster's queries, so the sums are 4x the cluster sums, exactly
            const uint8_t *flag_row = flag_s + (l32 & 7) * kFlagPitch + 8 * half;
#pragma unroll
            for (int ks = 0; ks < kBlock / 16; ++ks) {
                const uint2 f = *reinterpret_cast<const uint2 *>(flag_row + 16 * ks);
                const uint4 oh = onehot4(f.x, f.y);
                const uint4 b = xt_s[d * 16 + ((2 * ks + half) ^ xt_swz(d))];
                sum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, oh),
                                                              __builtin_bit_cast(bf16x8, b), sum, 0, 0, 0);
            }
            // counts of clusters 4half .. 4half+3: the four wavefronts' shares
            const int4 c0 = *reinterpret_cast<const int4 *>(&cnt_s[0][4 * half]);
            const int4 c1 = *reinterpret_cast<const int4 *>(&cnt_s[1][4 * half]);
            const int4 c2 = *reinterpret_cast<const int4 *>(&cnt_s[2][4 * half]);
            const int4 c3 = *reinterpret_cast<const int4 *>(&cnt_s[3][4 * half]);
            const int cnts[4] = {c0.x + c1.x + c2.x + c3.x, c0.y + c1.y + c2.y + c3.y, c0.z + c1.z + c2.z + c3.z,
                                 c0.w + c1.w + c2.w + c3.w};
            // lane holds the sums of clusters 4half .. 4half+3 for dim d
            float sq[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * half + r;
                const int cn = cnts[r];
                float cv;
                if (m < C && cn > 0) {
                    // (4 sum) x approximate 1 / (4 n): within 2 ulp of the mean
                    cv = sum[r] * __builtin_amdgcn_rcpf((float)(4 * cn));
                    const uint16_t hb = f32_to_bf16_bits(cv);
                    const float r1 = cv - bf16_bits_to_f32(hb);
                    const uint16_t mb = f32_to_bf16_bits(r1);
                    const uint16_t lb = f32_to_bf16_bits(r1 - bf16_bits_to_f32(mb));
                    part_at(0, m, d) = hb;
                    part_at(1, m, d) = mb;
                    part_at(2, m, d) = lb;
                } else {
                    cv = centroid(m, d);   // an empty cluster keeps its centroid
                }
                sq[r] = cv * cv;
            }
            // this wavefront's share of |c_m|^2: sum over its 32 dims (lanes of one half)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
#pragma unroll
                for (int o = 1; o < 32; o <<= 1) sq[r] += __shfl_xor(sq[r], o, 64);
            }
            if (l32 == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r) cn_part[wave][4 * half + r] = sq[r];
            }
        }
        __syncthreads();
    }

    float *co = cent_out + (long)row * C * D;
    for (int i = tid; i < C * D; i += 256) co[i] = centroid(i / D, i % D);
    if (tid < C) {   // weights from the last assignment
        const int cn = cnt_s[0][tid] + cnt_s[1][tid] + cnt_s[2][tid] + cnt_s[3][tid];
        w_out[(long)row * C + tid] = (float)((double)cn / (double)n);
    }
}


// Sum of x over the 32 lanes of each wavefront half, in every lane: butterflies
// within quads (quad_perm), 8-lane (row_half_mirror) and 16-lane (row_mirror)
// groups by DPP, then the two rows of the half by v_permlane16_swap; no LDS.
__device__ __forceinline__ float half_sum32(float x)
{
#define ABA_DPP(v, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, true))
    x += ABA_DPP(x, 0xB1);    // quad_perm(1, 0, 3, 2)
    x += ABA_DPP(x, 0x4E);    // quad_perm(2, 3, 0, 1)
    x += ABA_DPP(x, 0x141);   // row_half_mirror
    x += ABA_DPP(x, 0x140);   // row_mirror
#undef ABA_DPP
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// bf16 at head_dim 128: the same rounds with the block's query rows kept in LDS
// row-major, as they arrive.  Direct buffer->LDS loads copy the 128 rows (no
// registers, no transposing pass, q read once); the assignment's B fragments
// are plain 16-byte LDS reads of those rows, and the update's X operand comes
// from transposing LDS reads (ds_read_b64_tr_b16), so the update's one-hot
// operand takes its queries in the order the transposing reads deliver them.
// The key rows for the pooling are loaded right after the queries and summed
// only after the rounds: their latency and bandwidth overlap the rounds, and no
// barrier inside the rounds waits for them (the barriers are bare s_barriers
// after an LDS wait; a workgroup fence would drain every load in flight).
// The arithmetic is that of kmeans_mfma_kernel; only the order in which the
// update's MFMA adds its (exact) products differs, so sums may differ in the
// last place.
// ---------------------------------------------------------------------------
template <int D, int KB>   // KB: tokens per key block of the pooling (128 or 4)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void kmeans_lds_kernel(
    const uint16_t *__restrict__ q, int N, int N_pad, int NB, int C, int T_iters, float *__restrict__ cent_out,
    float *__restrict__ w_out, const uint16_t *__restrict__ k, int NBk, float *__restrict__ kbar)
{
    static_assert(KB == kBlock || KB == kFineBlock, "128-token or 4-token key blocks");
    static_assert(D == 128, "a direct load of 1024 bytes fills 4 query rows of 256 bytes");
    constexpr int KS = D / 16;          // k-steps over the head dimension
    constexpr int DCH = D / 8;          // 16-byte chunks per row
    constexpr int kPitch = D * 2;       // bytes per query row in LDS
    // X: row r (query) holds its D bf16 values, chunk c stored at c ^ xswz(r) with
    // xswz(r) = 4 (r % 4) + (r / 4) % 4: the 16 rows of a 16-lane phase of the
    // assignment's 16-byte reads land on 16 different chunks, and so do the 4
    // rows x 4 chunks of a 32-lane phase of the update's transposing reads
    __shared__ __align__(16) char xs[kBlock * kPitch];
    __shared__ uint4 cs_s[24 * DCH];                  // split centroids, as in kmeans_mfma_kernel
    __shared__ __align__(16) float cn_part[4][kMaxClusters];
    constexpr int kFlagPitch = kBlock + 8;
    __shared__ __align__(16) uint8_t flag_s[kMaxClusters * kFlagPitch];
    __shared__ int cnt_s[4][kMaxClusters];
    __shared__ int chg_s[4];

    const int row = blockIdx.x;                           // (b*H + h) * NB + query block
    const int qb = row % NB;
    const long bh = row / NB;
    const int n = min(kBlock, N - qb * kBlock);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, half = lane >> 5;
    auto xrow = [&](int r) __attribute__((always_inline)) { return xs + r * kPitch; };
    auto xswz = [](int r) __attribute__((always_inline)) { return 4 * (r & 3) + ((r >> 2) & 3); };
    auto xchunk = [&](int r, int c) __attribute__((always_inline)) { return 16 * (c ^ xswz(r)); };

    // ---- the block's query rows into LDS: wavefront w copies rows 32w .. 32w+31,
    // four per load; the row offset rides in the range-checked per-lane offset,
    // so rows >= N (past the descriptor) arrive as zeros
    {
        const int4v rq = head_rsrc(q + bh * N_pad * D, N * D * 2);
        // load t fills LDS rows 32w + 4t .. +3: lane L row 32w + 4t + L / 16, chunk
        // position L % 16, which holds logical chunk (L % 16) ^ xswz(row)
        const int r4 = lane >> 4;
        const int voff = (qb * kBlock + 32 * wave + r4) * kPitch;
        char *dst = xrow(32 * wave);
#pragma unroll
        for (int t = 0; t < 8; ++t)
            load_lds16(rq, voff + 4 * t * kPitch + 16 * ((lane & 15) ^ (4 * r4 + (t & 3))), 0, dst + 1024 * t);
    }
    // ---- the keys of the block's 128 tokens (one 128-token key block, or 32
    // 4-token ones), eight 16-byte rows per thread, issued now and summed after
    // the rounds; rows >= N read as zeros (range-checked buffer loads, always
    // issued, so the count of loads in flight below is exact)
    constexpr int G = 256 / DCH;           // 128-token key block: thread (group g, chunk c), rows g + G i
    constexpr int RPT = kBlock / G;
    constexpr int kFine = kBlock / kFineBlock;
    constexpr int IPT = kFine * DCH / 256; // 4-token key blocks: (block, chunk) items per thread
    static_assert(RPT == 8 && RPT == IPT * kFineBlock, "eight key loads per thread in both cases");
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(k + bh * N_pad * D), (short)0, N * D * 2, 0x00020000);
    uint4 kraw[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        int r, c;
        if (KB == kBlock) {
            c = tid % DCH;
            r = tid / DCH + G * i;
        } else {
            const int it = i / kFineBlock, item = tid + 256 * it;
            c = item % DCH;
            r = kFineBlock * (item / DCH) + i % kFineBlock;
        }
        kraw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                rk, (qb * kBlock + r) * kPitch + 16 * c, 0, 0));
    }
    // the query copies are in LDS once at most the eight key loads remain in flight
    wait_loads_and_sync<RPT>();

    // this wavefront's 32 queries: the B fragments of the assignment product are
    // read from LDS in every round (holding them would leave too few registers
    // for the key rows kept across the rounds)
    const int my_q = wave * 32 + l32;
    const bool qv = my_q < n;

    // strided initial centroids q[floor(m n / C)] (bf16: the high part is the row
    // itself, the other two zero) and |c_m|^2, as in kmeans_mfma_kernel
    if (tid < kMaxClusters * DCH) {
        const int m = tid / DCH, c = tid % DCH;
        uint4 hi = make_uint4(0, 0, 0, 0);
        if (m < C) {
            const int r = m * n / C;
            hi = *reinterpret_cast<const uint4 *>(xrow(r) + xchunk(r, c));
        }
        const uint32_t *h = reinterpret_cast<const uint32_t *>(&hi);
        float nrm = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x0 = bf16_lo(h[e]), x1 = bf16_hi(h[e]);
            nrm = fmaf(x0, x0, nrm);
            nrm = fmaf(x1, x1, nrm);
        }
#pragma unroll
        for (int pp = 0; pp < 3; ++pp) {
            const int r = 8 * pp + m;
            cs_s[r * DCH + (c ^ (r & (DCH - 1)))] = pp == 0 ? hi : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int o = 1; o < DCH; o <<= 1) nrm += __shfl_xor(nrm, o, 64);
        if (c == 0) {
            cn_part[0][m] = nrm;
            cn_part[1][m] = cn_part[2][m] = cn_part[3][m] = 0.f;
        }
    }
    wait_loads_lds_and_sync<RPT>();
    uint16_t *cs16 = reinterpret_cast<uint16_t *>(cs_s);
    auto part_at = [&](int p, int m, int d) __attribute__((always_inline)) -> uint16_t & {
        const int rr = 8 * p + m;
        return cs16[(rr * DCH + ((d >> 3) ^ (rr & (DCH - 1)))) * 8 + (d & 7)];
    };
    auto centroid = [&](int m, int d) __attribute__((always_inline)) {
        return (bf16_bits_to_f32(part_at(0, m, d)) + bf16_bits_to_f32(part_at(1, m, d))) +
               bf16_bits_to_f32(part_at(2, m, d));
    };

    // Transposing reads of X for the update (the lane layout of the attention
    // kernel's V operand): lane (l32, half) of wavefront w receives dimension
    // 32w + l32 of queries 16ks + 4half + j (first read, rows row0 + 16ks) and
    // 16ks + 8 + 4half + j (second read, rows row0 + 8 + 16ks), j = 0..3; a
    // k-step of 16 rows keeps xswz, the 8 rows between the two reads do not.
    int x_rd0, x_rd1;
    {
        const int g = lane >> 4, m = lane & 15, row0 = 4 * (g >> 1) + (m >> 2);
        const int chunk = 4 * wave + 2 * (g & 1) + ((m & 3) >> 1);
        x_rd0 = row0 * kPitch + xchunk(row0, chunk) + 8 * (m & 1);
        x_rd1 = (row0 + 8) * kPitch + xchunk(row0 + 8, chunk) + 8 * (m & 1);
    }

    const int rounds = T_iters > 0 ? T_iters : 1;
    int prev = -1;
    for (int it = 0; it < rounds; ++it) {
        // ---- assignment: dots^T = C_split X^T for this wavefront's 32 queries
        floatx16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int ar = l32 < 24 ? l32 : l32 - 8;
            const uint4 a = cs_s[ar * DCH + ((2 * ks + half) ^ (ar & (DCH - 1)))];
            const uint4 x = *reinterpret_cast<const uint4 *>(xrow(my_q) + xchunk(my_q, 2 * ks + half));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, x),
                                                          acc, 0, 0, 0);
        }
        // the four wavefronts' shares of |c_m|^2 for this half's clusters 4half .. 4half+3
        float4 cnv[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) cnv[w] = *reinterpret_cast<const float4 *>(&cn_part[w][4 * half]);
        float bd = INFINITY;
        int bm = 4 * half;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = 4 * half + j;
            const float dot = acc[j] + acc[4 + j] + acc[8 + j];
            const float cn2 = cnv[0][j] + cnv[1][j] + cnv[2][j] + cnv[3][j];
            const float dist = m < C ? fmaf(-2.f, dot, cn2) : INFINITY;
            if (dist < bd) {
                bd = dist;
                bm = m;
            }
        }
        // the other half's candidate (lane l ^ 32), by one lane swap each
        const auto dsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bd), __float_as_uint(bd), false, false);
        const auto msw = __builtin_amdgcn_permlane32_swap((uint32_t)bm, (uint32_t)bm, false, false);
        const float od = __uint_as_float(half ? dsw[0] : dsw[1]);
        const int om = (int)(half ? msw[0] : msw[1]);
        if (od < bd || (od == bd && om < bm)) {
            bd = od;
            bm = om;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = 4 * half + j;
            flag_s[m * kFlagPitch + my_q] = (qv && bm == m) ? (uint8_t)0x80 : (uint8_t)0;
        }
        // this wavefront's cluster counts: lane m keeps count m, lanes 0..7 store
        int my_cnt = 0;
#pragma unroll
        for (int m = 0; m < kMaxClusters; ++m) {
            const int c = __popcll(__ballot(half == 0 && qv && bm == m));
            my_cnt = lane == m ? c : my_cnt;
        }
        if (lane < kMaxClusters) cnt_s[wave][lane] = my_cnt;
        const bool changed = __ballot(half == 0 && qv && bm != prev) != 0;
        prev = bm;
        if (lane == 0) chg_s[wave] = changed ? 1 : 0;
        wait_loads_lds_and_sync<RPT>();
        const bool any_changed = (chg_s[0] | chg_s[1] | chg_s[2] | chg_s[3]) != 0;
        if (T_iters == 0 || !any_changed) break;   // initial-centroid weights, or converged

        // ---- update: sums = onehot^T X, wavefront w owns dims [32w, 32w + 32)
        {
            floatx16 sum;
#pragma unroll
            for (int r = 0; r < 16; ++r) sum[r] = 0.f;
            const int d = wave * 32 + l32;
            // A operand row l32 is cluster l32 % 8; its k-step entries are the
            // flags of queries 16ks + 4half + j and 16ks + 8 + 4half + j, the
            // order in which the transposing reads hand over X
            const uint8_t *flag_row = flag_s + (l32 & 7) * kFlagPitch + 4 * half;
#pragma unroll
            for (int ks = 0; ks < kBlock / 16; ++ks) {
                const uint32_t f0 = *reinterpret_cast<const uint32_t *>(flag_row + 16 * ks);
                const uint32_t f1 = *reinterpret_cast<const uint32_t *>(flag_row + 16 * ks + 8);
                const uint4 oh = onehot4(f0, f1);
                const v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(xs + x_rd0 + 16 * ks * kPitch));
                const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(xs + x_rd1 + 16 * ks * kPitch));
                const bf16x8 b = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
                sum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, oh), b, sum, 0, 0, 0);
                // operands of at most two k-steps in flight: the registers go to
                // the key rows held across the rounds
                if (ks & 1) __builtin_amdgcn_sched_barrier(0);
            }
            const int4 c0 = *reinterpret_cast<const int4 *>(&cnt_s[0][4 * half]);
            const int4 c1 = *reinterpret_cast<const int4 *>(&cnt_s[1][4 * half]);
            const int4 c2 = *reinterpret_cast<const int4 *>(&cnt_s[2][4 * half]);
            const int4 c3 = *reinterpret_cast<const int4 *>(&cnt_s[3][4 * half]);
            const int cnts[4] = {c0.x + c1.x + c2.x + c3.x, c0.y + c1.y + c2.y + c3.y, c0.z + c1.z + c2.z + c3.z,
                                 c0.w + c1.w + c2.w + c3.w};
            float sq[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * half + r;
                const int cn = cnts[r];
                float cv;
                if (m < C && cn > 0) {
                    cv = sum[r] * __builtin_amdgcn_rcpf((float)(4 * cn));
                    const uint16_t hb = f32_to_bf16_bits(cv);
                    const float r1 = cv - bf16_bits_to_f32(hb);
                    const uint16_t mb = f32_to_bf16_bits(r1);
                    const uint16_t lb = f32_to_bf16_bits(r1 - bf16_bits_to_f32(mb));
                    part_at(0, m, d) = hb;
                    part_at(1, m, d) = mb;
                    part_at(2, m, d) = lb;
                } else {
                    cv = centroid(m, d);
                }
                sq[r] = cv * cv;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sq[r] = half_sum32(sq[r]);
            if (l32 == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r) cn_part[wave][4 * half + r] = sq[r];
            }
        }
        wait_loads_lds_and_sync<RPT>();
    }

    float *co = cent_out + (long)row * C * D;
    for (int i = tid; i < C * D; i += 256) co[i] = centroid(i / D, i % D);
    if (tid < C) {   // weights from the last assignment
        const int cn = cnt_s[0][tid] + cnt_s[1][tid] + cnt_s[2][tid] + cnt_s[3][tid];
        w_out[(long)row * C + tid] = (float)((double)cn / (double)n);
    }

    // ---- the pooled keys, from the rows loaded before the rounds (the same
    // summation order as kmeans_mfma_kernel and the standalone pooling kernels)
    if (KB == kBlock) {
        const int g = tid / DCH;
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            if (g + G * i >= n) break;
            const uint32_t w4[4] = {kraw[i].x, kraw[i].y, kraw[i].z, kraw[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += bf16_lo(w4[e]);
                acc[2 * e + 1] += bf16_hi(w4[e]);
            }
        }
        // the four groups of a wavefront (lanes c + 16 j) add up by lane swaps
        // between rows and between halves, no LDS
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[e]), __float_as_uint(acc[e]), false, false);
            acc[e] = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
            const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[e]), __float_as_uint(acc[e]), false, false);
            acc[e] = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
        }
        // every wavefront's last read of X lies before the loop's last barrier
        float *part = reinterpret_cast<float *>(xs);
        if (lane < DCH) {
#pragma unroll
            for (int e = 0; e < 8; ++e) part[wave * D + 8 * lane + e] = acc[e];
        }
        wait_loads_lds_and_sync<0>();
        if (tid < D)
            kbar[((long)bh * NBk + qb) * D + tid] =
                (((part[tid] + part[D + tid]) + part[2 * D + tid]) + part[3 * D + tid]) / (float)n;
    } else {
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int i = tid + 256 * it, g = i / DCH, c = i % DCH;
            const int j = qb * kFine + g;
            if (j >= NBk) continue;
            const int nr = min(kFineBlock, N - kFineBlock * j);
            float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int r = 0; r < kFineBlock; ++r) {
                if (r >= nr) break;
                const uint4 x = kraw[it * kFineBlock + r];
                const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] += bf16_lo(w4[e]);
                    acc[2 * e + 1] += bf16_hi(w4[e]);
                }
            }
            const float fn = (float)nr;
            float4 *dst = reinterpret_cast<float4 *>(kbar + ((long)bh * NBk + j) * D + 8 * c);
            dst[0] = make_float4(acc[0] / fn, acc[1] / fn, acc[2] / fn, acc[3] / fn);
            dst[1] = make_float4(acc[4] / fn, acc[5] / fn, acc[6] / fn, acc[7] / fn);
        }
    }
}

}  // namespace

hipError_t launch_kmeans(const void *q, const void *k, int dtype, int B, int H, int N, int N_pad, int D, int NB, int C,
                         int T, int kb, int NBk, float *cent, float *weight, float *kbar, bool *pooled, hipStream_t s)
{
    const dim3 grid((unsigned)((long)B * H * NB)), block(256);
    *pooled = dtype == kBF16;
    if (dtype == kBF16 && D == 128)
        (kb == kBlock ? kmeans_lds_kernel<128, kBlock> : kmeans_lds_kernel<128, kFineBlock>)<<<grid, block, 0, s>>>(
            (const uint16_t *)q, N, N_pad, NB, C, T, cent, weight, (const uint16_t *)k, NBk, kbar);
    else if (dtype == kBF16 && D == 64)
        kmeans_mfma_kernel<64><<<grid, block, 0, s>>>((const uint16_t *)q, N, N_pad, NB, C, T, cent, weight,
                                                      (const uint16_t *)k, kb, NBk, kbar);
    else if (dtype == kF32 && D == 64)
        kmeans_kernel<float, 64><<<grid, block, 0, s>>>((const float *)q, N, N_pad, NB, C, T, cent, weight);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace aba
