// pool_score.hip -- IBCS key pooling and block scoring (gfx950).
//
// AB-Attention page, section "Три приёма AB-Attention", IBCS paragraph: each key
// block is represented by its averaged keys, and scored by the cluster-weighted
// attention of the query block's centroids to them.
//
// pool : one workgroup per (b, h, key block) streams the block's keys once from
//        HBM with 16-byte loads and writes the fp32 mean of its valid rows.
//        HBM-bound: 128 * D * elem bytes read per block.
// score: one workgroup per (b, h, query block).  Logits l_mj = s * c_m . kbar_j
//        for all key blocks stay in registers, then a per-centroid softmax over
//        j and the weighted sum over centroids give one row of scores.
#include "aba_internal.h"

namespace aba {
namespace {

// ---------------------------------------------------------------------------
// Key pooling
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T *__restrict__ k, int N, int N_pad, int NB,
                                                   float *__restrict__ kbar)
{
    constexpr int kChunks = D / 8;             // 8-element chunks per row
    constexpr int kGroups = 256 / kChunks;     // row groups
    __shared__ float part[kGroups][D];

    const int blk = blockIdx.x;                // (b*H + h) * NB + j
    const int j = blk % NB;
    const long bh = blk / NB;
    const int n = min(kBlock, N - j * kBlock);
    const T *base = k + (bh * N_pad + (long)j * kBlock) * D;

    const int c = threadIdx.x % kChunks, g = threadIdx.x / kChunks;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 4
    for (int r = g; r < n; r += kGroups) {
        float x[8];
        load8(base + (long)r * D + 8 * c, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += x[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[g][8 * c + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
        float s = 0.f;
#pragma unroll 8
        for (int gg = 0; gg < kGroups; ++gg) s += part[gg][threadIdx.x];
        kbar[(long)blk * D + threadIdx.x] = s / (float)n;
    }
}

// ---------------------------------------------------------------------------
// Block scores.  Thread j owns key blocks j, j + 256, ...: it streams its pooled
// key rows from L1/L2 and reads the query block's centroids from LDS as
// broadcasts (every lane the same address), so the 8 x NB x D contraction is
// plain FMAs.  Per-centroid max and normaliser over the key blocks are two
// workgroup reductions; the logits never leave registers.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void score_kernel(const float *__restrict__ cent, const float *__restrict__ weight,
                                                    const float *__restrict__ kbar, int NB, int C, float scale,
                                                    float *__restrict__ scores)
{
    constexpr int JPT = kMaxBlocks / 256;     // key blocks per thread at most
    __shared__ float4 c_s[kMaxClusters][D / 4];
    __shared__ float red[2][4][kMaxClusters];

    const int row = blockIdx.x;               // (b*H + h) * NB + query block
    const long bh = row / NB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *kb = kbar + bh * NB * D;

    // centroids of this query block; rows >= C are zero (their logits are dropped)
    const float4 *c4 = reinterpret_cast<const float4 *>(cent + (long)row * C * D);
    for (int i = tid; i < kMaxClusters * D / 4; i += 256)
        c_s[i / (D / 4)][i % (D / 4)] = (i / (D / 4) < C) ? c4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();

    float lg[JPT][kMaxClusters];
#pragma unroll
    for (int t = 0; t < JPT; ++t) {
        const int j = tid + 256 * t;
        float acc[kMaxClusters];
#pragma unroll
        for (int m = 0; m < kMaxClusters; ++m) acc[m] = 0.f;
        if (j < NB) {
            const float4 *kr = reinterpret_cast<const float4 *>(kb + (long)j * D);
#pragma unroll 4
            for (int d4 = 0; d4 < D / 4; ++d4) {
                const float4 x = kr[d4];
#pragma unroll
                for (int m = 0; m < kMaxClusters; ++m) {
                    const float4 cc = c_s[m][d4];
                    float a = acc[m];
                    a = fmaf(cc.x, x.x, a);
                    a = fmaf(cc.y, x.y, a);
                    a = fmaf(cc.z, x.z, a);
                    a = fmaf(cc.w, x.w, a);
                    acc[m] = a;
                }
            }
        }
#pragma unroll
        for (int m = 0; m < kMaxClusters; ++m) lg[t][m] = (j < NB && m < C) ? scale * acc[m] : -INFINITY;
    }

    // per-centroid max over key blocks
    float mx[kMaxClusters];
#pragma unroll
    for (int m = 0; m < kMaxClusters; ++m) {
        float v = lg[0][m];
#pragma unroll
        for (int t = 1; t < JPT; ++t) v = fmaxf(v, lg[t][m]);
        v = wave_max(v);
        if (lane == 0) red[0][wave][m] = v;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < kMaxClusters; ++m)
        mx[m] = fmaxf(fmaxf(red[0][0][m], red[0][1][m]), fmaxf(red[0][2][m], red[0][3][m]));

    // exponentials and per-centroid normalisers
#pragma unroll
    for (int m = 0; m < kMaxClusters; ++m) {
        float v = 0.f;
#pragma unroll
        for (int t = 0; t < JPT; ++t) {
            lg[t][m] = (m < C) ? __expf(lg[t][m] - mx[m]) : 0.f;
            v += lg[t][m];
        }
        v = wave_sum(v);
        if (lane == 0) red[1][wave][m] = v;
    }
    __syncthreads();
    float coef[kMaxClusters];
#pragma unroll
    for (int m = 0; m < kMaxClusters; ++m)
        coef[m] = (m < C) ? weight[(long)row * C + m] / (red[1][0][m] + red[1][1][m] + red[1][2][m] + red[1][3][m])
                          : 0.f;

    float *out = scores + (long)row * NB;
#pragma unroll
    for (int t = 0; t < JPT; ++t) {
        const int j = tid + 256 * t;
        if (j < NB) {
            float s = 0.f;
#pragma unroll
            for (int m = 0; m < kMaxClusters; ++m) s = fmaf(coef[m], lg[t][m], s);
            out[j] = s;
        }
    }
}

}  // namespace

hipError_t launch_pool(const void *k, int dtype, int B, int H, int N, int N_pad, int D, int NB, float *kbar,
                       hipStream_t s)
{
    const dim3 grid((unsigned)((long)B * H * NB)), block(256);
    if (dtype == kBF16 && D == 128)
        pool_kernel<uint16_t, 128><<<grid, block, 0, s>>>((const uint16_t *)k, N, N_pad, NB, kbar);
    else if (dtype == kBF16 && D == 64)
        pool_kernel<uint16_t, 64><<<grid, block, 0, s>>>((const uint16_t *)k, N, N_pad, NB, kbar);
    else if (dtype == kF32 && D == 64)
        pool_kernel<float, 64><<<grid, block, 0, s>>>((const float *)k, N, N_pad, NB, kbar);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_score(const float *cent, const float *weight, const float *kbar, int B, int H, int NB, int C, int D,
                        float scale, float *scores, hipStream_t s)
{
    const dim3 grid((unsigned)((long)B * H * NB)), block(256);
    if (D == 128)
        score_kernel<128><<<grid, block, 0, s>>>(cent, weight, kbar, NB, C, scale, scores);
    else if (D == 64)
        score_kernel<64><<<grid, block, 0, s>>>(cent, weight, kbar, NB, C, scale, scores);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace aba
