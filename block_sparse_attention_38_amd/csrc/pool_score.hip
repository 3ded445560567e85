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
//        for all key blocks are kept in LDS, then a per-centroid softmax over j
//        and the weighted sum over centroids give one row of scores.
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
// Block scores
// ---------------------------------------------------------------------------
constexpr int kTileRows = 32;

template <int D>
__global__ __launch_bounds__(256) void score_kernel(const float *__restrict__ cent, const float *__restrict__ weight,
                                                    const float *__restrict__ kbar, int NB, int C, float scale,
                                                    float *__restrict__ scores)
{
    __shared__ float4 c_s[kMaxClusters][D / 4];
    __shared__ float4 k_s[kTileRows][D / 4 + 1];   // +1 float4 per row: conflict-free column reads
    __shared__ float logit[kMaxClusters][kMaxBlocks];
    __shared__ float w_s[kMaxClusters], mx_s[kMaxClusters], iz_s[kMaxClusters];

    const int row = blockIdx.x;                    // (b*H + h) * NB + query block
    const long bh = row / NB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int i = tid; i < C * D / 4; i += 256)
        c_s[i / (D / 4)][i % (D / 4)] = reinterpret_cast<const float4 *>(cent + (long)row * C * D)[i];
    if (tid < C) w_s[tid] = weight[(long)row * C + tid];

    const float4 *kb = reinterpret_cast<const float4 *>(kbar + bh * NB * D);
    const int jl = tid % kTileRows, m = tid / kTileRows;     // 8 clusters x 32 key blocks per pass
    for (int j0 = 0; j0 < NB; j0 += kTileRows) {
        __syncthreads();
        for (int i = tid; i < kTileRows * D / 4; i += 256) {
            const int r = i / (D / 4), cc = i % (D / 4);
            k_s[r][cc] = (j0 + r < NB) ? kb[(long)(j0 + r) * (D / 4) + cc] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        __syncthreads();
        if (m < C && j0 + jl < NB) {
            float dot = 0.f;
#pragma unroll 8
            for (int cc = 0; cc < D / 4; ++cc) {
                const float4 a = c_s[m][cc], b = k_s[jl][cc];
                dot = fmaf(a.x, b.x, dot);
                dot = fmaf(a.y, b.y, dot);
                dot = fmaf(a.z, b.z, dot);
                dot = fmaf(a.w, b.w, dot);
            }
            logit[m][j0 + jl] = scale * dot;
        }
    }
    __syncthreads();

    // Per-centroid softmax statistics over the key blocks: wave w handles
    // clusters w and w + 4.
    for (int mm = wave; mm < C; mm += 4) {
        float mx = -INFINITY;
        for (int j = lane; j < NB; j += 64) mx = fmaxf(mx, logit[mm][j]);
        mx = wave_max(mx);
        float z = 0.f;
        for (int j = lane; j < NB; j += 64) z += __expf(logit[mm][j] - mx);
        z = wave_sum(z);
        if (lane == 0) {
            mx_s[mm] = mx;
            iz_s[mm] = 1.f / z;
        }
    }
    __syncthreads();

    float *out = scores + (long)row * NB;
    for (int j = tid; j < NB; j += 256) {
        float s = 0.f;
        for (int mm = 0; mm < C; ++mm) s += w_s[mm] * (__expf(logit[mm][j] - mx_s[mm]) * iz_s[mm]);
        out[j] = s;
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
