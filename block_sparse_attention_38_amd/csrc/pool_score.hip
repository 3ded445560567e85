// pool_score.hip -- IBCS key pooling of 128-token key blocks (gfx950).
//
// AB-Attention page, section "Три приёма AB-Attention", IBCS paragraph: each key
// block is represented by its averaged keys.  One workgroup per (b, h, key
// block) streams the block's keys once from HBM with 16-byte loads and writes
// the fp32 mean of its valid rows: HBM-bound, 128 * D * elem bytes read per
// block.  The scoring contraction (for either key block size) is in
// fine_score.hip.
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

}  // namespace aba
