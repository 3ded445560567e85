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

__device__ __forceinline__ float to_f32(uint16_t bits) { return __uint_as_float((uint32_t)bits << 16); }
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

}  // namespace

hipError_t launch_kmeans(const void *q, int dtype, int B, int H, int N, int N_pad, int D, int NB, int C, int T,
                         float *cent, float *weight, hipStream_t s)
{
    const dim3 grid((unsigned)((long)B * H * NB)), block(256);
    if (dtype == kBF16 && D == 128)
        kmeans_kernel<uint16_t, 128><<<grid, block, 0, s>>>((const uint16_t *)q, N, N_pad, NB, C, T, cent, weight);
    else if (dtype == kBF16 && D == 64)
        kmeans_kernel<uint16_t, 64><<<grid, block, 0, s>>>((const uint16_t *)q, N, N_pad, NB, C, T, cent, weight);
    else if (dtype == kF32 && D == 64)
        kmeans_kernel<float, 64><<<grid, block, 0, s>>>((const float *)q, N, N_pad, NB, C, T, cent, weight);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace aba
