// sample.hip -- SIP inclusion probabilities, counter-based draws and list
// compaction (gfx950).
//
// AB-Attention page, section "Три приёма AB-Attention", SIP paragraph: a key
// block is sampled with probability proportional to its score, the most
// important blocks always, every other block with a non-zero chance; a kept
// block counts 1/pi times (Horvitz-Thompson: 25% counts as four).
//
// One workgroup per (b, h, query block) row.  All decisions are integer so
// that they are bit-reproducible:
//   sigma_j = clamp(floor(S_j * 2^32), 1, 2^32)     (uint64, exact)
//   bitonic sort of (sigma desc, j asc) in LDS; water-filling over the sorted
//   prefix by one lane (at most K steps); thresholds by exact 96/64-bit long
//   division; draws from Philox4x32-10 addressed by (seed, b, h, qb, j);
//   kept blocks compacted in ascending order with a workgroup prefix sum.
#include "aba_internal.h"

namespace aba {
namespace {

constexpr uint64_t kOne = 1ull << 32;
constexpr int kIdxBits = 10;   // kMaxBlocks = 2^10: block index packed under sigma

__device__ __forceinline__ uint64_t fixed_point(float s)
{
    if (!(s > 0.f)) return 1;                       // zero, negative, NaN
    const double v = floor((double)s * 4294967296.0);
    if (v >= 4294967296.0) return kOne;
    const uint64_t r = (uint64_t)v;
    return r < 1 ? 1 : r;
}

// ceil(x * 2^32 / r) for x < r, by restoring long division (32 quotient bits).
__device__ __forceinline__ uint64_t ceil_scaled_ratio(uint64_t x, uint64_t r)
{
    uint64_t rem = x, quo = 0;
#pragma unroll 4
    for (int i = 0; i < 32; ++i) {
        rem <<= 1;
        quo <<= 1;
        if (rem >= r) {
            rem -= r;
            quo |= 1;
        }
    }
    return quo + (rem != 0 ? 1 : 0);
}

// Philox4x32-10 block function (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds,
// each two 32x32 -> 64-bit products with the published multipliers, the key
// advanced by the published Weyl increments between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
        const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

__global__ __launch_bounds__(256) void sample_kernel(const float *__restrict__ scores, int H, int NB, int K,
                                                     uint64_t seed, int cap, int32_t *__restrict__ idx,
                                                     int32_t *__restrict__ cnt, float *__restrict__ w)
{
    __shared__ uint64_t keys[kMaxBlocks];
    __shared__ uint8_t capped[kMaxBlocks];
    __shared__ uint64_t red[4];
    __shared__ int scan[256];
    __shared__ int t_s;
    __shared__ uint64_t r_s;

    const int row = blockIdx.x;
    const int qb = row % NB, h = (row / NB) % H, b = row / (NB * H);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *srow = scores + (long)row * NB;

    int P = 1;
    while (P < NB) P <<= 1;

    // fixed-point scores, packed sort keys, row total
    uint64_t part = 0;
    for (int j = tid; j < P; j += 256) {
        if (j < NB) {
            const uint64_t sg = fixed_point(srow[j]);
            part += sg;
            keys[j] = (sg << kIdxBits) | (uint64_t)(kMaxBlocks - 1 - j);
            capped[j] = 0;
        } else {
            keys[j] = 0;   // below every real key
        }
    }
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    if (lane == 0) red[wave] = part;
    __syncthreads();
    const uint64_t total = red[0] + red[1] + red[2] + red[3];

    // bitonic sort, descending
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < P / 2; i += 256) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool desc = ((lo & size) == 0);
                const uint64_t a = keys[lo], c = keys[hi];
                if ((a < c) == desc) {
                    keys[lo] = c;
                    keys[hi] = a;
                }
            }
            __syncthreads();
        }
    }

    // water-filling over the sorted order (the first block is always kept)
    if (tid == 0) {
        int t = 1;
        uint64_t R = total - (keys[0] >> kIdxBits);
        while (t < NB && K - t > 0) {
            const uint64_t sg = keys[t] >> kIdxBits;
            if ((uint64_t)(K - t) * sg < R) break;
            R -= sg;
            ++t;
        }
        t_s = t;
        r_s = R;
    }
    __syncthreads();
    const int t = t_s;
    const uint64_t R = r_s;
    for (int p = tid; p < t; p += 256) capped[kMaxBlocks - 1 - (int)(keys[p] & (kMaxBlocks - 1))] = 1;
    __syncthreads();

    // draws: thread g owns key blocks 4g .. 4g+3 (one Philox block)
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const int groups = (NB + 3) / 4;
    int32_t *irow = idx + (long)row * cap;
    float *wrow = w + (long)row * cap;
    int base = 0;
    for (int g0 = 0; g0 < groups; g0 += 256) {
        const int g = g0 + tid;
        uint32_t keep = 0;
        uint64_t theta[4] = {0, 0, 0, 0};
        if (g < groups) {
            const uint4 r = philox4x32_10(make_uint4((uint32_t)g, (uint32_t)qb, (uint32_t)h, (uint32_t)b), k0, k1);
            const uint32_t draw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * g + e;
                if (j >= NB) break;
                uint64_t th;
                if (capped[j]) {
                    th = kOne;
                } else if (K - t <= 0) {
                    th = 1;
                } else {
                    const uint64_t x = (uint64_t)(K - t) * fixed_point(srow[j]);
                    th = (x >= R) ? kOne : ceil_scaled_ratio(x, R);
                    th = th < 1 ? 1 : (th > kOne ? kOne : th);
                }
                theta[e] = th;
                if ((uint64_t)draw[e] < th) keep |= 1u << e;
            }
        }
        // exclusive prefix sum of the kept counts over the workgroup
        const int mine = __popc(keep);
        scan[tid] = mine;
        __syncthreads();
        for (int o = 1; o < 256; o <<= 1) {
            const int v = tid >= o ? scan[tid - o] : 0;
            __syncthreads();
            scan[tid] += v;
            __syncthreads();
        }
        int pos = base + scan[tid] - mine;
        const int chunk_total = scan[255];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (keep & (1u << e)) {
                if (pos < cap) {
                    irow[pos] = 4 * g + e;
                    wrow[pos] = (float)(4294967296.0 / (double)theta[e]);
                }
                ++pos;
            }
        }
        base += chunk_total;
        __syncthreads();
    }
    if (tid == 0) cnt[row] = base < cap ? base : cap;
}

}  // namespace

hipError_t launch_sample(const float *scores, int B, int H, int NB, int K, uint64_t seed, int cap, int32_t *idx,
                         int32_t *cnt, float *w, hipStream_t s)
{
    if (NB > kMaxBlocks) return hipErrorInvalidValue;
    sample_kernel<<<dim3((unsigned)((long)B * H * NB)), dim3(256), 0, s>>>(scores, H, NB, K, seed, cap, idx, cnt, w);
    return hipGetLastError();
}

}  // namespace aba
