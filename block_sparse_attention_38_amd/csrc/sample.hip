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

__global__ __launch_bounds__(256) void sample_kernel(const float *__restrict__ scores, int H, int NBq, int NB, int K,
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
    const int qb = row % NBq, h = (row / NBq) % H, b = row / (NBq * H);
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


// ---------------------------------------------------------------------------
// Long rows (more than kMaxBlocks key blocks: 4-token key blocks give N/4 per
// row).  The decisions are the ones above, bit for bit, without sorting the
// row: the water-filling loop never looks past position min(K, NB) - 1 of the
// sorted order, so only the top T = min(K, NB) keys (sigma desc, j asc) are
// sorted.
//   1. sigma - 1 of every block into LDS (uint32), row total;
//   2. radix select (4 passes of 8 bits) of the T-th largest sigma, v, and
//      how many of the blocks with sigma - 1 == v belong to the top T (the
//      lowest indices among them);
//   3. the top T gathered in index order (per-thread ranges + a workgroup
//      scan) and bitonic-sorted by the packed key (sigma - 1) << 15 | ~j;
//   4. the loop's stopping point t: the first position p >= 1 of the sorted
//      prefix where (K - p) sigma_p < R_p (R_p = total - sum of the first p),
//      found in parallel from a prefix sum, else min(K, NB);
//   5. capped blocks are those whose key is >= the key at position t - 1;
//      another block is kept iff draw < theta = ceil(x 2^32 / R) with x =
//      (K - t) sigma, which for an integer draw is draw * R < x * 2^32, an
//      exact 128-bit comparison; theta itself (for the weight) is formed only
//      for kept blocks.  Kept blocks are written in index order.
// K >= NB caps every block (the loop then ends at t = NB), so that case keeps
// everything with weight 1 and skips 2-5.
// ---------------------------------------------------------------------------
constexpr int kKeyIdxBits = 15;                       // key blocks per row < 2^15
constexpr uint32_t kKeyIdxMask = (1u << kKeyIdxBits) - 1;

__device__ __forceinline__ uint64_t pack_key(uint32_t sig_m1, int j)
{
    return ((uint64_t)sig_m1 << kKeyIdxBits) | (uint64_t)(kKeyIdxMask - (uint32_t)j);
}

// Exclusive prefix sum over the 256 threads of the workgroup (tmp: 4 slots).
template <typename T> __device__ __forceinline__ T block_excl_scan(T v, T *tmp, T &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    T inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const T y = __shfl_up(inc, d, 64);
        if (lane >= d) inc += y;
    }
    if (lane == 63) tmp[wave] = inc;
    __syncthreads();
    T base = 0, all = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i < wave) base += tmp[i];
        all += tmp[i];
    }
    __syncthreads();
    total = all;
    return base + inc - v;
}

// 128-bit test a * b < c * 2^32 for a < 2^32, b, c < 2^63.
__device__ __forceinline__ bool mul_less_shift32(uint64_t a, uint64_t b, uint64_t c)
{
    const uint64_t lo = a * b, hi = __umul64hi(a, b);
    const uint64_t clo = c << 32, chi = c >> 32;
    return hi < chi || (hi == chi && lo < clo);
}

__global__ __launch_bounds__(256) void sample_topk_kernel(const float *__restrict__ scores, int H, int NBq, int NB,
                                                          int K, uint64_t seed, int cap, int P,
                                                          int32_t *__restrict__ idx, int32_t *__restrict__ cnt,
                                                          float *__restrict__ w)
{
    extern __shared__ __align__(16) char dyn[];
    uint64_t *top = reinterpret_cast<uint64_t *>(dyn);          // P sorted keys
    uint32_t *sig = reinterpret_cast<uint32_t *>(dyn + 8 * (size_t)P);   // NB values sigma - 1
    __shared__ int hist[256];
    __shared__ int itmp[4];
    __shared__ uint64_t utmp[4];
    __shared__ int sel_s[2];          // radix digit, remaining count
    __shared__ int t_s;
    __shared__ uint64_t r_s, cut_s;

    const int row = blockIdx.x;
    const int qb = row % NBq, h = (row / NBq) % H, b = row / (NBq * H);
    const int tid = threadIdx.x;
    const float *srow = scores + (long)row * NB;
    int32_t *irow = idx + (long)row * cap;
    float *wrow = w + (long)row * cap;

    // 1. fixed-point scores and the row total
    uint64_t part = 0;
    for (int j = tid; j < NB; j += 256) {
        const uint64_t sg = fixed_point(srow[j]);
        part += sg;
        sig[j] = (uint32_t)(sg - 1);
    }
    uint64_t total;
    block_excl_scan<uint64_t>(part, utmp, total);   // also a barrier: sig[] is complete

    // per-thread contiguous ranges of 4-aligned indices (one Philox block per 4)
    const int per = 4 * ((((NB + 3) / 4) + 255) / 256);
    const int lo_j = min(NB, tid * per), hi_j = min(NB, lo_j + per);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);

    if (K >= NB) {   // every block capped: keep all, weight 1
        for (int j = tid; j < NB; j += 256)
            if (j < cap) {
                irow[j] = j;
                wrow[j] = 1.0f;
            }
        if (tid == 0) cnt[row] = NB < cap ? NB : cap;
        return;
    }
    const int T = K;   // K < NB here

    // 2. radix select of the T-th largest sigma - 1
    uint32_t prefix = 0, himask = 0;
    int need = T;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        hist[tid] = 0;
        __syncthreads();
        for (int j = tid; j < NB; j += 256) {
            const uint32_t v = sig[j];
            if (((v ^ prefix) & himask) == 0) atomicAdd(&hist[(v >> shift) & 255], 1);
        }
        __syncthreads();
        const int c = hist[255 - tid];                // digits from high to low
        int tot;
        const int before = block_excl_scan<int>(c, itmp, tot);
        if (before < need && need <= before + c) {
            sel_s[0] = 255 - tid;
            sel_s[1] = need - before;
        }
        __syncthreads();
        prefix |= (uint32_t)sel_s[0] << shift;
        himask |= 255u << shift;
        need = sel_s[1];
    }
    const uint32_t v = prefix;   // T-th largest sigma - 1; `need` of its ties (lowest j) are in the top T

    // 3. gather the top T in index order, then sort them
    int n_gt = 0, n_eq = 0;
    for (int j = lo_j; j < hi_j; ++j) {
        const uint32_t x = sig[j];
        n_gt += x > v;
        n_eq += x == v;
    }
    int tot_packed;
    const int base_packed = block_excl_scan<int>((n_gt << 16) | n_eq, itmp, tot_packed);
    int gt_before = base_packed >> 16, eq_before = base_packed & 0xFFFF;
    for (int j = lo_j; j < hi_j; ++j) {
        const uint32_t x = sig[j];
        if (x > v) {
            top[gt_before + min(eq_before, need)] = pack_key(x, j);
            ++gt_before;
        } else if (x == v) {
            if (eq_before < need) top[gt_before + eq_before] = pack_key(x, j);
            ++eq_before;
        }
    }
    for (int i = T + tid; i < P; i += 256) top[i] = 0;   // below every real key (or equal to, and decoding alike)
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < P / 2; i += 256) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool desc = ((lo & size) == 0);
                const uint64_t a = top[lo], c = top[hi];
                if ((a < c) == desc) {
                    top[lo] = c;
                    top[hi] = a;
                }
            }
            __syncthreads();
        }
    }

    // 4. stopping point of the water-filling loop over positions 1 .. T-1
    if (tid == 0) t_s = T;
    const int q = (T + 255) / 256;
    const int p0 = min(T, tid * q), p1 = min(T, p0 + q);
    uint64_t local = 0;
    for (int p = p0; p < p1; ++p) local += (top[p] >> kKeyIdxBits) + 1;
    uint64_t dummy;
    uint64_t pre = block_excl_scan<uint64_t>(local, utmp, dummy);   // barrier: t_s is set
    for (int p = p0; p < p1; ++p) {
        const uint64_t sg = (top[p] >> kKeyIdxBits) + 1;
        if (p >= 1 && (uint64_t)(K - p) * sg < total - pre) {
            atomicMin(&t_s, p);
            break;
        }
        pre += sg;
    }
    __syncthreads();
    const int t = t_s;
    if (tid == 0) cut_s = top[t - 1];
    {   // R = total - (sum of the first t sorted sigma)
        uint64_t pre2 = block_excl_scan<uint64_t>(local, utmp, dummy);
        for (int p = p0; p < p1; ++p) {
            const uint64_t sg = (top[p] >> kKeyIdxBits) + 1;
            if (p == t - 1) r_s = total - (pre2 + sg);
            pre2 += sg;
        }
    }
    __syncthreads();
    const uint64_t R = r_s, cut = cut_s;
    const uint64_t Kt = (uint64_t)(K - t);   // >= 0 since t <= T = K

    // 5. keep decisions over this thread's range, then the compaction in index order
    uint32_t mask[(kMaxFineBlocks / 256 + 31) / 32] = {};
    int mine = 0;
    // a non-empty range starts at a multiple of 4 (ranges past the row are empty
    // and start at NB, which need not be one)
    for (int g = lo_j / 4; lo_j < hi_j && 4 * g < hi_j; ++g) {
        const uint4 r = philox4x32_10(make_uint4((uint32_t)g, (uint32_t)qb, (uint32_t)h, (uint32_t)b), k0, k1);
        const uint32_t draw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * g + e;
            if (j >= hi_j) break;
            const uint32_t x = sig[j];
            bool keep;
            if (pack_key(x, j) >= cut) keep = true;
            else if (Kt == 0) keep = draw[e] == 0;                       // theta = 1
            else keep = mul_less_shift32(draw[e], R, Kt * ((uint64_t)x + 1));
            if (keep) {
                const int o = j - lo_j;
                mask[o >> 5] |= 1u << (o & 31);
                ++mine;
            }
        }
    }
    int kept_total;
    int pos = block_excl_scan<int>(mine, itmp, kept_total);
    for (int o = 0; lo_j + o < hi_j; ++o) {
        if (!(mask[o >> 5] & (1u << (o & 31)))) continue;
        const int j = lo_j + o;
        if (pos < cap) {
            const uint32_t x = sig[j];
            uint64_t th;
            if (pack_key(x, j) >= cut) {
                th = kOne;
            } else if (Kt == 0) {
                th = 1;
            } else {
                const uint64_t xx = Kt * ((uint64_t)x + 1);
                th = (xx >= R) ? kOne : ceil_scaled_ratio(xx, R);
                th = th < 1 ? 1 : (th > kOne ? kOne : th);
            }
            irow[pos] = j;
            wrow[pos] = (float)(4294967296.0 / (double)th);
        }
        ++pos;
    }
    if (tid == 0) cnt[row] = kept_total < cap ? kept_total : cap;
}

}  // namespace

// Keys of the sorted top (P of them, P = 2^ceil(log2 K) when K < NB, else 1)
// followed by sigma - 1 of every block.
static int topk_pad(int NB, int K)
{
    int P = 1;
    while (K < NB && P < K) P <<= 1;
    return P;
}

size_t sample_lds_bytes(int NB, int K)
{
    if (NB <= kMaxBlocks) return 0;
    return 8 * (size_t)topk_pad(NB, K) + 4 * (size_t)NB;
}

hipError_t launch_sample(const float *scores, int B, int H, int NBq, int NB, int K, uint64_t seed, int cap,
                         int32_t *idx, int32_t *cnt, float *w, hipStream_t s)
{
    const dim3 grid((unsigned)((long)B * H * NBq)), block(256);
    if (NB <= kMaxBlocks) {
        sample_kernel<<<grid, block, 0, s>>>(scores, H, NBq, NB, K, seed, cap, idx, cnt, w);
        return hipGetLastError();
    }
    if (NB > kMaxFineBlocks) return hipErrorInvalidValue;
    const size_t lds = sample_lds_bytes(NB, K);
    if (lds > kSampleLdsLimit) return hipErrorInvalidValue;
    const int P = topk_pad(NB, K);
    // allow more than the default dynamic LDS (a host-side attribute of the current device)
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&sample_topk_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSampleLdsLimit);
    if (e != hipSuccess) return e;
    sample_topk_kernel<<<grid, block, lds, s>>>(scores, H, NBq, NB, K, seed, cap, P, idx, cnt, w);
    return hipGetLastError();
}

}  // namespace aba
