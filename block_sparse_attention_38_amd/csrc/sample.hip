// sample.hip -- SIP inclusion probabilities, counter-based draws and list
// compaction (gfx950).
//
// AB-Attention page, section "Три приёма AB-Attention", SIP paragraph: a key
// block is sampled with probability proportional to its score, the most
// important blocks always, every other block with a non-zero chance; a kept
// block counts 1/pi times (Horvitz-Thompson: 25% counts as four).
//
// One workgroup per (b, h, query block) row, for rows of any length (256
// 128-token blocks or N/4 4-token blocks).  All decisions are integer so that
// they are bit-reproducible:
//   sigma_j = clamp(floor(S_j * 2^32), 1, 2^32)     (uint64, exact)
//   water-filling over the order (sigma desc, j asc); thresholds by exact
//   128-bit comparisons; draws from Philox4x32-10 addressed by (seed, b, h,
//   qb, j), with b and h the global batch and head indices (a call may cover
//   a slice of heads of a larger layer); kept blocks compacted in ascending
//   order.
#include "aba_internal.h"

#include <array>

namespace aba {
namespace {

constexpr uint64_t kOne = 1ull << 32;

// clamp(floor(s * 2^32), 1, 2^32), exactly, from the bits of s: a positive
// float below 1 is m * 2^(e - 150) with m its 24-bit significand (e the biased
// exponent; subnormals: e = 1 and no hidden bit), so s * 2^32 = m * 2^(e - 118)
// and the floor is a shift.  (Equal to the fp64 evaluation for every float.)
__device__ __forceinline__ uint64_t fixed_point(float s)
{
    if (!(s > 0.f)) return 1;                       // zero, negative, NaN
    const uint32_t b = __float_as_uint(s);
    const int e = (int)(b >> 23);
    if (e >= 127) return kOne;                      // s >= 1, inf
    const uint32_t m = e ? ((b & 0x7FFFFFu) | 0x800000u) : (b & 0x7FFFFFu);
    const int sh = (e ? e : 1) - 118;
    const uint64_t r = sh >= 0 ? ((uint64_t)m << sh) : (sh > -32 ? (uint64_t)(m >> -sh) : 0);
    return r < 1 ? 1 : r;
}

// Philox4x32-10 block function (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds,
// each two 32x32 -> 64-bit products with the published multipliers, the key
// advanced by the published Weyl increments between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        // each 32 x 32 -> 64-bit product is one instruction (v_mad_u64_u32)
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.x, p1 = (uint64_t)0xCD9E8D57u * c.z;
        const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
        const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// ---------------------------------------------------------------------------
// The row is never sorted: the water-filling loop stops at the first position
// p >= 1 of the sorted order where (K - p) sigma_p < R_p (R_p = total - sum of
// the first p), and never looks past position min(K, NB) - 1, so only a sorted
// top of the row is needed.
//
// Work is split in "quads" of 4 consecutive blocks (one Philox call, one
// 16-byte LDS read): wavefront w owns a contiguous run of quads and its lane l
// takes quad q0 + 64k + l at step k, so reads are conflict-free and every
// ordered pass runs in index order.
//   1. sigma - 1 of every block into LDS (uint32), the row total, min and max;
//   2. top(T), ordered by the packed key (sigma - 1) << 15 | ~j: for T <= 64
//      the blocks at or above a bound (the T-th largest of the threads'
//      maxima) are collected, and when at most 512 of them, each one's rank
//      among them places it; otherwise the T-th largest sigma - 1, v, comes
//      from a radix select over [bound, max] (8 bits per pass from the top of
//      the range, per-wavefront LDS histograms with one atomic per distinct
//      bin; v = min directly when fewer than T blocks exceed it), the lowest
//      indices are taken when more blocks equal v than the top has room for
//      (an 8-way bisection on the index), and the top is gathered unsorted;
//   3. the stopping point: first with T = min(K, 64), sorted and scanned inside
//      one wavefront with shuffles; when the loop stops inside that top (fewer
//      than 64 blocks capped, the usual case) nothing more is needed;
//      otherwise the top T = K is sorted by the whole workgroup in LDS and
//      scanned in parallel;
//   4. capped blocks are those whose key is >= the key at position t - 1;
//      another block is kept iff draw < theta = ceil(x 2^32 / R) with x =
//      (K - t) sigma, which for an integer draw is draw * R < x * 2^32, an
//      exact 128-bit comparison.  theta itself (for the weight) is formed only
//      for kept blocks: an fp64 estimate (x 2^32 times 1/R), corrected to the
//      exact ceiling with two 128-bit products.  Kept blocks are compacted in
//      index order (a count pass, a scan over wavefronts, a pass with a shuffle
//      scan per step that places the indices in LDS), then every thread forms
//      the weights of consecutive list positions.
// K >= NB caps every block (the loop then ends at t = NB), so that case keeps
// everything with weight 1 and skips 2-4.
// ---------------------------------------------------------------------------
constexpr int kKeyIdxBits = 15;                       // key blocks per row < 2^15
constexpr uint32_t kKeyIdxMask = (1u << kKeyIdxBits) - 1;
constexpr int kFastTop = 64;                          // sorted top tried first (one wavefront)
constexpr int kCandMax = 512;                         // blocks ranked directly for the fast top

__device__ __forceinline__ uint64_t pack_key(uint32_t sig_m1, int j)
{
    return ((uint64_t)sig_m1 << kKeyIdxBits) | (uint64_t)(kKeyIdxMask - (uint32_t)j);
}

// 128-bit a * b for a < 2^33, b < 2^48, against c * 2^32 for c < 2^48.
__device__ __forceinline__ int cmp_mul_shift32(uint64_t a, uint64_t b, uint64_t c)
{
    const uint64_t lo = a * b, hi = __umul64hi(a, b);
    const uint64_t clo = c << 32, chi = c >> 32;
    if (hi != chi) return hi < chi ? -1 : 1;
    return lo < clo ? -1 : (lo > clo ? 1 : 0);
}

// ceil(x * 2^32 / r) for 1 <= x < r < 2^48, given inv_r ~ 1/r in fp64: the
// estimate is within a few 2^-52 relative of x 2^32 / r < 2^32, so its ceiling
// is off by at most one; fixed exactly.
__device__ __forceinline__ uint64_t ceil_ratio_shift32(uint64_t x, uint64_t r, double inv_r)
{
    uint64_t th = (uint64_t)ceil((double)x * 4294967296.0 * inv_r);
    if (cmp_mul_shift32(th, r, x) < 0) ++th;                        // th * r < x 2^32: too small
    else if (th > 0 && cmp_mul_shift32(th - 1, r, x) >= 0) --th;    // (th - 1) r >= x 2^32: too large
    return th;
}

// Whether block j (sigma - 1 = x) is kept: capped blocks always, any other iff
// its draw is below theta = ceil((K - t) sigma 2^32 / R), i.e. (the draw being
// an integer) draw < y = (K - t) sigma 2^32 / R, or draw == 0 when K - t = 0.
// The test runs in fp32 first: c = fl((K - t) 2^32 / R) once per row, y ~
// fl(fl(x) c + c), whose relative error is below 3 x 2^-24 (about 1546 units
// where y <= 2^33; beyond, the draw is below y anyway), and fl(draw) is within
// 256 of the draw.  Outside a guard band of 4096 around y the fp32 comparison
// decides; inside it the exact 128-bit test draw R < (K - t) sigma 2^32 does,
// so the decision is exactly the integer one.
constexpr float kKeepGuard = 4096.f;

// c of keep_block for a row (0 when K - t = 0, which keep_block handles apart).
__device__ __forceinline__ float keep_scale(uint64_t Kt, uint64_t R)
{
    return (Kt == 0 || R == 0) ? 0.f : (float)((double)Kt * 4294967296.0 / (double)R);
}

__device__ __forceinline__ bool keep_block(int j, uint32_t x, uint32_t draw, uint64_t cut, uint64_t Kt, uint64_t R,
                                           float c)
{
    if (pack_key(x, j) >= cut) return true;
    if (Kt == 0) return draw == 0;
    const float d = (float)draw - fmaf((float)x, c, c);
    if (d <= -kKeepGuard) return true;
    if (d >= kKeepGuard) return false;
    return cmp_mul_shift32(draw, R, Kt * ((uint64_t)x + 1)) < 0;
}

// Horvitz-Thompson weight 2^32 / theta of kept block j (an fp64 division,
// rounded to fp32); inv_r ~ 1/R for the exact ceiling of theta.
__device__ __forceinline__ float kept_weight(int j, uint32_t x, uint64_t cut, uint64_t Kt, uint64_t R, double inv_r)
{
    uint64_t th;
    if (pack_key(x, j) >= cut) {
        th = kOne;
    } else if (Kt == 0) {
        th = 1;
    } else {
        const uint64_t xx = Kt * ((uint64_t)x + 1);
        th = (xx >= R) ? kOne : ceil_ratio_shift32(xx, R, inv_r);
        th = th < 1 ? 1 : (th > kOne ? kOne : th);
    }
    return (float)(4294967296.0 / (double)th);
}

template <typename T> __device__ __forceinline__ T wave_sum_t(T x)
{
    return wave_allreduce(x, [](T a, T b) { return a + b; });
}

// Maximum over the 64 lanes of a wavefront.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x)
{
    return wave_allreduce(x, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
template <typename T> __device__ __forceinline__ T wave_incl_scan(T x, int /*lane*/)
{
    return wave_incl_scan_dpp(x);
}

// Per-row result of the chunked path for rows of more than kChunkBlocks blocks
// (below): the stopping point t, R and the cut key, or a request that the
// whole-row kernel take the row.
struct ChunkRowState {
    uint64_t R, cut;
    int32_t t, fallback;
    int32_t pad[2];
};

template <int W, int STEPS>   // wavefronts per workgroup, quad steps per thread: rows of up to 256 W STEPS blocks
__global__ __launch_bounds__(64 * W) void sample_topk_kernel(const float *__restrict__ scores, int H, int NBq, int NB,
                                                          int K, uint64_t seed, uint32_t h0, uint32_t b0, int cap, int P,
                                                          int32_t *__restrict__ idx, int32_t *__restrict__ cnt,
                                                          float *__restrict__ w,
                                                          const ChunkRowState *__restrict__ only)
{
    // with `only`, this kernel takes just the rows the chunked path handed over
    if (only && !only[blockIdx.x].fallback) return;
    constexpr int NT = 64 * W;
    extern __shared__ __align__(16) char dyn[];
    uint64_t *top = reinterpret_cast<uint64_t *>(dyn);                          // P keys
    __shared__ uint32_t red[2][W][4];
    __shared__ __align__(16) int hist[W][256];
    // the fast top's candidates share the histograms' space (the radix select
    // that uses them runs only when the candidates did not fit)
    uint64_t *const cand = reinterpret_cast<uint64_t *>(&hist[0][0]);
    static_assert(sizeof(hist) >= kCandMax * sizeof(uint64_t), "candidates fit in the histogram space");
    __shared__ int sel_s[3];
    __shared__ uint64_t ured[W];
    __shared__ uint32_t mm_s[2][W];
    __shared__ int wtot[W];
    __shared__ int top_n, t_s;
    __shared__ uint64_t r_s, cut_s;
    __shared__ uint32_t lmax_s[NT];   // largest sigma - 1 of each thread's blocks
    __shared__ uint32_t lo_s;
    __shared__ int cand_n;
    __shared__ uint64_t top2_s[2][W];   // each wavefront's two largest packed keys

    const int row = blockIdx.x;
    const int qb = row % NBq, h = (row / NBq) % H, b = row / (NBq * H);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *srow = scores + (long)row * NB;
    int32_t *irow = idx + (long)row * cap;
    float *wrow = w + (long)row * cap;

    const int NB4 = (NB + 3) / 4;
    const int Qw = ((NB4 + W - 1) / W + 63) / 64 * 64;   // quads per wavefront
    const int steps = Qw / 64;
    const int q0 = wave * Qw;
    auto quad = [&](int k) __attribute__((always_inline)) { return q0 + 64 * k + lane; };   // valid if < NB4
    // sigma - 1 of this thread's quads, quad(k) in xr[k] (zero past the row): every
    // pass below reads registers, and the LDS holds only the sorted top
    uint4 xr[STEPS];
#pragma unroll
    for (int k = 0; k < STEPS; ++k) xr[k] = make_uint4(0, 0, 0, 0);

    // 1. fixed-point scores, row total, min and max of sigma - 1
    // (the scores of 8 steps are loaded before any is used, so that their
    // latencies overlap)
    uint64_t part = 0;
    uint32_t vmin = 0xFFFFFFFFu, vmax = 0;
    constexpr int kLoadBatch = 8;
    static_assert(STEPS % kLoadBatch == 0 || STEPS < kLoadBatch, "whole load batches");
#pragma unroll
    for (int k0 = 0; k0 < STEPS; k0 += kLoadBatch) {
        if (k0 >= steps) break;
        float sv[kLoadBatch][4];
#pragma unroll
        for (int kk = 0; kk < kLoadBatch && k0 + kk < STEPS; ++kk) {
            const int q = quad(k0 + kk);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * q + e;
                sv[kk][e] = (k0 + kk < steps && j < NB) ? srow[j] : 0.f;
            }
        }
#pragma unroll
        for (int kk = 0; kk < kLoadBatch && k0 + kk < STEPS; ++kk) {
            const int q = quad(k0 + kk);
            if (k0 + kk >= steps || q >= NB4) continue;
            uint32_t x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * q + e;
                x[e] = 0;
                if (j < NB) {
                    const uint64_t sg = fixed_point(sv[kk][e]);
                    part += sg;
                    x[e] = (uint32_t)(sg - 1);
                    vmin = min(vmin, x[e]);
                    vmax = max(vmax, x[e]);
                }
            }
            xr[k0 + kk] = make_uint4(x[0], x[1], x[2], x[3]);
        }
    }
    part = wave_sum_t<uint64_t>(part);
    lmax_s[tid] = vmax;
    vmin = wave_allreduce(vmin, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
    vmax = wave_allreduce(vmax, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
    if (lane == 0) {
        ured[wave] = part;
        mm_s[0][wave] = vmin;
        mm_s[1][wave] = vmax;
    }
    if (tid == 0) {
        top_n = 0;
        cand_n = 0;
    }
    __syncthreads();
    uint64_t total = 0;
    vmin = 0xFFFFFFFFu;
    vmax = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) {
        total += ured[i];
        vmin = min(vmin, mm_s[0][i]);
        vmax = max(vmax, mm_s[1][i]);
    }

    if (K >= NB) {   // every block capped: keep all, weight 1
        for (int j = tid; j < NB; j += NT)
            if (j < cap) {
                irow[j] = j;
                wrow[j] = 1.0f;
            }
        if (tid == 0) cnt[row] = NB < cap ? NB : cap;
        return;
    }

    // Workgroup counts of a per-block predicate at 7 pivots (16-bit fields), one barrier.
    int parity = 0;
    auto count7 = [&](auto pred) __attribute__((always_inline)) {
        uint32_t c[4] = {0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < STEPS; ++k) {
            if (k >= steps) break;
            const int q = quad(k);
            if (q >= NB4) continue;
            const uint4 xv = xr[k];
            const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * q + e;
                if (j >= NB) continue;
#pragma unroll
                for (int i = 0; i < 7; ++i) c[i >> 1] += (uint32_t)pred(xs[e], j, i) << (16 * (i & 1));
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = wave_sum_t<uint32_t>(c[i]);
        if (lane == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[parity][wave][i] = c[i];
        __syncthreads();
        int out[7];
#pragma unroll
        for (int i = 0; i < 7; ++i) {
            uint32_t s4 = 0;
#pragma unroll
            for (int v = 0; v < W; ++v) s4 += red[parity][v][i >> 1];
            out[i] = (int)((s4 >> (16 * (i & 1))) & 0xFFFFu);
        }
        parity ^= 1;
        return std::array<int, 7>{out[0], out[1], out[2], out[3], out[4], out[5], out[6]};
    };

    // the T-th largest of the threads' maxima (T <= 64 W, wavefront 0, into
    // lo_s): a lower bound on the T-th largest value, since T threads each hold
    // a block at least that large
    auto threads_bound = [&](int T) __attribute__((always_inline)) {
        if (wave == 0) {
            uint32_t a[W];
#pragma unroll
            for (int i = 0; i < W; ++i) a[i] = lmax_s[lane + 64 * i];
            uint32_t v = 0;
            for (int bit = 31; bit >= 0; --bit) {   // largest v with >= T maxima >= v
                const uint32_t c = v | (1u << bit);
                int n = 0;
#pragma unroll
                for (int i = 0; i < W; ++i) n += __popcll(__ballot(a[i] >= c));
                if (n >= T) v = c;
            }
            if (lane == 0) lo_s = v > vmin ? v : vmin;
        }
        __syncthreads();
        return lo_s;
    };

    // 2. gathers the top T into top[0 .. T), pads top[T .. PT) with 0.  For a
    // small T the blocks at or above the bound are collected first; when they
    // are few, each one's rank among them (by the packed key, which orders
    // sigma descending and index ascending) places the top T directly, sorted.
    // Otherwise the radix select below finds the T-th value and the top is
    // gathered unsorted.
    auto gather_top = [&](int T, int PT) __attribute__((always_inline)) {
        if (T <= kFastTop) {
            const uint32_t lo = threads_bound(T);
#pragma unroll
            for (int k = 0; k < STEPS; ++k) {
                if (k >= steps) break;
                const int q = quad(k);
                const uint4 xv = xr[k];
                const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 4 * q + e;
                    const bool sel = q < NB4 && j < NB && xs[e] >= lo;
                    const uint64_t bal = __ballot(sel);
                    if (bal) {
                        int base = 0;
                        if (lane == __builtin_ctzll(bal)) base = atomicAdd(&cand_n, __popcll(bal));
                        base = lane_value(base, __builtin_ctzll(bal));
                        const int at = base + __popcll(bal & ((1ull << lane) - 1));
                        if (sel && at < kCandMax) cand[at] = pack_key(xs[e], j);
                    }
                }
            }
            __syncthreads();
            const int C = cand_n;
            if (C <= kCandMax) {
                for (int i = tid; i < C; i += NT) {
                    const uint64_t key = cand[i];
                    int rank = 0;
                    for (int m = 0; m < C; ++m) rank += cand[m] > key;
                    if (rank < T) top[rank] = key;
                }
                for (int i = T + tid; i < PT; i += NT) top[i] = 0;
                __syncthreads();
                return;
            }
        }
        // v: the T-th largest sigma - 1; need: how many blocks equal to v are in the top; n_eq: blocks equal to v
        uint32_t v;
        int need, n_eq;
        {
            // shortcut: fewer than T blocks above the minimum (rows whose scores mostly underflow)
            int above = 0;
#pragma unroll
            for (int k = 0; k < STEPS; ++k) {
                if (k >= steps) break;
                const int q = quad(k);
                if (q >= NB4) continue;
                const uint4 xv = xr[k];
                const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) above += (4 * q + e < NB) && xs[e] > vmin;
            }
            above = wave_sum_t<int>(above);
            if (lane == 0) wtot[wave] = above;
            __syncthreads();
            above = 0;
#pragma unroll
            for (int i = 0; i < W; ++i) above += wtot[i];
            __syncthreads();
            if (above < T) {
                v = vmin;
                need = T - above;
                n_eq = NB - above;
            } else {
                // blocks below the threads' bound are never counted
                const uint32_t lo = T <= NT ? threads_bound(T) : vmin;
                // radix select over [lo, vmax], 8 bits per pass from the top of the range
                uint32_t base = lo;
                int bits = 0;
                while (bits < 32 && ((uint64_t)(vmax - lo) >> bits) != 0) ++bits;   // range < 2^bits
                int rem = T;   // blocks still needed from the current range [base, base + 2^bits)
                int cnt_bin = 0;
                for (;;) {
                    const int shift = bits > 8 ? bits - 8 : 0;
                    hist[wave][lane] = 0;
                    hist[wave][lane + 64] = 0;
                    hist[wave][lane + 128] = 0;
                    hist[wave][lane + 192] = 0;
                    __syncthreads();
#pragma unroll
                    for (int k = 0; k < STEPS; ++k) {
                        if (k >= steps) break;
                        const int q = quad(k);
                        const uint4 xv = xr[k];
                        const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint64_t off = (uint64_t)xs[e] - base;
                            const bool in = q < NB4 && 4 * q + e < NB && xs[e] >= base && (off >> bits) == 0;
                            const int bin = in ? (int)(off >> shift) : -1;
                            // one atomic per distinct bin among the wavefront's blocks
                            uint64_t pending = __ballot(in);
                            while (pending) {
                                const int leader = __builtin_ctzll(pending);
                                const int b0 = __builtin_amdgcn_readlane(bin, leader);
                                const uint64_t same = __ballot(bin == b0) & pending;
                                if (lane == leader) atomicAdd(&hist[wave][b0], (int)__popcll(same));
                                pending &= ~same;
                            }
                        }
                    }
                    __syncthreads();
                    const int bb = 255 - tid;   // bins from the top (the first 256 threads)
                    int c = 0;
                    if (bb >= 0)
#pragma unroll
                        for (int v = 0; v < W; ++v) c += hist[v][bb];
                    const int incl = wave_incl_scan<int>(c, lane);
                    if (lane == 63) wtot[wave] = incl;
                    __syncthreads();
                    int before = incl - c;
                    for (int i = 0; i < wave; ++i) before += wtot[i];
                    if (before < rem && rem <= before + c) {
                        sel_s[0] = bb;
                        sel_s[1] = rem - before;
                        sel_s[2] = c;
                    }
                    __syncthreads();
                    base += (uint32_t)sel_s[0] << shift;
                    rem = sel_s[1];
                    cnt_bin = sel_s[2];
                    bits = shift;
                    __syncthreads();   // sel_s and wtot are rewritten by the next pass
                    if (shift == 0) break;
                }
                v = base;
                need = rem;
                n_eq = cnt_bin;
            }
        }
        int jcut = NB;                          // those with index < jcut
        if (n_eq > need) {                      // more ties at v than room: the lowest indices
            int jl = 0, jh = NB;                // count(eq, j < jl) < need <= count(eq, j < jh)
            while (jh - jl > 1) {
                int piv[7];
#pragma unroll
                for (int i = 0; i < 7; ++i) piv[i] = jl + (int)(((int64_t)(jh - jl) * (i + 1)) / 8);
                const auto c = count7([&](uint32_t x, int j, int i) { return x == v && j < piv[i]; });
                int njl = jl, njh = jh;
#pragma unroll
                for (int i = 0; i < 7; ++i) {
                    if (c[i] < need) njl = max(njl, piv[i]);
                    else njh = min(njh, piv[i]);
                }
                jl = njl;
                jh = njh;
            }
            jcut = jh;
        }
#pragma unroll
        for (int k = 0; k < STEPS; ++k) {
            if (k >= steps) break;
            const int q = quad(k);
            const uint4 xv = xr[k];
            const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * q + e;
                const bool sel = q < NB4 && j < NB && (xs[e] > v || (xs[e] == v && j < jcut));
                const uint64_t bal = __ballot(sel);
                if (bal) {
                    int base = 0;
                    if (lane == __builtin_ctzll(bal)) base = atomicAdd(&top_n, __popcll(bal));
                    base = lane_value(base, __builtin_ctzll(bal));
                    if (sel) top[base + __popcll(bal & ((1ull << lane) - 1))] = pack_key(xs[e], j);
                }
            }
        }
        for (int i = T + tid; i < PT; i += NT) top[i] = 0;   // below every real key (or equal, decoding alike)
        __syncthreads();
    };

    // The stopping point is 1 (only the top block forced) exactly when K = 1 or
    // (K - 1) sigma_(2) < total - sigma_(1): the two largest keys of the row
    // decide it, and the top is gathered only otherwise.
    int t = 0;
    bool two_key = false;
    uint64_t R1 = 0, cut1 = 0;
    {
        uint64_t k1 = 0, k2 = 0;   // this thread's largest and second largest keys
#pragma unroll
        for (int k = 0; k < STEPS; ++k) {
            if (k >= steps) break;
            const int q = quad(k);
            if (q >= NB4) continue;
            const uint32_t xs[4] = {xr[k].x, xr[k].y, xr[k].z, xr[k].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * q + e;
                if (j >= NB) continue;
                const uint64_t kk = pack_key(xs[e], j);
                if (kk > k1) {
                    k2 = k1;
                    k1 = kk;
                } else if (kk > k2) {
                    k2 = kk;
                }
            }
        }
        const uint64_t w1 = wave_max_u64(k1);
        const uint64_t w2 = wave_max_u64(k1 == w1 ? k2 : k1);
        if (lane == 0) {
            top2_s[0][wave] = w1;
            top2_s[1][wave] = w2;
        }
        __syncthreads();
        uint64_t m1 = 0, m2 = 0;   // keys are distinct, so the second is the largest one below the first
#pragma unroll
        for (int i = 0; i < W; ++i) m1 = top2_s[0][i] > m1 ? top2_s[0][i] : m1;
#pragma unroll
        for (int i = 0; i < W; ++i)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const uint64_t c = top2_s[r][i];
                if (c < m1 && c > m2) m2 = c;
            }
        const uint64_t s1 = (m1 >> kKeyIdxBits) + 1, s2 = (m2 >> kKeyIdxBits) + 1;   // NB >= 2 here
        if (K == 1 || (uint64_t)(K - 1) * s2 < total - s1) {
            t = 1;
            two_key = true;
            R1 = total - s1;
            cut1 = m1;
        }
    }
    if (t == 0) {   // fast path: the top min(K, 64), sorted and scanned by wavefront 0
        const int T = min(K, kFastTop);
        gather_top(T, kFastTop);
        if (wave == 0) {
            uint64_t key = top[lane];
#pragma unroll
            for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
                for (int stride = size >> 1; stride > 0; stride >>= 1) {
                    const uint64_t other = __shfl_xor(key, stride, 64);
                    const bool desc = (lane & size) == 0, lower = (lane & stride) == 0;
                    const uint64_t mx = key > other ? key : other, mn = key > other ? other : key;
                    key = (lower == desc) ? mx : mn;
                }
            const uint64_t sg = lane < T ? (key >> kKeyIdxBits) + 1 : 0;
            const uint64_t incl = wave_incl_scan<uint64_t>(sg, lane);
            const bool fail = lane >= 1 && lane < T && (uint64_t)(K - lane) * sg < total - (incl - sg);
            const uint64_t fb = __ballot(fail);
            int tt = fb ? __builtin_ctzll(fb) : T;
            const bool found = tt < T || T == K;
            if (found) {
                const uint64_t r = total - lane_value(incl, tt - 1);
                const uint64_t c = lane_value(key, tt - 1);
                if (lane == 0) {
                    r_s = r;
                    cut_s = c;
                }
            }
            if (lane == 0) t_s = found ? tt : 0;
        }
        __syncthreads();
        t = t_s;
    }
    if (t == 0) {   // 64 or more blocks capped: the top K, sorted by the workgroup
        if (tid == 0) top_n = 0;
        __syncthreads();
        int PT = 1;
        while (PT < K) PT <<= 1;
        gather_top(K, PT);
        for (int size = 2; size <= PT; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = tid; i < PT / 2; i += NT) {
                    const int a = 2 * i - (i & (stride - 1));
                    const int c = a + stride;
                    const bool desc = ((a & size) == 0);
                    const uint64_t x = top[a], y = top[c];
                    if ((x < y) == desc) {
                        top[a] = y;
                        top[c] = x;
                    }
                }
                __syncthreads();
            }
        }
        // first failure at a position 1 .. K-1, else K
        if (tid == 0) t_s = K;
        const int qn = (K + NT - 1) / NT;
        const int p0 = min(K, tid * qn), p1 = min(K, p0 + qn);
        uint64_t local = 0;
        for (int p = p0; p < p1; ++p) local += (top[p] >> kKeyIdxBits) + 1;
        const uint64_t wincl = wave_incl_scan<uint64_t>(local, lane);
        if (lane == 63) ured[wave] = wincl;
        __syncthreads();
        uint64_t pre = wincl - local;
        for (int i = 0; i < wave; ++i) pre += ured[i];
        const uint64_t pre0 = pre;
        for (int p = p0; p < p1; ++p) {
            const uint64_t sg = (top[p] >> kKeyIdxBits) + 1;
            if (p >= 1 && (uint64_t)(K - p) * sg < total - pre) {
                atomicMin(&t_s, p);
                break;
            }
            pre += sg;
        }
        __syncthreads();
        t = t_s;
        pre = pre0;
        for (int p = p0; p < p1; ++p) {
            const uint64_t sg = (top[p] >> kKeyIdxBits) + 1;
            if (p == t - 1) {
                r_s = total - (pre + sg);
                cut_s = top[p];
            }
            pre += sg;
        }
        __syncthreads();
    }
    const uint64_t R = two_key ? R1 : r_s, cut = two_key ? cut1 : cut_s;
    const uint64_t Kt = (uint64_t)(K - t);   // >= 0 since t <= K
    const float keep_c = keep_scale(Kt, R);

    // 4. keep decisions (4 bits per quad step), then the compaction in index order
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    uint32_t bits[(STEPS + 7) / 8] = {};
    int mine = 0;
#pragma unroll
    for (int k = 0; k < STEPS; ++k) {
        const int q = quad(k);
        if (k < steps && q < NB4) {
            const uint4 r = philox4x32_10(make_uint4((uint32_t)q, (uint32_t)qb, h0 + (uint32_t)h, b0 + (uint32_t)b), k0, k1);
            const uint32_t draw[4] = {r.x, r.y, r.z, r.w};
            const uint32_t xs[4] = {xr[k].x, xr[k].y, xr[k].z, xr[k].w};
            uint32_t nib = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * q + e;
                if (j < NB) nib |= (uint32_t)keep_block(j, xs[e], draw[e], cut, Kt, R, keep_c) << e;
            }
            bits[k >> 3] |= nib << (4 * (k & 7));
            mine += __popc(nib);
        }
    }
    mine = wave_sum_t<int>(mine);
    if (lane == 0) wtot[wave] = mine;
    __syncthreads();
    int running = 0, kept_total = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) {
        if (i < wave) running += wtot[i];
        kept_total += wtot[i];
    }
    const double inv_r = R > 0 ? 1.0 / (double)R : 0.0;
    auto weight_of = [&](int j, uint32_t x) __attribute__((always_inline)) {
        return kept_weight(j, x, cut, Kt, R, inv_r);
    };
    // Positions in index order; the kept indices go to LDS (the space of the
    // sorted top, no longer needed), and all threads then form the weights of
    // consecutive positions: balanced work and coalesced stores.  A list
    // longer than that space is written directly, each thread its own blocks.
    const int n_out = kept_total < cap ? kept_total : cap;
    uint32_t *const lst = reinterpret_cast<uint32_t *>(top);   // P indices, then their sigma - 1
    const bool staged = n_out <= P;
#pragma unroll
    for (int k = 0; k < STEPS; ++k) {
        if (k < steps) {
            const uint32_t nib = (bits[k >> 3] >> (4 * (k & 7))) & 15u;
            const int c = __popc(nib);
            const int incl = wave_incl_scan<int>(c, lane);
            int pos = running + incl - c;
            running += lane_value(incl, 63);
            const int q = quad(k);
            const uint32_t xs[4] = {xr[k].x, xr[k].y, xr[k].z, xr[k].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if ((nib >> e) & 1u) {
                    const int j = 4 * q + e;
                    if (pos < cap) {
                        if (staged) {
                            lst[pos] = (uint32_t)j;
                            lst[P + pos] = xs[e];
                        } else {
                            irow[pos] = j;
                            wrow[pos] = weight_of(j, xs[e]);
                        }
                    }
                    ++pos;
                }
            }
        }
    }
    if (staged) {
        __syncthreads();
        for (int p = tid; p < n_out; p += NT) {
            const int j = (int)lst[p];
            irow[p] = j;
            wrow[p] = weight_of(j, lst[P + p]);
        }
    }
    if (tid == 0) cnt[row] = kept_total < cap ? kept_total : cap;
}

// ---------------------------------------------------------------------------
// Rows of more than kChunkBlocks blocks (4-token key blocks beyond 32K tokens:
// 29,700 at the 118,800-token layer) are split into chunks of kChunkBlocks
// consecutive blocks, one workgroup each, so that sigma always fits in
// registers and the row is spread over several CUs.  The integer decisions are
// exactly those of the whole-row kernel above:
//   A  per chunk: sigma - 1 of its blocks, their total, and the chunk's top 64
//      packed keys (the blocks at or above the 64th largest of the threads'
//      maxima, ranked among themselves);
//   B  per row: the total, the row's top 64 (a bitonic sort of the chunks'
//      tops), and the stopping point t scanned over it (positions 1 .. 63):
//      R and the cut key.  A row whose stopping point lies past the top 64
//      (64 or more blocks capped), or a chunk with more than kCandMax blocks at
//      or above its bound (many ties), is handed to the whole-row kernel;
//   C  per chunk: the draws and keep decisions, the kept blocks compacted in
//      index order into the row's list at the chunk's own offset c * kChunkBlocks
//      (the list holds NB entries, so every chunk has room), with their weights;
//   D  per row: the chunks' lists moved down to close the gaps, and the count.
// Chunk c holds blocks [c kChunkBlocks, min(NB, (c + 1) kChunkBlocks)); thread
// (wavefront w, lane l) of its workgroup (8 wavefronts) holds the quads
// 256 w + 64 k + l, k = 0 .. 3, as the whole-row kernel lays them out.
// ---------------------------------------------------------------------------
constexpr int kChunkBlocks = 8192;
constexpr int kChunkWaves = 8;                            // wavefronts per chunk workgroup
constexpr int kChunkThreads = 64 * kChunkWaves;
constexpr int kChunkSteps = kChunkBlocks / 4 / kChunkThreads;   // quad steps per thread
constexpr int kMaxChunks = kMaxFineBlocks / kChunkBlocks;
constexpr int kChunkTop = 64;

__device__ __forceinline__ int chunk_quad(int wave, int k, int lane)
{
    return (kChunkBlocks / 4 / kChunkWaves) * wave + 64 * k + lane;
}

// sigma - 1 of this thread's blocks of chunk c (0 past the row), and the thread's
// total, minimum and maximum over its valid blocks.
__device__ __forceinline__ void load_chunk(const float *__restrict__ srow, int NB, int c, int wave, int lane,
                                           uint4 xr[kChunkSteps], uint64_t &part, uint32_t &vmax)
{
    const int jb = c * kChunkBlocks;
    float sv[kChunkSteps][4];
    if ((NB & 3) == 0) {   // rows of whole quads start 16-byte aligned: one load per quad
#pragma unroll
        for (int k = 0; k < kChunkSteps; ++k) {
            const int j0 = jb + 4 * chunk_quad(wave, k, lane);
            const float4 v = j0 < NB ? *reinterpret_cast<const float4 *>(srow + j0) : make_float4(0, 0, 0, 0);
            sv[k][0] = v.x;
            sv[k][1] = v.y;
            sv[k][2] = v.z;
            sv[k][3] = v.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < kChunkSteps; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = jb + 4 * chunk_quad(wave, k, lane) + e;
                sv[k][e] = j < NB ? srow[j] : 0.f;
            }
    }
    part = 0;
    vmax = 0;
#pragma unroll
    for (int k = 0; k < kChunkSteps; ++k) {
        uint32_t x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = jb + 4 * chunk_quad(wave, k, lane) + e;
            x[e] = 0;
            if (j < NB) {
                const uint64_t sg = fixed_point(sv[k][e]);
                part += sg;
                x[e] = (uint32_t)(sg - 1);
                vmax = max(vmax, x[e]);
            }
        }
        xr[k] = make_uint4(x[0], x[1], x[2], x[3]);
    }
}

// A: chunk totals and tops.  ctot [rows][nc], ctop [rows][nc][64] (descending,
// 0-padded), cflag [rows][nc] (1: too many candidates for the direct ranking).
__global__ __launch_bounds__(kChunkThreads) void sample_chunk_top_kernel(const float *__restrict__ scores, int NB, int nc,
                                                               uint64_t *__restrict__ ctot, uint64_t *__restrict__ ctop,
                                                               int32_t *__restrict__ cflag)
{
    __shared__ uint32_t lmax_s[kChunkThreads];
    __shared__ __align__(16) uint64_t cand[kCandMax + 8];   // + padding read by the ranking's 16-byte reads
    __shared__ uint64_t ured[kChunkWaves];
    __shared__ uint32_t lo_s;
    __shared__ int cand_n;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = blockIdx.x % nc;
    const long row = blockIdx.x / nc;
    const long item = row * nc + c;
    const int jb = c * kChunkBlocks;
    uint4 xr[kChunkSteps];
    uint64_t part;
    uint32_t vmax;
    load_chunk(scores + row * NB, NB, c, wave, lane, xr, part, vmax);
    part = wave_sum_t<uint64_t>(part);
    if (lane == 0) ured[wave] = part;
    lmax_s[tid] = vmax;
    if (tid == 0) cand_n = 0;
    __syncthreads();
    // the 64th largest of the threads' maxima bounds the chunk's 64th largest
    // value from below (threads without blocks report 0, which only lowers it)
    if (wave == 0) {
        uint32_t a[kChunkWaves], mn = 0xFFFFFFFFu, mx = 0;
#pragma unroll
        for (int i = 0; i < kChunkWaves; ++i) {
            a[i] = lmax_s[lane + 64 * i];
            mn = min(mn, a[i]);
            mx = max(mx, a[i]);
        }
        mn = wave_allreduce(mn, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
        mx = wave_allreduce(mx, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
        // the answer lies in [mn, mx]: only the bits below their common prefix are searched
        const uint32_t diff = mn ^ mx;
        const int top = diff ? 31 - __clz(diff) : -1;
        uint32_t v = top >= 0 ? (mx & ~((2u << top) - 1u)) : mx;
        if (top == 31) v = 0;
        for (int bit = top; bit >= 0; --bit) {
            const uint32_t cnd = v | (1u << bit);
            int n = 0;
#pragma unroll
            for (int i = 0; i < kChunkWaves; ++i) n += __popcll(__ballot(a[i] >= cnd));
            if (n >= kChunkTop) v = cnd;
        }
        if (lane == 0) lo_s = v;
    }
    __syncthreads();
    const uint32_t lo = lo_s;
#pragma unroll
    for (int k = 0; k < kChunkSteps; ++k) {
        const int q = chunk_quad(wave, k, lane);
        const uint32_t xs[4] = {xr[k].x, xr[k].y, xr[k].z, xr[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = jb + 4 * q + e;
            const bool sel = j < NB && xs[e] >= lo;
            const uint64_t bal = __ballot(sel);
            if (bal) {
                int base = 0;
                if (lane == __builtin_ctzll(bal)) base = atomicAdd(&cand_n, __popcll(bal));
                base = lane_value(base, __builtin_ctzll(bal));
                const int at = base + __popcll(bal & ((1ull << lane) - 1));
                if (sel && at < kCandMax) cand[at] = pack_key(xs[e], j);
            }
        }
    }
    __syncthreads();
    const int C = cand_n;
    if (tid == 0) {
        uint64_t t = 0;
#pragma unroll
        for (int i = 0; i < kChunkWaves; ++i) t += ured[i];
        ctot[item] = t;
        cflag[item] = C > kCandMax ? 1 : 0;
    }
    if (C > kCandMax) return;
    uint64_t *out = ctop + item * kChunkTop;
    // rank of each candidate among all of them (keys are distinct: each rank is
    // taken once); the candidates are read eight at a time in 16-byte pieces,
    // all lanes at the same address, and the padding past C holds zeros, which
    // rank below every key
    if (tid < 8) cand[C + tid] = 0;
    __syncthreads();
    for (int i = tid; i < C; i += kChunkThreads) {
        const uint64_t key = cand[i];
        int rank = 0;
        for (int m = 0; m < C; m += 8) {
            const uint4 *p = reinterpret_cast<const uint4 *>(cand + m);
            const uint4 a = p[0], b = p[1], c4 = p[2], d = p[3];
            auto gt = [&](uint32_t lo, uint32_t hi) { return ((uint64_t)hi << 32 | lo) > key ? 1 : 0; };
            rank += gt(a.x, a.y) + gt(a.z, a.w) + gt(b.x, b.y) + gt(b.z, b.w) + gt(c4.x, c4.y) + gt(c4.z, c4.w) +
                    gt(d.x, d.y) + gt(d.z, d.w);
        }
        if (rank < kChunkTop) out[rank] = key;
    }
    for (int i = C + tid; i < kChunkTop; i += kChunkThreads) out[i] = 0;
}

// B: one wavefront per row.
__global__ __launch_bounds__(64) void sample_chunk_merge_kernel(const uint64_t *__restrict__ ctot,
                                                                const uint64_t *__restrict__ ctop,
                                                                const int32_t *__restrict__ cflag, int nc, int K,
                                                                ChunkRowState *__restrict__ state)
{
    constexpr int kKeys = kMaxChunks * kChunkTop;
    __shared__ uint64_t keys[kKeys];
    const int lane = threadIdx.x;
    const long row = blockIdx.x;
    uint64_t total = 0;
    int overflow = 0;
    for (int c = 0; c < nc; ++c) {
        total += ctot[row * nc + c];
        overflow |= cflag[row * nc + c];
    }
    ChunkRowState st = {0, 0, 0, 1, {0, 0}};
    if (overflow) {
        if (lane == 0) state[row] = st;
        return;
    }
    for (int i = lane; i < kKeys; i += 64) keys[i] = i < nc * kChunkTop ? ctop[row * nc * kChunkTop + i] : 0;
    __syncthreads();
    // bitonic sort, descending: each step compares kKeys / 2 pairs, two per lane
    for (int size = 2; size <= kKeys; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = lane; i < kKeys / 2; i += 64) {
                const int a = 2 * i - (i & (stride - 1)), b = a + stride;
                const bool desc = (a & size) == 0;
                const uint64_t x = keys[a], y = keys[b];
                if ((x < y) == desc) {
                    keys[a] = y;
                    keys[b] = x;
                }
            }
            __syncthreads();
        }
    // the stopping point: the first position p in 1 .. T-1 where (K - p) sigma_p
    // < total - (sigma_0 + .. + sigma_{p-1}); none and T = K: t = K
    const int T = min(K, kChunkTop);
    const uint64_t key = keys[lane];
    const uint64_t sg = lane < T ? (key >> kKeyIdxBits) + 1 : 0;
    const uint64_t incl = wave_incl_scan<uint64_t>(sg, lane);
    const bool fail = lane >= 1 && lane < T && (uint64_t)(K - lane) * sg < total - (incl - sg);
    const uint64_t fb = __ballot(fail);
    const int tt = fb ? __builtin_ctzll(fb) : T;
    const uint64_t r_inc = lane_value(incl, tt - 1);
    const uint64_t cut = lane_value(key, tt - 1);
    if (lane == 0) {
        if (tt < T || T == K) {
            st.R = total - r_inc;
            st.cut = cut;
            st.t = tt;
            st.fallback = 0;
        }
        state[row] = st;
    }
}

// C: draws, keep decisions and the chunk's list at offset c * kChunkBlocks.
__global__ __launch_bounds__(kChunkThreads) void sample_chunk_draw_kernel(const float *__restrict__ scores, int H, int NBq, int NB,
                                                                int nc, int K, uint64_t seed, uint32_t h0, uint32_t b0,
                                                                int cap, const ChunkRowState *__restrict__ state,
                                                                int32_t *__restrict__ ccnt, int32_t *__restrict__ idx,
                                                                float *__restrict__ w)
{
    // the first kChunkStage kept blocks (index and sigma - 1), whose weights all
    // threads then form over consecutive positions: a weight takes an fp64
    // division, and formed where each block is found it would run, divergent,
    // for almost every block slot of almost every wavefront
    constexpr int kChunkStage = 2048;
    __shared__ int32_t stage_j[kChunkStage];
    __shared__ uint32_t stage_x[kChunkStage];
    __shared__ int wtot[kChunkWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = blockIdx.x % nc;
    const long row = blockIdx.x / nc;
    const ChunkRowState st = state[row];
    if (st.fallback) return;   // uniform over the workgroup
    const int qb = (int)(row % NBq), h = (int)((row / NBq) % H), b = (int)(row / ((long)NBq * H));
    const int jb = c * kChunkBlocks;
    uint4 xr[kChunkSteps];
    uint64_t part;
    uint32_t vmax;
    load_chunk(scores + row * NB, NB, c, wave, lane, xr, part, vmax);
    const uint64_t R = st.R, cut = st.cut, Kt = (uint64_t)(K - st.t);
    const float keep_c = keep_scale(Kt, R);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    uint32_t bits = 0;   // 4 bits per quad step
    int mine = 0;
#pragma unroll
    for (int k = 0; k < kChunkSteps; ++k) {
        const int q = jb / 4 + chunk_quad(wave, k, lane);   // the row's quad index
        if (4 * q < NB) {
            const uint4 r = philox4x32_10(make_uint4((uint32_t)q, (uint32_t)qb, h0 + (uint32_t)h, b0 + (uint32_t)b),
                                          k0, k1);
            const uint32_t draw[4] = {r.x, r.y, r.z, r.w};
            const uint32_t xs[4] = {xr[k].x, xr[k].y, xr[k].z, xr[k].w};
            uint32_t nib = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * q + e;
                if (j < NB) nib |= (uint32_t)keep_block(j, xs[e], draw[e], cut, Kt, R, keep_c) << e;
            }
            bits |= nib << (4 * k);
            mine += __popc(nib);
        }
    }
    mine = wave_sum_t<int>(mine);
    if (lane == 0) wtot[wave] = mine;
    __syncthreads();
    int running = 0, kept = 0;
#pragma unroll
    for (int i = 0; i < kChunkWaves; ++i) {
        if (i < wave) running += wtot[i];
        kept += wtot[i];
    }
    const double inv_r = R > 0 ? 1.0 / (double)R : 0.0;
    int32_t *irow = idx + row * cap + jb;
    float *wrow = w + row * cap + jb;
#pragma unroll
    for (int k = 0; k < kChunkSteps; ++k) {
        const uint32_t nib = (bits >> (4 * k)) & 15u;
        const int cn = __popc(nib);
        const int incl = wave_incl_scan<int>(cn, lane);
        int pos = running + incl - cn;
        running += lane_value(incl, 63);
        const int q = jb / 4 + chunk_quad(wave, k, lane);
        const uint32_t xs[4] = {xr[k].x, xr[k].y, xr[k].z, xr[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if ((nib >> e) & 1u) {
                const int j = 4 * q + e;
                if (pos < kChunkStage) {
                    stage_j[pos] = j;
                    stage_x[pos] = xs[e];
                } else {   // a chunk keeping more than the stage holds: formed here
                    irow[pos] = j;
                    wrow[pos] = kept_weight(j, xs[e], cut, Kt, R, inv_r);
                }
                ++pos;
            }
        }
    }
    __syncthreads();
    const int staged = kept < kChunkStage ? kept : kChunkStage;
    for (int p = tid; p < staged; p += kChunkThreads) {
        const int j = stage_j[p];
        irow[p] = j;
        wrow[p] = kept_weight(j, stage_x[p], cut, Kt, R, inv_r);
    }
    if (tid == 0) ccnt[row * nc + c] = kept;
}

// D: close the gaps between the chunks' lists (each moves down, in order, a
// tile at a time: a tile's destination never reaches a later tile's source).
__global__ __launch_bounds__(256) void sample_chunk_compact_kernel(const ChunkRowState *__restrict__ state,
                                                                   const int32_t *__restrict__ ccnt, int nc, int cap,
                                                                   int32_t *__restrict__ idx, int32_t *__restrict__ cnt,
                                                                   float *__restrict__ w)
{
    constexpr int kPer = 4;
    const int tid = threadIdx.x;
    const long row = blockIdx.x;
    if (state[row].fallback) return;
    int32_t *irow = idx + row * cap;
    float *wrow = w + row * cap;
    int off = ccnt[row * nc];
    for (int c = 1; c < nc; ++c) {
        const int n = ccnt[row * nc + c], src = c * kChunkBlocks;
        if (off != src) {
            for (int i0 = 0; i0 < n; i0 += 256 * kPer) {
                int32_t jv[kPer];
                float wv[kPer];
#pragma unroll
                for (int r = 0; r < kPer; ++r) {
                    const int i = i0 + r * 256 + tid;
                    jv[r] = i < n ? irow[src + i] : 0;
                    wv[r] = i < n ? wrow[src + i] : 0.f;
                }
                __syncthreads();
#pragma unroll
                for (int r = 0; r < kPer; ++r) {
                    const int i = i0 + r * 256 + tid;
                    if (i < n) {
                        irow[off + i] = jv[r];
                        wrow[off + i] = wv[r];
                    }
                }
                __syncthreads();
            }
        }
        off += n;
    }
    if (tid == 0) cnt[row] = off < cap ? off : cap;
}

// ---------------------------------------------------------------------------
// Rows of at most 256 blocks (128-token rows up to 32K tokens): one wavefront per row,
// four rows per workgroup, no workgroup barriers.  The wavefront keeps sigma - 1
// of its row in registers (quad 64k + lane at step k).  The two largest packed
// keys tell whether the water-filling stops right after the top block; only
// when it does not does the wavefront sort the packed keys of the whole row in
// its own LDS region (bitonic, descending) and find the stopping point with a
// scan over the sorted prefix.  It then draws, keeps and compacts in index order
// as the long-row kernel does; the decisions are the same, bit for bit.
// ---------------------------------------------------------------------------
constexpr int kWaveRowMax = 256;   // longer rows: a whole-row sort per wavefront costs more than the top-K kernel

template <int QPL>   // quads per lane: rows of up to 256 QPL blocks
__global__ __launch_bounds__(256) void sample_wave_kernel(const float *__restrict__ scores, int H, int NBq, int NB,
                                                          int K, uint64_t seed, uint32_t h0, uint32_t b0, int cap,
                                                          int rows,
                                                          int32_t *__restrict__ idx, int32_t *__restrict__ cnt,
                                                          float *__restrict__ w)
{
    constexpr int kKeys = 256 * QPL;
    __shared__ uint64_t keys_s[4][kKeys];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * 4 + wave;
    if (row >= rows) return;   // the whole wavefront: nothing below waits for other wavefronts
    uint64_t *keys = keys_s[wave];
    const int qb = row % NBq, h = (row / NBq) % H, b = row / (NBq * H);
    const float *srow = scores + (long)row * NB;
    int32_t *irow = idx + (long)row * cap;
    float *wrow = w + (long)row * cap;
    const int NB4 = (NB + 3) / 4;

    // sigma - 1 of the row (all loads in flight together) and the row total
    float sv[QPL][4];
#pragma unroll
    for (int k = 0; k < QPL; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * (64 * k + lane) + e;
            sv[k][e] = j < NB ? srow[j] : 0.f;
        }
    uint32_t x[QPL][4];
    uint64_t part = 0;
#pragma unroll
    for (int k = 0; k < QPL; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * (64 * k + lane) + e;
            x[k][e] = 0;
            if (j < NB) {
                const uint64_t sg = fixed_point(sv[k][e]);
                part += sg;
                x[k][e] = (uint32_t)(sg - 1);
            }
        }
    const uint64_t total = wave_sum_t<uint64_t>(part);

    if (K >= NB) {   // every block capped: keep all, weight 1
        for (int j = lane; j < NB && j < cap; j += 64) {
            irow[j] = j;
            wrow[j] = 1.0f;
        }
        if (lane == 0) cnt[row] = NB < cap ? NB : cap;
        return;
    }

    // The stopping point is 1 (only the top block forced) exactly when K = 1 or
    // (K - 1) sigma_(2) < total - sigma_(1): the two largest keys decide it, and
    // the sort is needed only otherwise.
    int t = K;
    uint64_t pre_t = 0, cut = 0;
    bool sorted_path = true;
    {
        uint64_t k1 = 0, k2 = 0;   // this lane's largest and second largest keys
#pragma unroll
        for (int k = 0; k < QPL; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * (64 * k + lane) + e;
                if (j < NB) {
                    const uint64_t kk = pack_key(x[k][e], j);
                    if (kk > k1) {
                        k2 = k1;
                        k1 = kk;
                    } else if (kk > k2) {
                        k2 = kk;
                    }
                }
            }
        const uint64_t m1 = wave_max_u64(k1);
        const uint64_t m2 = wave_max_u64(k1 == m1 ? k2 : k1);   // NB >= 2 here, so a real key
        const uint64_t s1 = (m1 >> kKeyIdxBits) + 1, s2 = (m2 >> kKeyIdxBits) + 1;
        if (K == 1 || (uint64_t)(K - 1) * s2 < total - s1) {
            t = 1;
            pre_t = s1;
            cut = m1;
            sorted_path = false;
        }
    }
    if (sorted_path) {
        // packed keys (sigma desc, index asc when sorted descending); padding 0 sorts last
        int P = 64;
        while (P < NB) P <<= 1;
#pragma unroll
        for (int k = 0; k < QPL; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * (64 * k + lane) + e;
                if (j < P) keys[j] = j < NB ? pack_key(x[k][e], j) : 0;
            }
        // bitonic sort of keys[0 .. P) by this wavefront: LDS operations of one
        // wavefront complete in order, so each stage sees the previous one's writes
        for (int size = 2; size <= P; size <<= 1)
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                __builtin_amdgcn_wave_barrier();
                for (int i = lane; i < P / 2; i += 64) {
                    const int a = 2 * i - (i & (stride - 1)), c = a + stride;
                    const bool desc = (a & size) == 0;
                    const uint64_t ka = keys[a], kc = keys[c];
                    if ((ka < kc) == desc) {
                        keys[a] = kc;
                        keys[c] = ka;
                    }
                }
            }
        __builtin_amdgcn_wave_barrier();

        // stopping point: the first position p >= 1 with (K - p) sigma_p < total - sum of
        // the first p, else K; R = total - sum of the first t; cut = the key at t - 1
        uint64_t before = 0;   // sum of sigma over the positions before the current chunk
        bool found = false;
        for (int c0 = 0; c0 < K && !found; c0 += 64) {
            const int p = c0 + lane;
            const uint64_t sg = p < K ? (keys[p] >> kKeyIdxBits) + 1 : 0;
            const uint64_t incl = before + wave_incl_scan<uint64_t>(sg, lane);
            const bool fail = p >= 1 && p < K && (uint64_t)(K - p) * sg < total - (incl - sg);
            const uint64_t fb = __ballot(fail);
            if (fb) {
                const int tt = __builtin_ctzll(fb);   // >= 1 in the first chunk
                t = c0 + tt;
                pre_t = tt > 0 ? lane_value(incl, tt - 1) : before;
                found = true;
            } else {
                before = lane_value(incl, 63);
            }
        }
        if (!found) pre_t = before;
        cut = keys[t - 1];
    }
    const uint64_t R = total - pre_t;
    const uint64_t Kt = (uint64_t)(K - t);
    const float keep_c = keep_scale(Kt, R);
    const double inv_r = R > 0 ? 1.0 / (double)R : 0.0;

    // draws, keep decisions and the compaction in index order
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    int base = 0;
#pragma unroll
    for (int k = 0; k < QPL; ++k) {
        const int q = 64 * k + lane;
        uint32_t nib = 0;
        if (q < NB4) {
            const uint4 r = philox4x32_10(make_uint4((uint32_t)q, (uint32_t)qb, h0 + (uint32_t)h, b0 + (uint32_t)b), k0, k1);
            const uint32_t draw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * q + e;
                if (j < NB) nib |= (uint32_t)keep_block(j, x[k][e], draw[e], cut, Kt, R, keep_c) << e;
            }
        }
        const int c = __popc(nib);
        const int incl = wave_incl_scan<int>(c, lane);
        int pos = base + incl - c;
        base += lane_value(incl, 63);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (!((nib >> e) & 1u)) continue;
            const int j = 4 * q + e;
            if (pos < cap) {
                irow[pos] = j;
                wrow[pos] = kept_weight(j, x[k][e], cut, Kt, R, inv_r);
            }
            ++pos;
        }
    }
    if (lane == 0) cnt[row] = base < cap ? base : cap;
}

}  // namespace

// Keys of the sorted top (P of them, P = 2^ceil(log2 K) when K < NB, else 1)
// followed by sigma - 1 of every block.
static int topk_pad(int NB, int K)
{
    int P = kFastTop;
    while (K < NB && P < K) P <<= 1;
    return P;
}

size_t sample_lds_bytes(int NB, int K)
{
    if (NB <= kWaveRowMax) return 0;   // the wavefront-per-row kernel: static LDS only
    return 8 * (size_t)topk_pad(NB, K);
}

// Workspace of the chunked path (rows of more than kChunkBlocks blocks with a
// budget below the row length): chunk totals, tops, flags and counts, and the
// per-row state.
struct ChunkWs {
    size_t tot, top, flag, cnt, state, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static ChunkWs chunk_ws_layout(long rows, int NB)
{
    const size_t nc = (size_t)((NB + kChunkBlocks - 1) / kChunkBlocks), items = (size_t)rows * nc;
    ChunkWs l;
    l.tot = 0;
    l.top = l.tot + align256(items * sizeof(uint64_t));
    l.flag = l.top + align256(items * kChunkTop * sizeof(uint64_t));
    l.cnt = l.flag + align256(items * sizeof(int32_t));
    l.state = l.cnt + align256(items * sizeof(int32_t));
    l.total = l.state + align256((size_t)rows * sizeof(ChunkRowState));
    return l;
}

static bool chunked_rows(int NB, int K, int cap) { return NB > kChunkBlocks && K < NB && cap >= NB; }

size_t sample_workspace_bytes(int B, int H, int NBq, int NB, int K)
{
    return chunked_rows(NB, K, NB) ? chunk_ws_layout((long)B * H * NBq, NB).total : 0;
}

hipError_t launch_sample(const float *scores, int B, int H, int NBq, int NB, int K, uint64_t seed, int h0, int b0,
                         int cap, int32_t *idx, int32_t *cnt, float *w, void *ws, hipStream_t s)
{
    const long rows = (long)B * H * NBq;
    const dim3 grid((unsigned)rows), block(256);
    if (NB > kMaxFineBlocks) return hipErrorInvalidValue;
    if (NB <= kWaveRowMax) {   // one wavefront per row
        const dim3 wgrid((unsigned)((rows + 3) / 4));
        sample_wave_kernel<1><<<wgrid, block, 0, s>>>(scores, H, NBq, NB, K, seed, (uint32_t)h0, (uint32_t)b0, cap,
                                                       (int)rows, idx, cnt, w);
        return hipGetLastError();
    }
    const size_t lds = sample_lds_bytes(NB, K);
    if (lds > kSampleLdsLimit) return hipErrorInvalidValue;
    const int P = topk_pad(NB, K);
    // rows of more than kChunkBlocks blocks: the chunked path, the whole-row
    // kernel only for the rows it hands over
    const bool chunked = chunked_rows(NB, K, cap) && ws != nullptr;
    const ChunkRowState *only = nullptr;
    if (chunked) {
        const int nc = (NB + kChunkBlocks - 1) / kChunkBlocks;
        const ChunkWs l = chunk_ws_layout(rows, NB);
        char *base = static_cast<char *>(ws);
        uint64_t *ctot = reinterpret_cast<uint64_t *>(base + l.tot);
        uint64_t *ctop = reinterpret_cast<uint64_t *>(base + l.top);
        int32_t *cflag = reinterpret_cast<int32_t *>(base + l.flag);
        ChunkRowState *state = reinterpret_cast<ChunkRowState *>(base + l.state);
        sample_chunk_top_kernel<<<dim3((unsigned)(rows * nc)), dim3(kChunkThreads), 0, s>>>(scores, NB, nc, ctot, ctop,
                                                                                         cflag);
        sample_chunk_merge_kernel<<<grid, dim3(64), 0, s>>>(ctot, ctop, cflag, nc, K, state);
        only = state;
    }
    // as few quad steps per thread as the row needs: 1 to 8 on 4 wavefronts, 8 or 16 on 8
    auto launch = [&](auto kernel, int threads) {
        // allow more than the default dynamic LDS (a host-side attribute of the current device);
        // exactly this launch's size, which with the kernel's static LDS stays within a CU's
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        kernel<<<grid, dim3(threads), lds, s>>>(scores, H, NBq, NB, K, seed, (uint32_t)h0, (uint32_t)b0, cap, P, idx,
                                                cnt, w, only);
        hipError_t r = hipGetLastError();
        if (r != hipSuccess || !chunked) return r;
        const int nc = (NB + kChunkBlocks - 1) / kChunkBlocks;
        const ChunkWs l = chunk_ws_layout(rows, NB);
        char *base = static_cast<char *>(ws);
        int32_t *ccnt = reinterpret_cast<int32_t *>(base + l.cnt);
        sample_chunk_draw_kernel<<<dim3((unsigned)(rows * nc)), dim3(kChunkThreads), 0, s>>>(
            scores, H, NBq, NB, nc, K, seed, (uint32_t)h0, (uint32_t)b0, cap, only, ccnt, idx, w);
        sample_chunk_compact_kernel<<<grid, dim3(256), 0, s>>>(only, ccnt, nc, cap, idx, cnt, w);
        return hipGetLastError();
    };
    if (NB <= 256 * 4 * 1) return launch(&sample_topk_kernel<4, 1>, 256);
    if (NB <= 256 * 4 * 2) return launch(&sample_topk_kernel<4, 2>, 256);
    if (NB <= 256 * 4 * 4) return launch(&sample_topk_kernel<4, 4>, 256);
    if (NB <= 256 * 4 * 8) return launch(&sample_topk_kernel<4, 8>, 256);
    if (NB <= 256 * 8 * 8) return launch(&sample_topk_kernel<8, 8>, 512);
    return launch(&sample_topk_kernel<8, 16>, 512);
}

}  // namespace aba
