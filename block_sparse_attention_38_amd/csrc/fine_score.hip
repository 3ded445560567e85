// fine_score.hip -- IBCS block scoring on the matrix cores, and pooling of
// 4-token key blocks (gfx950).
//
// AB-Attention page, section "Три приёма AB-Attention": every key block is
// scored by the cluster-weighted attention of the query block's centroids to
// its averaged keys (IBCS paragraph),
//     S[b', j] = sum_m w_m softmax_j(s c_m . kbar_j),
// and key/value blocks may be only 4 tokens while queries stay in 128-token
// blocks (kernel paragraph).  With 4-token blocks a query block scores N/4 key
// blocks (8190 at 32K tokens), so the centroid x pooled-key contraction is a
// real matrix product (2 * C * N/4 * D flops per query block); the same
// kernels score 128-token key blocks (NB of them per row).
//
// Precision.  Scores must stay within 1e-4 relative of an fp64 evaluation, which
// bf16 operands (2^-9) cannot give.  Both operands are split into two bf16
// parts, x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), and a logit is
//     hi_c.hi_k + hi_c.lo_k + lo_c.hi_k
// with fp32 accumulation: the dropped lo.lo term and the residuals of the
// splits are below 2^-16 of |c||kbar| per term.
//
// Layout of the work.  The softmax over j needs each centroid's maximum and
// normaliser over every key block before any score can be written, so there
// are two passes over the same contraction, with a small merge in between:
//   fine_score_kernel<D, false>  per (b, h, chunk of 256 key blocks): logits of
//       every centroid of the head against the chunk; per centroid the chunk's
//       max and sum of exponentials (log2 domain) -> partial[b,h,chunk,slot];
//   fine_merge_kernel            per (b, h, slot): M = max over chunks,
//       Z = sum over chunks; coef = w_m / Z -> stat[b,h,slot] = (M, coef);
//   fine_score_kernel<D, true>   the same logits again; per query block and key
//       block the sum over its centroids of coef * 2^(x - M) -> scores.
// A workgroup keeps the split pooled keys of its chunk in registers (4
// wavefronts x 64 key blocks, the MFMA operand of both passes) and streams the
// head's centroids through LDS in tiles of 32 slots (4 query blocks x 8
// slots; slots >= C are zero centroids with zero weight).  The stats pass uses
// S^T orientation (rows = key blocks, columns = slots: one centroid per lane,
// so its reductions over key blocks stay in the lane); the write pass uses S
// orientation (rows = slots: a query block's 8 centroids are 4 accumulator
// rows in each half of the wavefront, one permlane32 swap apart).  Both
// passes evaluate identical MFMA sequences, so every logit of the write pass
// is bitwise the one the stats pass saw and 2^(x - M) <= 1.
//
// Short rows (at most kRowMaxBlocks key blocks, e.g. the 256 128-token blocks
// of a 32K sequence) take one pass instead: row_score_kernel gives a
// workgroup one tile of 32 centroid slots and every key block of the head,
// keeps all its logits in LDS, and reduces, normalises and writes from there.
#include "aba_internal.h"

namespace aba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSlots = 8;                         // centroid slots per query block
constexpr int kTileSlots = 32;                    // slots per MFMA tile (4 query blocks)
constexpr int kTileBlocks = kTileSlots / kSlots;
constexpr int kChunk = 256;                       // key blocks per workgroup (64 per wavefront)

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Pooling: one thread per (b, h, key block, 8-element chunk of the row).  A
// 4-token block of K is 4 consecutive rows, so consecutive threads read
// consecutive 16-byte pieces of them.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void fine_pool_kernel(const T *__restrict__ k, int N, int N_pad, int NBk,
                                                        long total, float *__restrict__ kbar)
{
    constexpr int CH = D / 8;
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int c = (int)(i % CH);
    const long row = i / CH;                      // (b*H + h) * NBk + j
    const int j = (int)(row % NBk);
    const long bh = row / NBk;
    const int n = min(kFineBlock, N - j * kFineBlock);
    const T *src = k + (bh * N_pad + (long)j * kFineBlock) * D + 8 * c;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int r = 0; r < n; ++r) {
        float x[8];
        load8(src + (long)r * D, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += x[e];
    }
    const float fn = (float)n;
    float4 *dst = reinterpret_cast<float4 *>(kbar + row * D + 8 * c);
    dst[0] = make_float4(acc[0] / fn, acc[1] / fn, acc[2] / fn, acc[3] / fn);
    dst[1] = make_float4(acc[4] / fn, acc[5] / fn, acc[6] / fn, acc[7] / fn);
}

// bf16 split of eight floats: hi = bf16(x) (round to nearest even), lo = bf16(x - hi).
__device__ __forceinline__ void split8(const float x[8], bf16x8 &hi, bf16x8 &lo)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = (__bf16)x[e];
        hi[e] = h;
        lo[e] = (__bf16)(x[e] - (float)h);
    }
}

// A tile of 32 centroid slots, split: hi rows 0..31 then lo rows 32..63, D
// bf16 each.  In memory (written once per call by fine_cent_kernel) the tiles
// of a head are consecutive and unswizzled; in LDS chunk c of row r sits at
// c ^ (r % (D/8)), so the 16 rows one phase of a 128-bit read touches fall on
// different banks.  The swizzle is applied by the direct loads: each lane
// fetches the source chunk that belongs at its LDS position.
template <int D> struct CentTile {
    static constexpr int chunks = D / 8;
    static constexpr int pitch = D * 2;
    static constexpr int part = kTileSlots * pitch;          // offset of the lo rows
    static constexpr int bytes = 2 * part;                   // 16 KB at D = 128
    static constexpr int loads = bytes / 1024;               // 1 KB direct loads per tile
    static constexpr int wave_loads = loads / 4;
    static constexpr int rows_per_load = 1024 / pitch;
    static constexpr int period = chunks / rows_per_load;    // distinct per-lane offsets
};
template <int D> __device__ __forceinline__ int cent_off(int r, int c)
{
    return r * CentTile<D>::pitch + 16 * (c ^ (r & (CentTile<D>::chunks - 1)));
}

// Split centroid tiles: one thread per (b, h, tile, slot, 8-element chunk).
template <int D>
__global__ __launch_bounds__(256) void fine_cent_kernel(const float *__restrict__ cent, int NBq, int C, int NT, long total,
                                                        uint16_t *__restrict__ tiles)
{
    using T = CentTile<D>;
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int c = (int)(i % T::chunks);
    const int s = (int)((i / T::chunks) % kTileSlots);
    const long tile = i / T::chunks / kTileSlots;   // (b*H + h) * NT + ct
    const int ct = (int)(tile % NT);
    const long bh = tile / NT;
    const int qb = kTileBlocks * ct + s / kSlots, m = s % kSlots;
    float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (qb < NBq && m < C) load8(cent + ((bh * NBq + qb) * C + m) * D + 8 * c, x);
    bf16x8 hi, lo;
    split8(x, hi, lo);
    uint16_t *base = tiles + tile * (T::bytes / 2);
    *reinterpret_cast<bf16x8 *>(base + s * D + 8 * c) = hi;
    *reinterpret_cast<bf16x8 *>(base + (kTileSlots + s) * D + 8 * c) = lo;
}

template <int D, bool write>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fine_score_kernel(
    const uint16_t *__restrict__ ctiles, const float *__restrict__ kbar, const float2 *__restrict__ stat, int NBq,
    int NBk, int n_chunks, int splits, float scale_log2, float2 *__restrict__ partial, float *__restrict__ scores)
{
    using CT = CentTile<D>;
    constexpr int KS = D / 16;
    constexpr int WL = CT::wave_loads;
    // three tile slots: the tile in use and the next two, whose loads are in flight
    __shared__ __align__(16) char ring[3][CT::bytes];
    __shared__ __align__(16) float2 st_ring[3][kTileSlots];
    __shared__ float2 red[2][4][kTileSlots];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, half = lane >> 5;
    const int sp = blockIdx.x % splits;
    const int chunk = (blockIdx.x / splits) % n_chunks;
    const long bh = blockIdx.x / splits / n_chunks;
    const int NT = (NBq + kTileBlocks - 1) / kTileBlocks;   // centroid tiles of the head
    const int n_my = NT > sp ? (NT - sp + splits - 1) / splits : 0;   // tiles sp, sp + splits, ...
    const int4v rc = head_rsrc(ctiles + bh * NT * (CT::bytes / 2), NT * CT::bytes);
    const int4v rs = head_rsrc(stat + bh * NT * kTileSlots, NT * kTileSlots * (int)sizeof(float2));

    // split pooled keys of this wavefront's 64 key blocks: fragment (kt, ks) is
    // block chunk*256 + 64 wave + 32 kt + l32, elements 16 ks + 8 half .. +7
    const int j0 = chunk * kChunk + 64 * wave;
    bf16x8 khi[2][KS], klo[2][KS];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        const int j = j0 + 32 * kt + l32;
        const float *row = kbar + (bh * NBk + j) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (j < NBk) load8(row + 16 * ks + 8 * half, x);
            split8(x, khi[kt][ks], klo[kt][ks]);
        }
    }

    // direct loads of tile ct into ring slot sl: load t (wavefront w issues t =
    // w*WL .. w*WL + WL - 1) fills rows t*rows_per_load .., lane L row L / chunks of
    // them and LDS chunk L % chunks, which holds source chunk (L % chunks) ^ (row % chunks)
    int voff[CT::period];
#pragma unroll
    for (int v = 0; v < CT::period; ++v) {
        const int r = CT::rows_per_load * v + lane / CT::chunks;   // row % chunks for loads t with t % period == v
        voff[v] = (lane / CT::chunks) * CT::pitch + 16 * ((lane % CT::chunks) ^ (r & (CT::chunks - 1)));
    }
    auto issue = [&](int sl, int ct) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < WL; ++i) {
            const int t = WL * wave + i;
            load_lds16(rc, voff[t % CT::period], ct * CT::bytes + t * 1024, ring[sl] + t * 1024);
        }
        if (write && wave == 0) load_lds4(rs, 4 * lane, ct * kTileSlots * (int)sizeof(float2), (char *)st_ring[sl]);
    };
    // wait for everything but the next-next tile's loads (or for everything);
    // the statistics pass has also written its partials to LDS before the barrier
    auto wait_tile = [&](bool more) __attribute__((always_inline)) {
        if (!more) wait_loads_lds_and_sync<0>();
        else if (write && wave == 0) wait_loads_lds_and_sync<WL + 1>();
        else wait_loads_lds_and_sync<WL>();
    };

    if (n_my > 0) issue(0, sp);
    if (n_my > 1) issue(1, sp + splits);
    // settle the pooled-key loads here, once, rather than inside the loop
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(khi[kt][ks]), "v"(klo[kt][ks]));
    wait_tile(n_my > 1);

    // scores of the previous tile, stored at the start of the next iteration so that
    // the stores are older than the loads a wait must leave in flight
    float pend[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    int pend_ct = -1;
    auto flush = [&]() __attribute__((always_inline)) {
        if (!write || pend_ct < 0) return;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const int j = j0 + 32 * kt + l32;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const int qb = kTileBlocks * pend_ct + 2 * half + pp;
                if (j < NBk && qb < NBq) scores[(bh * NBq + qb) * NBk + j] = pend[kt][pp];
            }
        }
    };

    for (int i = 0; i < n_my; ++i) {
        const int ct = sp + i * splits;
        const int sl = i % 3;
        flush();
        if (i + 2 < n_my) issue((i + 2) % 3, ct + 2 * splits);

        const char *hi_base = ring[sl], *lo_base = ring[sl] + CT::part;
        floatx16 acc[2] = {floatx16{}, floatx16{}};
        // centroid fragments are read PF steps ahead of their MFMAs; the
        // scheduling fences keep the compiler from pulling the reads back
        constexpr int PF = KS < 3 ? KS : 3;
        bf16x8 fh[PF], fl[PF];
#pragma unroll
        for (int f = 0; f < PF; ++f) {
            fh[f] = *reinterpret_cast<const bf16x8 *>(hi_base + cent_off<D>(l32, 2 * f + half));
            fl[f] = *reinterpret_cast<const bf16x8 *>(lo_base + cent_off<D>(l32, 2 * f + half));
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
            const bf16x8 chi = fh[ks % PF], clo = fl[ks % PF];
            if (ks + PF < KS) {
                fh[ks % PF] = *reinterpret_cast<const bf16x8 *>(hi_base + cent_off<D>(l32, 2 * (ks + PF) + half));
                fl[ks % PF] = *reinterpret_cast<const bf16x8 *>(lo_base + cent_off<D>(l32, 2 * (ks + PF) + half));
            }
            // the two accumulators alternate, so no MFMA waits on the one just issued
#pragma unroll
            for (int term = 0; term < 3; ++term)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    const bf16x8 kf = term == 1 ? klo[kt][ks] : khi[kt][ks];
                    const bf16x8 cf = term == 2 ? clo : chi;
                    // stats: rows = key blocks, columns = slots; write: rows = slots, columns = key blocks
                    acc[kt] = write ? mfma32(cf, kf, acc[kt]) : mfma32(kf, cf, acc[kt]);
                }
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);

        if (!write) {
            // lane (l32, half) element r of tile kt: key block j0 + 32kt + 8(r/4) + 4half + r%4, slot l32.
            // The maximum is taken on the raw products (the scale is positive and rounding
            // monotone, so scaling it gives the maximum of the scaled logits) and each
            // term is 2^(x s - M) in one fma, as in the write pass; blocks past NBk only
            // occur in the last chunk's wavefronts.
            float mraw = -INFINITY;
            if (j0 + 63 < NBk) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mraw = fmaxf(mraw, acc[kt][r]);
            } else {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = j0 + 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
                        if (j >= NBk) acc[kt][r] = -INFINITY;
                        mraw = fmaxf(mraw, acc[kt][r]);
                    }
            }
            mraw = xor32_max(mraw);
            const float mx = mraw * scale_log2;
            float sum = 0.f;
            if (mraw > -INFINITY) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(fmaf(acc[kt][r], scale_log2, -mx));
            }
            sum = xor32_sum(sum);
            if (half == 0) red[i & 1][wave][l32] = make_float2(mx, sum);
        } else {
            // lane (l32, half) element r of tile kt: slot 8(r/4) + 4half + r%4 (query block
            // 4ct + r/4, centroid 4half + r%4), key block j0 + 32kt + l32
            float part[2][4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float2 sv[4];   // (M, coef) of the slots 8p + 4half + e
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[e] = st_ring[sl][8 * p + 4 * half + e];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    float a = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        a += sv[e].y * __builtin_amdgcn_exp2f(fmaf(acc[kt][4 * p + e], scale_log2, -sv[e].x));
                    part[kt][p] = xor32_sum(a);
                }
            }
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {   // lane half h stores query blocks 2h and 2h + 1
                pend[kt][0] = half ? part[kt][2] : part[kt][0];
                pend[kt][1] = half ? part[kt][3] : part[kt][1];
            }
            pend_ct = ct;
        }

        wait_tile(i + 2 < n_my);
        if (!write && tid < kTileSlots) {   // combine the four wavefronts' partials of this tile
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < 4; ++w) M = fmaxf(M, red[i & 1][w][tid].x);
            float Z = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float2 r = red[i & 1][w][tid];
                if (r.x > -INFINITY) Z += r.y * __builtin_amdgcn_exp2f(r.x - M);
            }
            partial[((bh * n_chunks + chunk) * (long)NT + ct) * kTileSlots + tid] = make_float2(M, Z);
        }
    }
    flush();
}

// Per (b, h, slot): maximum and normaliser over all chunks, and the slot's
// coefficient w_m / Z (0 for slots >= C and for query blocks past the end).
__global__ __launch_bounds__(64) void fine_merge_kernel(const float2 *__restrict__ partial,
                                                         const float *__restrict__ weight, int NBq, int C,
                                                         int n_chunks, long total, float2 *__restrict__ stat)
{
    const long i = (long)blockIdx.x * 64 + threadIdx.x;
    if (i >= total) return;
    const int NT = (NBq + kTileBlocks - 1) / kTileBlocks;
    const int slot = (int)(i % ((long)NT * kTileSlots));
    const long bh = i / ((long)NT * kTileSlots);
    const int qb = slot / kSlots, m = slot % kSlots;
    const float2 *p = partial + bh * n_chunks * (long)NT * kTileSlots + slot;
    const long stride = (long)NT * kTileSlots;
    // (M, Z) of two chunks combined into one: exact in the max, one rounding per sum
    auto combine = [](float2 a, float2 b) {
        const float M = fmaxf(a.x, b.x);
        float Z = 0.f;
        if (a.x > -INFINITY) Z += a.y * __builtin_amdgcn_exp2f(a.x - M);
        if (b.x > -INFINITY) Z += b.y * __builtin_amdgcn_exp2f(b.x - M);
        return make_float2(M, Z);
    };
    // chunks are read eight at a time, all loads in flight together
    float2 acc = make_float2(-INFINITY, 0.f);
    for (int c0 = 0; c0 < n_chunks; c0 += 8) {
        float2 r[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) r[u] = c0 + u < n_chunks ? p[(c0 + u) * stride] : make_float2(-INFINITY, 0.f);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = combine(acc, r[u]);
    }
    const float M = acc.x, Z = acc.y;
    float coef = 0.f;
    if (qb < NBq && m < C && Z > 0.f) coef = weight[(bh * NBq + qb) * C + m] / Z;
    stat[i] = make_float2(M, coef);
}

// ---------------------------------------------------------------------------
// One-pass scoring of short rows.  Workgroup (b, h, centroid tile ct): the
// workgroup loads the 32 slots' centroids once and splits them into bf16 hi and
// lo parts in LDS, from where every wavefront takes its A operand into registers;
// wavefront w computes the logit tiles of key blocks [32t, 32t + 32) for
// t = w, w + 4, ... (three split-bf16 MFMA terms per k-step, as in the
// two-pass kernels, in S orientation: rows = slots, columns = key blocks) and
// stores them, in the log2 domain, to LDS rows of one slot each.  Then 8 threads
// per slot reduce its row to the maximum M and the normaliser Z (coefficient
// w_m / Z), and every (query block, key block) score is summed over the block's
// centroids.
// ---------------------------------------------------------------------------
// Rows up to 512 key blocks: their logit rows (66 KB of LDS at 512) leave room for
// two workgroups per CU.  Longer rows go to the two-pass scorer, which streams the
// centroids instead; at 929 blocks (119K tokens) it takes the score stage from
// 1.12 to 0.82 ms.
constexpr int kRowMaxBlocks = 512;

// LDS row pitch (floats) of one slot's logits: whole 32-block tiles plus 8, so
// that the 8 slots one wavefront of the reduction reads start on different banks.
__host__ __device__ constexpr int row_pitch(int NBk) { return 32 * ((NBk + 31) / 32) + 8; }

template <int D>
__global__ __launch_bounds__(256) void row_score_kernel(const float *__restrict__ cent,
                                                        const float *__restrict__ weight,
                                                        const float *__restrict__ kbar, int NBq, int NBk, int C,
                                                        float scale_log2, float *__restrict__ scores)
{
    constexpr int KS = D / 16, DCH = D / 8;
    extern __shared__ float xs[];              // logits [32 slots][pitch]
    __shared__ float2 st[kTileSlots];          // (M, coefficient) per slot
    // split centroid tile: chunk c (8 elements) of slot r at r * DCH + (c ^ (r % DCH)),
    // so the 16 slots one phase of a fragment read touches sit on different banks
    __shared__ bf16x8 c_hi[kTileSlots * DCH], c_lo[kTileSlots * DCH];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, half = lane >> 5;
    const int NT = (NBq + kTileBlocks - 1) / kTileBlocks;
    const int ct = blockIdx.x % NT;
    const long bh = blockIdx.x / NT;
    const int pitch = row_pitch(NBk);
    const int n32 = 32 * ((NBk + 31) / 32);    // logit columns written (-inf past NBk)

    // pooled keys of key tile t (block 32t + l32), elements 16ks + 8half .. +7
    const int n_tiles = n32 / 32;
    auto load_keys = [&](int t, float (&kx)[KS][8]) __attribute__((always_inline)) {
        const int j = 32 * t + l32;
        const float *krow = kbar + (bh * NBk + j) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) kx[ks][e] = 0.f;
            if (t < n_tiles && j < NBk) load8(krow + 16 * ks + 8 * half, kx[ks]);
        }
    };
    // the first key tile's loads go out with the centroids'
    float kx[KS][8];
    load_keys(wave, kx);
    // slot r = query block 4ct + r/8, centroid r%8; slots past C or past the last
    // query block are zero
#pragma unroll
    for (int i = 0; i < kTileSlots * DCH / 256; ++i) {
        const int q = tid + 256 * i, r = q / DCH, c = q % DCH;
        const int qb = kTileBlocks * ct + r / kSlots, m = r % kSlots;
        float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (qb < NBq && m < C) load8(cent + ((bh * NBq + qb) * C + m) * D + 8 * c, x);
        bf16x8 hi, lo;
        split8(x, hi, lo);
        c_hi[r * DCH + (c ^ (r % DCH))] = hi;
        c_lo[r * DCH + (c ^ (r % DCH))] = lo;
    }
    __syncthreads();
    // A operand: slot l32, elements 16ks + 8half .. +7 (chunk 2ks + half)
    bf16x8 chi[KS], clo[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        chi[ks] = c_hi[l32 * DCH + ((2 * ks + half) ^ (l32 % DCH))];
        clo[ks] = c_lo[l32 * DCH + ((2 * ks + half) ^ (l32 % DCH))];
    }

    for (int t = wave; t < n_tiles; t += 4) {
        const int j = 32 * t + l32;
        if (t != wave) load_keys(t, kx);
        floatx16 acc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 khi, klo;
            split8(kx[ks], khi, klo);
            acc = mfma32(chi[ks], khi, acc);
            acc = mfma32(chi[ks], klo, acc);
            acc = mfma32(clo[ks], khi, acc);
        }
        // lane (l32, half) element r: slot 8(r/4) + 4half + r%4, key block j
#pragma unroll
        for (int r = 0; r < 16; ++r)
            xs[(8 * (r >> 2) + 4 * half + (r & 3)) * pitch + j] = j < NBk ? acc[r] * scale_log2 : -INFINITY;
    }
    __syncthreads();

    {   // per-slot maximum and normaliser: 8 consecutive threads per slot, four
        // independent chains each so that the LDS reads overlap (columns past NBk
        // hold -inf and add nothing)
        const int sl = tid >> 3, sub = tid & 7;
        const float *row = xs + sl * pitch;
        float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        for (int j = sub; j < n32; j += 32)
#pragma unroll
            for (int u = 0; u < 4; ++u) m4[u] = fmaxf(m4[u], row[j + 8 * u]);
        float M = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
        M = group8_max(M);
        float z4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int j = sub; j < n32; j += 32)
#pragma unroll
            for (int u = 0; u < 4; ++u) z4[u] += __builtin_amdgcn_exp2f(row[j + 8 * u] - M);
        float Z = (z4[0] + z4[1]) + (z4[2] + z4[3]);
        Z = group8_sum(Z);
        if (sub == 0) {
            const int qb = kTileBlocks * ct + sl / kSlots, m = sl % kSlots;
            float coef = 0.f;
            if (qb < NBq && m < C && Z > 0.f) coef = weight[(bh * NBq + qb) * C + m] / Z;
            st[sl] = make_float2(M, coef);
        }
    }
    __syncthreads();

    // scores of the tile's query blocks: consecutive threads, consecutive key
    // blocks; slots past C have coefficient 0 and finite logits (zero centroids)
    const int n_qb = min(kTileBlocks, NBq - kTileBlocks * ct);
    for (int i = tid; i < n_qb * NBk; i += 256) {
        const int p = i / NBk, j = i - p * NBk;
        float a = 0.f;
#pragma unroll
        for (int m = 0; m < kSlots; ++m) {
            const float2 sv = st[kSlots * p + m];
            a += sv.y * __builtin_amdgcn_exp2f(xs[(kSlots * p + m) * pitch + j] - sv.x);
        }
        scores[(bh * NBq + kTileBlocks * ct + p) * (long)NBk + j] = a;
    }
}

}  // namespace

hipError_t launch_fine_pool(const void *k, int dtype, int B, int H, int N, int N_pad, int D, int NBk, float *kbar,
                            hipStream_t s)
{
    const long total = (long)B * H * NBk * (D / 8);
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    if (dtype == kBF16 && D == 128)
        fine_pool_kernel<uint16_t, 128><<<grid, block, 0, s>>>((const uint16_t *)k, N, N_pad, NBk, total, kbar);
    else if (dtype == kBF16 && D == 64)
        fine_pool_kernel<uint16_t, 64><<<grid, block, 0, s>>>((const uint16_t *)k, N, N_pad, NBk, total, kbar);
    else if (dtype == kF32 && D == 64)
        fine_pool_kernel<float, 64><<<grid, block, 0, s>>>((const float *)k, N, N_pad, NBk, total, kbar);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// Work split over the centroid tiles: the kernel holds two workgroups per CU
// (512 at once); pick the split count that minimises rounds of 512 per unit of
// work, the smaller one on ties.
static int fine_splits(long base_wgs, int NT)
{
    int best = 1;
    double best_t = 1e30;
    for (int sp = 1; sp <= 16 && sp <= NT; sp *= 2) {
        const double rounds = (double)((base_wgs * sp + 511) / 512);
        const double t = rounds / sp;
        if (t < best_t - 1e-9) {
            best_t = t;
            best = sp;
        }
    }
    return best;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t fine_score_workspace_bytes(int B, int H, int NBq, int NBk)
{
    const long NT = (NBq + kTileBlocks - 1) / kTileBlocks;
    const long n_chunks = (NBk + kChunk - 1) / kChunk;
    const size_t part = (size_t)B * H * n_chunks * NT * kTileSlots * sizeof(float2);
    const size_t stat = (size_t)B * H * NT * kTileSlots * sizeof(float2);
    const size_t tiles = (size_t)B * H * NT * CentTile<128>::bytes;   // the larger of D = 64, 128
    return align256(part) + align256(stat) + align256(tiles);
}

hipError_t launch_fine_score(const float *cent, const float *weight, const float *kbar, int B, int H, int NBq, int NBk,
                             int C, int D, float scale, void *ws, float *scores, hipStream_t s)
{
    if (C < 1 || C > kSlots) return hipErrorInvalidValue;
    const int NT = (NBq + kTileBlocks - 1) / kTileBlocks;
    const float sl2 = scale * kLog2e;
    if (NBk <= kRowMaxBlocks) {   // short rows: one pass, logits in LDS
        const size_t lds = (size_t)kTileSlots * row_pitch(NBk) * sizeof(float);
        const dim3 grid((unsigned)((long)B * H * NT)), block(256);
        if (D == 128) {
            const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&row_score_kernel<128>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            row_score_kernel<128><<<grid, block, lds, s>>>(cent, weight, kbar, NBq, NBk, C, sl2, scores);
        } else if (D == 64) {
            const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&row_score_kernel<64>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            row_score_kernel<64><<<grid, block, lds, s>>>(cent, weight, kbar, NBq, NBk, C, sl2, scores);
        } else {
            return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const int n_chunks = (NBk + kChunk - 1) / kChunk;
    const size_t part_bytes = (size_t)B * H * n_chunks * NT * kTileSlots * sizeof(float2);
    const size_t stat_bytes = (size_t)B * H * NT * kTileSlots * sizeof(float2);
    char *w = static_cast<char *>(ws);
    float2 *partial = reinterpret_cast<float2 *>(w);
    float2 *stat = reinterpret_cast<float2 *>(w + align256(part_bytes));
    uint16_t *tiles = reinterpret_cast<uint16_t *>(w + align256(part_bytes) + align256(stat_bytes));
    const long base = (long)B * H * n_chunks;
    const int splits = fine_splits(base, NT);
    const dim3 grid((unsigned)(base * splits)), block(256);
    const long slots = (long)B * H * NT * kTileSlots;
    const dim3 merge_grid((unsigned)((slots + 63) / 64)), merge_block(64);   // many small groups: latency-bound
    if (D == 128) {
        const long tt = (long)B * H * NT * kTileSlots * CentTile<128>::chunks;
        fine_cent_kernel<128><<<dim3((unsigned)((tt + 255) / 256)), block, 0, s>>>(cent, NBq, C, NT, tt, tiles);
        fine_score_kernel<128, false><<<grid, block, 0, s>>>(tiles, kbar, nullptr, NBq, NBk, n_chunks, splits, sl2,
                                                             partial, nullptr);
        fine_merge_kernel<<<merge_grid, merge_block, 0, s>>>(partial, weight, NBq, C, n_chunks, slots, stat);
        fine_score_kernel<128, true><<<grid, block, 0, s>>>(tiles, kbar, stat, NBq, NBk, n_chunks, splits, sl2,
                                                            nullptr, scores);
    } else if (D == 64) {
        const long tt = (long)B * H * NT * kTileSlots * CentTile<64>::chunks;
        fine_cent_kernel<64><<<dim3((unsigned)((tt + 255) / 256)), block, 0, s>>>(cent, NBq, C, NT, tt, tiles);
        fine_score_kernel<64, false><<<grid, block, 0, s>>>(tiles, kbar, nullptr, NBq, NBk, n_chunks, splits, sl2,
                                                            partial, nullptr);
        fine_merge_kernel<<<merge_grid, merge_block, 0, s>>>(partial, weight, NBq, C, n_chunks, slots, stat);
        fine_score_kernel<64, true><<<grid, block, 0, s>>>(tiles, kbar, stat, NBq, NBk, n_chunks, splits, sl2,
                                                           nullptr, scores);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace aba
