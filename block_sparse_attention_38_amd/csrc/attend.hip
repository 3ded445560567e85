// attend.hip -- block-sparse flash attention with Horvitz-Thompson block
// weights (gfx950).
//
// AB-Attention page, section "Три приёма AB-Attention": each kept key block is
// weighted by its inverse inclusion probability in both the numerator and the
// softmax normaliser, which keeps the computation ordinary softmax attention
// with shifted logits (SIP paragraph); the kernel gathers the selected key
// blocks by index into full matrix-core tiles, in the original token order,
// with no permutation and no copies (third paragraph).  The dense path is the
// same kernel over every key block with unit weights.
//
// bf16 path (the hot path): one workgroup of 4 wavefronts per (b, h, query
// block), two workgroups per CU; wavefront w owns query rows [32w, 32w + 32).
// Each kept key block is streamed as two 64-key sub-tiles through a
// double-buffered LDS stage: the next sub-tile's global loads are issued into
// registers before the current one is computed and written to the other LDS
// buffer afterwards, so one barrier per sub-tile remains.  Per sub-tile:
//   S^T = K Q^T      32x32x16 bf16 MFMA, K from LDS, Q fragments in registers
//   online softmax   in the exp2 domain; the block's log2(w_j) is added to its
//                    logits, so the weight enters numerator and normaliser; the
//                    running max moves only when it grows by more than 2^8
//   O^T += V^T P^T   32x32x16 bf16 MFMA, P^T straight from the S^T accumulators
// Computing the transposed products makes every lane own one query column, so
// row statistics need a single cross-half exchange and the rescale of O is a
// per-lane scalar multiply.  K sits in LDS row-major; V is transposed on its
// way into LDS (key-contiguous) so that the PV operand is two 8-byte reads.
// Both use padded rows, which keeps the reads free of bank conflicts and every
// LDS address a per-lane base plus an immediate offset.
//
// fp32 path: a plain VALU kernel (pairs of lanes per query row) for fp32
// inputs with head_dim 64.
#include "aba_internal.h"

namespace aba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Key blocks are streamed as sub-tiles of 64 keys.
constexpr int kSub = 64;
// Lazy rescaling: the running max only moves when a sub-tile's max exceeds it
// by more than this many powers of two (exp2 values then stay below 2^8).
constexpr float kRescaleSlack = 8.f;
// Two wavefronts per workgroup, 64 query rows each (two 32-row MFMA tiles).
constexpr int kThreads = 128;
constexpr int QT = 2;

// LDS layout of one stage: K and V sub-tiles of 64 rows x D bf16, unpadded
// (one direct global->LDS load fills four whole rows), with XOR swizzles of the
// 16-byte chunks chosen per tensor:
//   K  chunk c of row r at c ^ (r % 16): the 16 rows one 16-lane phase of a
//      128-bit read touches hit 16 different chunks;
//   V  chunk c of row r at c ^ 4(r % 4): the four rows x 64 bytes that 32 lanes
//      of a transposing 64-bit read touch fall on distinct banks.
template <int D> struct Lds {
    static constexpr int pitch = D * 2;
    static constexpr int chunks = D / 8;
    static constexpr int kBytes = kSub * pitch;
    static constexpr int vBytes = kSub * pitch;
    static constexpr int stage = kBytes + vBytes;
};
template <int D> __device__ __forceinline__ int k_swz(int r) { return r & (Lds<D>::chunks - 1); }
template <int D> __device__ __forceinline__ int v_swz(int r) { return (4 * (r & 3)) & (Lds<D>::chunks - 1); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void glb_void;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element (i % 4) of the 8-byte chunks addressed by
// lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4: if lane L addresses row kb + L/4,
// columns c0 + 4(L % 4) .. +3 of a row-major 16-bit matrix, lane i receives
// column c0 + i at rows kb .. kb+3.
__device__ __forceinline__ uint2 lds_read_tr16(const char *p)
{
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p)));
}

// Direct global -> LDS copy of 16 bytes per lane; lane L's bytes land at
// dst + 16 L (dst is wavefront-uniform).
__device__ __forceinline__ void load_lds16(const uint16_t *src, char *dst)
{
    __builtin_amdgcn_global_load_lds((glb_void *)src, (lds_void *)dst, 16, 0, 0);
}

// Issue the direct loads of one 64-key sub-tile of K and V (rows key0 ..
// key0 + 63) into an LDS stage.  Wavefront w fills rows [32w, 32w + 32) of
// both tensors with loads of 1024 bytes (four rows at D = 128).  The source
// byte offset of every lane is precomputed (DmaOffsets), so a full sub-tile is
// scalar base + per-lane offset only.  On the ragged last block, rows past the
// last valid one are read from that row instead (finite values; those keys are
// masked and their probabilities are zero).  Needs a vmcnt wait and a barrier
// before the stage is read.
template <int D> struct DmaOffsets {
    static constexpr int rows_per_load = 1024 / (D * 2);   // 4 (D=128) or 8 (D=64)
    static constexpr int loads = 32 / rows_per_load;
    static constexpr int kPeriod = 16 / rows_per_load;     // loads after which the K swizzle repeats
    int k[kPeriod];
    int v;
};

template <int D>
__device__ __forceinline__ DmaOffsets<D> dma_offsets(int wave, int lane)
{
    using L = Lds<D>;
    DmaOffsets<D> off;
    const int lr = lane / L::chunks, pc = lane % L::chunks;
#pragma unroll
    for (int t = 0; t < DmaOffsets<D>::kPeriod; ++t) {
        const int r = 32 * wave + DmaOffsets<D>::rows_per_load * t + lr;
        off.k[t] = r * L::pitch + 16 * (pc ^ k_swz<D>(r));
    }
    const int r0 = 32 * wave + lr;
    off.v = r0 * L::pitch + 16 * (pc ^ v_swz<D>(r0));
    return off;
}

template <int D>
__device__ __forceinline__ void stage_issue(const uint16_t *kh, const uint16_t *vh, int key0, int valid, char *stage,
                                            int wave, int lane, const DmaOffsets<D> &off)
{
    using L = Lds<D>;
    using O = DmaOffsets<D>;
    const char *kb = reinterpret_cast<const char *>(kh + (long)key0 * D);
    const char *vb = reinterpret_cast<const char *>(vh + (long)key0 * D);
    char *kd = stage + 32 * wave * L::pitch;
    if (valid >= kSub) {
#pragma unroll
        for (int t = 0; t < O::loads; ++t) {
            const int step = O::rows_per_load * t * L::pitch;   // whole rows: the V swizzle is unchanged
            load_lds16(reinterpret_cast<const uint16_t *>(kb + (off.k[t % O::kPeriod] + (t / O::kPeriod) * 16 * L::pitch)),
                       kd + step);
            load_lds16(reinterpret_cast<const uint16_t *>(vb + off.v + step), kd + L::kBytes + step);
        }
    } else {
        const int lr = lane / L::chunks, pc = lane % L::chunks;
#pragma unroll
        for (int t = 0; t < O::loads; ++t) {
            const int r = 32 * wave + O::rows_per_load * t + lr;
            const int rs = r < valid ? r : valid - 1;
            load_lds16(kh + (long)(key0 + rs) * D + 8 * (pc ^ k_swz<D>(r)), kd + O::rows_per_load * t * L::pitch);
            load_lds16(vh + (long)(key0 + rs) * D + 8 * (pc ^ v_swz<D>(r)),
                       kd + L::kBytes + O::rows_per_load * t * L::pitch);
        }
    }
}

// One list entry: key block j with log2 weight lw; j < 0 marks an entry to skip.
struct Entry {
    int j;
    float lw;
};

template <bool full>
__device__ __forceinline__ Entry list_entry(const int32_t *lrow, const float *wrow, int e, int NB)
{
    if (full) return Entry{e, 0.f};
    const int j = lrow[e];
    const float wj = wrow[e];
    if (j < 0 || j >= NB || !(wj > 0.f) || !(wj < INFINITY)) return Entry{-1, 0.f};
    return Entry{j, __log2f(wj)};
}

template <int D, bool full>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void attend_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ cnt, const float *__restrict__ w,
    uint16_t *__restrict__ out, int N, int N_pad, int NB, int cap, float scale_log2)
{
    using L = Lds<D>;
    constexpr int KS = D / 16;         // k-steps of S^T = K Q^T
    constexpr int DT = D / 32;         // 32-row tiles of O^T
    constexpr int KT = kSub / 32;      // 32-key tiles per sub-tile
    __shared__ __align__(16) char lds[2 * L::stage];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, half = lane >> 5, grp = lane >> 4, i16 = lane & 15;
    const int blk = xcd_contiguous_id(blockIdx.x, gridDim.x);   // (b*H + h) * NB + query block
    const int qb = blk % NB;
    const long bh = blk / NB;
    const uint16_t *qh = q + bh * N_pad * D;
    const uint16_t *kh = k + bh * N_pad * D;
    const uint16_t *vh = v + bh * N_pad * D;

    // this lane's two query rows (one per 32-row tile); padding rows read as zero
    int qrow[QT];
    bool qvalid[QT];
    bf16x8 qf[QT][KS];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        qrow[qt] = qb * kBlock + wave * 64 + qt * 32 + l32;
        qvalid[qt] = qrow[qt] < N;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 raw = make_uint4(0, 0, 0, 0);
            if (qvalid[qt]) raw = *reinterpret_cast<const uint4 *>(qh + (long)qrow[qt] * D + 16 * ks + 8 * half);
            qf[qt][ks] = __builtin_bit_cast(bf16x8, raw);
        }
    }

    floatx16 o[QT][DT];
    float m_run[QT], l_run[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        m_run[qt] = -INFINITY;
        l_run[qt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qt][dt][r] = 0.f;
    }
    const floatx16 zero16 = {};

    int n_list = NB;
    const int32_t *lrow = nullptr;
    const float *wrow = nullptr;
    if (!full) {
        n_list = cnt[blk];
        n_list = n_list < 0 ? 0 : (n_list > cap ? cap : n_list);
        lrow = idx + (long)blk * cap;
        wrow = w + (long)blk * cap;
    }
    const int n_sub = 2 * n_list;   // sub-tile u = half (u & 1) of list entry u >> 1

    // Per-lane LDS read offsets (compile-time row offsets are added in the loops).
    // K: row 32kt + l32, logical chunk 2ks + half; row % 16 == l32 % 16.
    int k_rd[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k_rd[ks] = l32 * L::pitch + 16 * ((2 * ks + half) ^ k_swz<D>(l32));
    // V (transposing reads): lane group grp addresses row kb + i16/4 (kb a
    // multiple of 4) at dims 32dt + 16(grp & 1) + 4(i16 % 4), with kb = 32kt +
    // 16sub + 4half (+8 for the second read), so lane (l32, half) receives dim
    // 32dt + l32 at the keys its P^T operand holds.
    int v_rd[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        const int rr = 4 * half + (i16 >> 2);
        const int c = 4 * dt + 2 * (grp & 1) + ((i16 & 3) >> 1);
        v_rd[dt] = L::kBytes + rr * L::pitch + 16 * (c ^ v_swz<D>(rr)) + 8 * (i16 & 1);
    }

    const DmaOffsets<D> dma = dma_offsets<D>(wave, lane);
    Entry cur{-1, 0.f};
    if (n_sub > 0) {
        cur = list_entry<full>(lrow, wrow, 0, NB);
        if (cur.j >= 0)
            stage_issue<D>(kh, vh, cur.j * kBlock, min(kSub, N - cur.j * kBlock), lds, wave, lane, dma);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // Per sub-tile: S^T = K Q^T for both query tiles; s[qt][kt] holds keys
    // [32kt, 32kt+32) of the sub-tile, lane (l32, half) key 32kt + 8(r/4) + 4half + r%4.
    floatx16 s[QT][KT];
    float m_tile[QT];
    auto scores = [&](const char *stage, int key0) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            const char *kr = stage + kt * 32 * L::pitch;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(kr + k_rd[ks]));
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) s[qt][kt] = mfma32(a, qf[qt][ks], ks == 0 ? zero16 : s[qt][kt]);
            }
        }
        if (key0 + kSub > N) {   // ragged end of the sequence: mask padding keys
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (key0 + kt * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= N) s[qt][kt][r] = -INFINITY;
        }
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qt][kt][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            m_tile[qt] = fmaf(mx, scale_log2, cur.lw);   // block weight enters as a logit shift
        }
    };
    // Probabilities against the running max, then O^T += V^T P^T.  MFMA (kt, sub)
    // contracts the 16 keys held in accumulator rows [8sub, 8sub+8) of tile kt:
    // for lane half h, element e is key 32kt + 16sub + 8(e/4) + 4h + e%4,
    // fetched by two transposing reads at rows 32kt + 16sub + 4h (+8).
    auto accumulate = [&](const char *stage) {
        // query tile 0's PV MFMAs are independent of tile 1's softmax, so the
        // two can be co-issued
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            bf16x8 pb[KT][2];
            const float bias = cur.lw - m_run[qt];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[qt][kt][r], scale_log2, bias));
                    l_run[qt] += p;
                    pb[kt][r >> 3][r & 7] = (__bf16)p;
                }
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const char *vr = stage + v_rd[dt] + (32 * kt + 16 * sub) * L::pitch;
                        const uint2 a0 = lds_read_tr16(vr);
                        const uint2 a1 = lds_read_tr16(vr + 8 * L::pitch);
                        const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(a0.x, a0.y, a1.x, a1.y));
                        o[qt][dt] = mfma32(a, pb[kt][sub], o[qt][dt]);
                    }
        }
    };
    // Issue the direct loads of sub-tile u + 1 into the other stage.
    auto prefetch = [&](int u, Entry &nxt) {
        nxt = cur;
        if (u + 1 < n_sub) {
            if (u & 1) nxt = list_entry<full>(lrow, wrow, (u + 1) >> 1, NB);
            const int nkey0 = nxt.j * kBlock + kSub * ((u + 1) & 1);
            if (nxt.j >= 0 && nkey0 < N)
                stage_issue<D>(kh, vh, nkey0, min(kSub, N - nkey0), lds + ((u + 1) & 1) * L::stage, wave, lane, dma);
        }
    };

    // The running max only moves when a sub-tile's max exceeds it by more than
    // the slack (always on the first sub-tile).  Such sub-tiles leave the hot
    // loop for the rescale below, so inside the hot loop the output
    // accumulators are touched by MFMAs only.
    int u = 0;
    while (u < n_sub) {
        bool grow = false;
        Entry nxt;
        for (; u < n_sub; ++u) {
            const char *stage = lds + (u & 1) * L::stage;
            prefetch(u, nxt);
            const int key0 = cur.j * kBlock + kSub * (u & 1);
            if (cur.j >= 0 && key0 < N) {   // uniform over the workgroup
                scores(stage, key0);
                const bool g0 = m_tile[0] > m_run[0] + kRescaleSlack, g1 = m_tile[1] > m_run[1] + kRescaleSlack;
                if (__ballot(g0 || g1) != 0) {
                    grow = true;
                    break;
                }
                accumulate(stage);
            }
            cur = nxt;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
        if (!grow) break;
        // rescale (rare): sub-tile u's scores are in s, its successor is in flight
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const float m_new = fmaxf(m_run[qt], m_tile[qt]);
            const float alpha = __builtin_amdgcn_exp2f(m_run[qt] - m_new);
            m_run[qt] = m_new;
            l_run[qt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[qt][dt][r] *= alpha;
        }
        accumulate(lds + (u & 1) * L::stage);
        cur = nxt;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        ++u;
    }

    // normalise and store: lane holds dims dt*32 + 8(r/4) + 4half + r%4 of its query
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const float lsum = l_run[qt] + __shfl_xor(l_run[qt], 32, 64);
        const float inv = (lsum > 0.f && qvalid[qt]) ? 1.f / lsum : 0.f;
        uint16_t *orow = out + (bh * N_pad + qrow[qt]) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = dt * 32 + 8 * g + 4 * half;
                __bf16 b0 = (__bf16)(o[qt][dt][4 * g + 0] * inv), b1 = (__bf16)(o[qt][dt][4 * g + 1] * inv);
                __bf16 b2 = (__bf16)(o[qt][dt][4 * g + 2] * inv), b3 = (__bf16)(o[qt][dt][4 * g + 3] * inv);
                const uint32_t lo =
                    (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
                const uint32_t hi =
                    (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
                *reinterpret_cast<uint2 *>(orow + d) = make_uint2(lo, hi);
            }
    }
}

// ---------------------------------------------------------------------------
// fp32 path: two lanes per query row, each owning half of the head dimension;
// key/value tiles of 64 rows in LDS.
// ---------------------------------------------------------------------------
template <int D, bool full>
__global__ __launch_bounds__(256) void attend_f32_kernel(const float *__restrict__ q, const float *__restrict__ k,
                                                         const float *__restrict__ v, const int32_t *__restrict__ idx,
                                                         const int32_t *__restrict__ cnt, const float *__restrict__ w,
                                                         float *__restrict__ out, int N, int N_pad, int NB, int cap,
                                                         float scale_log2)
{
    constexpr int kTile = 64, HD = D / 2, kChunk = 16;
    __shared__ float4 k_s[kTile][D / 4];
    __shared__ float4 v_s[kTile][D / 4];

    const int tid = threadIdx.x;
    const int blk = xcd_contiguous_id(blockIdx.x, gridDim.x);
    const int qb = blk % NB;
    const long bh = blk / NB;
    const int r = tid >> 1, hd = tid & 1;
    const int qrow = qb * kBlock + r;
    const bool qvalid = qrow < N;
    const float *kh = k + bh * N_pad * D, *vh = v + bh * N_pad * D;

    float qv[HD], ov[HD];
#pragma unroll
    for (int d = 0; d < HD; ++d) {
        qv[d] = qvalid ? q[(bh * N_pad + qrow) * D + hd * HD + d] : 0.f;
        ov[d] = 0.f;
    }
    float m_run = -INFINITY, l_run = 0.f;

    int n_list = NB;
    if (!full) {
        n_list = cnt[blk];
        n_list = n_list < 0 ? 0 : (n_list > cap ? cap : n_list);
    }
    for (int e = 0; e < n_list; ++e) {
        int j = e;
        float lw = 0.f;
        if (!full) {
            j = idx[(long)blk * cap + e];
            const float wj = w[(long)blk * cap + e];
            if (j < 0 || j >= NB || !(wj > 0.f) || !(wj < INFINITY)) continue;
            lw = __log2f(wj);
        }
        for (int t0 = 0; t0 < kBlock; t0 += kTile) {
            const int key0 = j * kBlock + t0;
            __syncthreads();
            for (int i = tid; i < kTile * D / 4; i += 256) {
                const int rr = i / (D / 4), c = i % (D / 4);
                const bool ok = key0 + rr < N;
                k_s[rr][c] = ok ? reinterpret_cast<const float4 *>(kh + (long)(key0 + rr) * D)[c] : make_float4(0, 0, 0, 0);
                v_s[rr][c] = ok ? reinterpret_cast<const float4 *>(vh + (long)(key0 + rr) * D)[c] : make_float4(0, 0, 0, 0);
            }
            __syncthreads();
            for (int c0 = 0; c0 < kTile; c0 += kChunk) {
                if (key0 + c0 >= N) break;
                float lg[kChunk];
                float cmax = -INFINITY;
#pragma unroll
                for (int tt = 0; tt < kChunk; ++tt) {
                    const float *kr = reinterpret_cast<const float *>(&k_s[c0 + tt][0]) + hd * HD;
                    float dot = 0.f;
#pragma unroll
                    for (int d = 0; d < HD; ++d) dot = fmaf(qv[d], kr[d], dot);
                    dot += __shfl_xor(dot, 1, 64);
                    lg[tt] = (key0 + c0 + tt < N) ? fmaf(dot, scale_log2, lw) : -INFINITY;
                    cmax = fmaxf(cmax, lg[tt]);
                }
                const float m_new = fmaxf(m_run, cmax);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int d = 0; d < HD; ++d) ov[d] *= alpha;
#pragma unroll
                for (int tt = 0; tt < kChunk; ++tt) {
                    const float p = __builtin_amdgcn_exp2f(lg[tt] - m_new);
                    l_run += p;
                    const float *vr = reinterpret_cast<const float *>(&v_s[c0 + tt][0]) + hd * HD;
#pragma unroll
                    for (int d = 0; d < HD; ++d) ov[d] = fmaf(p, vr[d], ov[d]);
                }
            }
        }
    }
    const float inv = (l_run > 0.f && qvalid) ? 1.f / l_run : 0.f;
    float *orow = out + (bh * N_pad + qrow) * D + hd * HD;
#pragma unroll
    for (int d = 0; d < HD; ++d) orow[d] = ov[d] * inv;
}

}  // namespace

template <bool full>
hipError_t launch_attend_t(const void *q, const void *k, const void *v, int dtype, int B, int H, int N, int N_pad,
                           int D, int NB, float scale, const int32_t *idx, const int32_t *cnt, const float *w, int cap,
                           void *out, hipStream_t s)
{
    const dim3 grid((unsigned)((long)B * H * NB)), block(256);
    const float sl2 = scale * kLog2e;
    if (dtype == kBF16 && D == 128)
        attend_bf16_kernel<128, full><<<grid, dim3(kThreads), 0, s>>>((const uint16_t *)q, (const uint16_t *)k,
                                                            (const uint16_t *)v, idx, cnt, w, (uint16_t *)out, N, N_pad,
                                                            NB, cap, sl2);
    else if (dtype == kBF16 && D == 64)
        attend_bf16_kernel<64, full><<<grid, dim3(kThreads), 0, s>>>((const uint16_t *)q, (const uint16_t *)k,
                                                           (const uint16_t *)v, idx, cnt, w, (uint16_t *)out, N, N_pad,
                                                           NB, cap, sl2);
    else if (dtype == kF32 && D == 64)
        attend_f32_kernel<64, full><<<grid, block, 0, s>>>((const float *)q, (const float *)k, (const float *)v, idx,
                                                          cnt, w, (float *)out, N, N_pad, NB, cap, sl2);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_attend(const void *q, const void *k, const void *v, int dtype, int B, int H, int N, int N_pad, int D,
                         int NB, float scale, const int32_t *idx, const int32_t *cnt, const float *w, int cap, bool full,
                         void *out, hipStream_t s)
{
    return full ? launch_attend_t<true>(q, k, v, dtype, B, H, N, N_pad, D, NB, scale, idx, cnt, w, cap, out, s)
                : launch_attend_t<false>(q, k, v, dtype, B, H, N, N_pad, D, NB, scale, idx, cnt, w, cap, out, s);
}

}  // namespace aba
