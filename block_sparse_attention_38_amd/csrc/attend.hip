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
// per-lane scalar multiply.  K sits in LDS row-major with a 16-byte XOR swizzle;
// V is transposed on its way into LDS (key-contiguous, 8-byte XOR swizzle) so
// that the PV operand is two 8-byte reads.
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

// K sub-tile: 64 rows x D bf16 in 16-byte chunks, chunk c of row r stored at
// r * (D/8) + (c ^ swz(r)); the swizzle spreads the 16 rows that one
// 16-lane phase of a 128-bit read touches over distinct banks.
template <int D> __device__ __forceinline__ int k_slot(int r, int c)
{
    constexpr int kChunks = D / 8;
    if constexpr (kChunks == 16)
        return r * 16 + (c ^ (r & 15));
    else
        return r * 8 + (c ^ ((r >> 1) & 7));   // 128-byte rows: row parity already splits the banks
}
// V^T sub-tile: D rows (dims) x 64 keys in 8-byte slots of 4 keys (16 slots,
// 128 bytes per row); slot s of row d stored at d * 16 + (s ^ ((d >> 1) & 15)),
// so that the 32 rows one 8-byte read phase touches hit distinct banks.
__device__ __forceinline__ int vt_slot(int d, int s) { return d * 16 + (s ^ ((d >> 1) & 15)); }

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// Global -> register staging of one 64-key sub-tile (each thread holds its
// share until it is written to LDS after the current sub-tile is computed).
template <int D> struct Stage {
    static constexpr int kChunks = D / 8;
    static constexpr int kKLoads = kSub * kChunks / 256;       // 16-byte K chunks per thread
    static constexpr bool kVAll = (kSub / 4) * kChunks >= 256; // every thread moves one V quad
    uint4 k[kKLoads];
    uint4 v[4];
};

template <int D>
__device__ __forceinline__ void stage_load(Stage<D> &st, const uint16_t *kh, const uint16_t *vh, int key0, int N,
                                           int tid, bool active)
{
    constexpr int kChunks = D / 8;
    const int c = tid % kChunks;
#pragma unroll
    for (int i = 0; i < Stage<D>::kKLoads; ++i) {
        const int r = tid / kChunks + i * (256 / kChunks);
        st.k[i] = make_uint4(0, 0, 0, 0);
        if (active && key0 + r < N) st.k[i] = *reinterpret_cast<const uint4 *>(kh + (long)(key0 + r) * D + 8 * c);
    }
    const int quad = tid / kChunks;   // keys 4*quad .. 4*quad+3
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int key = key0 + 4 * quad + rr;
        st.v[rr] = make_uint4(0, 0, 0, 0);
        if (active && quad < kSub / 4 && key < N)
            st.v[rr] = *reinterpret_cast<const uint4 *>(vh + (long)key * D + 8 * c);
    }
}

template <int D>
__device__ __forceinline__ void stage_store(const Stage<D> &st, uint4 *k_s, uint2 *vt_s, int tid)
{
    constexpr int kChunks = D / 8;
    const int c = tid % kChunks;
#pragma unroll
    for (int i = 0; i < Stage<D>::kKLoads; ++i) {
        const int r = tid / kChunks + i * (256 / kChunks);
        k_s[k_slot<D>(r, c)] = st.k[i];
    }
    const int quad = tid / kChunks;
    if (Stage<D>::kVAll || quad < kSub / 4) {
        const uint32_t *r0 = reinterpret_cast<const uint32_t *>(&st.v[0]);
        const uint32_t *r1 = reinterpret_cast<const uint32_t *>(&st.v[1]);
        const uint32_t *r2 = reinterpret_cast<const uint32_t *>(&st.v[2]);
        const uint32_t *r3 = reinterpret_cast<const uint32_t *>(&st.v[3]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int d = 8 * c + 2 * p;
            vt_s[vt_slot(d, quad)] = make_uint2(pack_lo(r0[p], r1[p]), pack_lo(r2[p], r3[p]));
            vt_s[vt_slot(d + 1, quad)] = make_uint2(pack_hi(r0[p], r1[p]), pack_hi(r2[p], r3[p]));
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
__global__ __launch_bounds__(256, 2) void attend_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ cnt, const float *__restrict__ w,
    uint16_t *__restrict__ out, int N, int N_pad, int NB, int cap, float scale_log2)
{
    constexpr int kChunks = D / 8;     // 16-byte chunks per K row
    constexpr int KS = D / 16;         // k-steps of S^T = K Q^T
    constexpr int DT = D / 32;         // 32-row tiles of O^T
    constexpr int KT = kSub / 32;      // 32-key tiles per sub-tile
    __shared__ uint4 k_s[2][kSub * kChunks];
    __shared__ uint2 vt_s[2][D * kSub / 4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, half = lane >> 5;
    const int blk = xcd_contiguous_id(blockIdx.x, gridDim.x);   // (b*H + h) * NB + query block
    const int qb = blk % NB;
    const long bh = blk / NB;
    const uint16_t *qh = q + bh * N_pad * D;
    const uint16_t *kh = k + bh * N_pad * D;
    const uint16_t *vh = v + bh * N_pad * D;

    // this lane's query row; padding rows read as zero
    const int qrow = qb * kBlock + wave * 32 + l32;
    const bool qvalid = qrow < N;
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (qvalid) raw = *reinterpret_cast<const uint4 *>(qh + (long)qrow * D + 16 * ks + 8 * half);
        qf[ks] = __builtin_bit_cast(bf16x8, raw);
    }

    floatx16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

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

    Stage<D> st;
    Entry cur{-1, 0.f};
    if (n_sub > 0) {
        cur = list_entry<full>(lrow, wrow, 0, NB);
        stage_load<D>(st, kh, vh, cur.j * kBlock, N, tid, cur.j >= 0);
        stage_store<D>(st, k_s[0], vt_s[0], tid);
    }
    __syncthreads();

    for (int u = 0; u < n_sub; ++u) {
        const int buf = u & 1;
        // prefetch the next sub-tile into registers; it lands while this one is computed
        Entry nxt = cur;
        if (u + 1 < n_sub) {
            if ((u & 1) == 1) nxt = list_entry<full>(lrow, wrow, (u + 1) >> 1, NB);
            stage_load<D>(st, kh, vh, nxt.j * kBlock + kSub * ((u + 1) & 1), N, tid, nxt.j >= 0);
        }

        const int key0 = cur.j * kBlock + kSub * (u & 1);
        if (cur.j >= 0 && key0 < N) {   // uniform over the workgroup
            // S^T = K Q^T: tile kt holds keys [32kt, 32kt+32) of the sub-tile x this
            // wave's 32 queries; lane (l32, half) holds key 32kt + 8(r/4) + 4half + r%4.
            floatx16 s[KT];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
                const int krow = kt * 32 + l32;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const uint4 a = k_s[buf][k_slot<D>(krow, 2 * ks + half)];
                    s[kt] = mfma32(__builtin_bit_cast(bf16x8, a), qf[ks], s[kt]);
                }
            }
            if (key0 + kSub > N) {   // ragged end of the sequence: mask padding keys
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (key0 + kt * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= N) s[kt][r] = -INFINITY;
            }

            // online softmax in the exp2 domain; the block weight is a logit shift
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_tile = fmaf(mx, scale_log2, cur.lw);
            if (__ballot(m_tile > m_run + kRescaleSlack) != 0) {   // wave-uniform
                const float m_new = fmaxf(m_run, m_tile);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
            }
            const float bias = cur.lw - m_run;

            bf16x8 pb[KT][2];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][r], scale_log2, bias));
                    l_run += p;
                    pb[kt][r >> 3][r & 7] = (__bf16)p;
                }

            // O^T += V^T P^T.  MFMA (kt, sub) contracts the 16 keys held in
            // accumulator rows [8sub, 8sub+8) of tile kt: for lane half h,
            // element e is key 32kt + 16sub + 8(e/4) + 4h + e%4.
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int d = dt * 32 + l32;
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                    for (int sub = 0; sub < 2; ++sub) {
                        const int slot = 8 * kt + 4 * sub + half;
                        const uint2 a0 = vt_s[buf][vt_slot(d, slot)];
                        const uint2 a1 = vt_s[buf][vt_slot(d, slot + 2)];
                        const uint4 a = make_uint4(a0.x, a0.y, a1.x, a1.y);
                        o[dt] = mfma32(__builtin_bit_cast(bf16x8, a), pb[kt][sub], o[dt]);
                    }
            }
        }

        if (u + 1 < n_sub) stage_store<D>(st, k_s[buf ^ 1], vt_s[buf ^ 1], tid);
        cur = nxt;
        __syncthreads();
    }

    // normalise and store: lane holds dims dt*32 + 8(r/4) + 4half + r%4 of its query
    l_run += __shfl_xor(l_run, 32, 64);
    const float inv = (l_run > 0.f && qvalid) ? 1.f / l_run : 0.f;
    uint16_t *orow = out + (bh * N_pad + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = dt * 32 + 8 * g + 4 * half;
            __bf16 b0 = (__bf16)(o[dt][4 * g + 0] * inv), b1 = (__bf16)(o[dt][4 * g + 1] * inv);
            __bf16 b2 = (__bf16)(o[dt][4 * g + 2] * inv), b3 = (__bf16)(o[dt][4 * g + 3] * inv);
            const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
            const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
            *reinterpret_cast<uint2 *>(orow + d) = make_uint2(lo, hi);
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
        attend_bf16_kernel<128, full><<<grid, block, 0, s>>>((const uint16_t *)q, (const uint16_t *)k,
                                                            (const uint16_t *)v, idx, cnt, w, (uint16_t *)out, N, N_pad,
                                                            NB, cap, sl2);
    else if (dtype == kBF16 && D == 64)
        attend_bf16_kernel<64, full><<<grid, block, 0, s>>>((const uint16_t *)q, (const uint16_t *)k,
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
