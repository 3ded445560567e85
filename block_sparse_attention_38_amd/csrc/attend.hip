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

// LDS layout of one stage.  Rows are padded instead of swizzled, so every LDS
// address is a per-lane base plus a compile-time offset:
//   K    64 rows x D bf16, row pitch D*2 + 16 bytes: the 16 rows one 16-lane
//        phase of a 128-bit read touches start 4 banks apart;
//   V^T  D rows x 64 keys, row pitch 136 bytes: the 32 rows one phase of a
//        64-bit read touches cover all 64 banks.
template <int D> struct Lds {
    static constexpr int kPitch = D * 2 + 16;
    static constexpr int vPitch = kSub * 2 + 8;
    static constexpr int kBytes = kSub * kPitch;
    static constexpr int vBytes = D * vPitch;
    static constexpr int stage = kBytes + vBytes;
};

__device__ __forceinline__ uint32_t perm_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t perm_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Global -> register staging of one 64-key sub-tile (each thread holds its
// share until it is written to LDS after the current sub-tile is computed).
// Thread (c, r0) moves 16-byte chunk c of K rows r0 + 16i and of V rows
// 4*r0' .. 4*r0'+3 (keys of one 8-byte V^T slot).
template <int D> struct Stage {
    static constexpr int kChunks = D / 8;
    static constexpr int kRowsPerPass = 256 / kChunks;
    static constexpr int kKLoads = kSub / kRowsPerPass;       // 16-byte K chunks per thread
    static constexpr bool kVAll = (kSub / 4) >= kRowsPerPass; // every thread moves one V quad
    uint4 k[kKLoads];
    uint4 v[4];
};

// full: every key of the sub-tile is valid (no bounds checks); otherwise rows
// >= N and the whole sub-tile when !active read as zero.
template <int D>
__device__ __forceinline__ void stage_load(Stage<D> &st, const uint16_t *kb, const uint16_t *vb, int valid, bool full,
                                           int tid)
{
    constexpr int kChunks = D / 8, RP = Stage<D>::kRowsPerPass;
    const int c = tid % kChunks, r0 = tid / kChunks;
    const uint16_t *kp = kb + r0 * D + 8 * c;
    const uint16_t *vp = vb + 4 * r0 * D + 8 * c;
    const bool vq = Stage<D>::kVAll || r0 < kSub / 4;
    if (full) {
#pragma unroll
        for (int i = 0; i < Stage<D>::kKLoads; ++i) st.k[i] = *reinterpret_cast<const uint4 *>(kp + i * RP * D);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            st.v[rr] = vq ? *reinterpret_cast<const uint4 *>(vp + rr * D) : make_uint4(0, 0, 0, 0);
    } else {
#pragma unroll
        for (int i = 0; i < Stage<D>::kKLoads; ++i)
            st.k[i] = (r0 + i * RP < valid) ? *reinterpret_cast<const uint4 *>(kp + i * RP * D) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            st.v[rr] = (vq && 4 * r0 + rr < valid) ? *reinterpret_cast<const uint4 *>(vp + rr * D) : make_uint4(0, 0, 0, 0);
    }
}

template <int D>
__device__ __forceinline__ void stage_store(const Stage<D> &st, char *stage_base, int tid)
{
    using L = Lds<D>;
    constexpr int kChunks = D / 8, RP = Stage<D>::kRowsPerPass;
    const int c = tid % kChunks, r0 = tid / kChunks;
    char *kbase = stage_base + r0 * L::kPitch + 16 * c;
#pragma unroll
    for (int i = 0; i < Stage<D>::kKLoads; ++i) *reinterpret_cast<uint4 *>(kbase + i * RP * L::kPitch) = st.k[i];
    if (Stage<D>::kVAll || r0 < kSub / 4) {
        // V^T rows 8c .. 8c+7, slot r0 (keys 4r0 .. 4r0+3)
        char *vbase = stage_base + L::kBytes + 8 * c * L::vPitch + 8 * r0;
        const uint32_t *a = reinterpret_cast<const uint32_t *>(&st.v[0]);
        const uint32_t *b = reinterpret_cast<const uint32_t *>(&st.v[1]);
        const uint32_t *e = reinterpret_cast<const uint32_t *>(&st.v[2]);
        const uint32_t *f = reinterpret_cast<const uint32_t *>(&st.v[3]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            *reinterpret_cast<uint2 *>(vbase + (2 * p) * L::vPitch) = make_uint2(perm_lo(a[p], b[p]), perm_lo(e[p], f[p]));
            *reinterpret_cast<uint2 *>(vbase + (2 * p + 1) * L::vPitch) =
                make_uint2(perm_hi(a[p], b[p]), perm_hi(e[p], f[p]));
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

template <int D>
__device__ __forceinline__ void load_subtile(Stage<D> &st, const uint16_t *kh, const uint16_t *vh, Entry en, int half_idx,
                                             int N, int tid)
{
    const int key0 = en.j * kBlock + kSub * half_idx;
    const int valid = (en.j < 0) ? 0 : min(kSub, N - key0);
    stage_load<D>(st, kh + (long)key0 * D, vh + (long)key0 * D, valid, valid == kSub, tid);
}

template <int D, bool full>
__global__ __launch_bounds__(256, 2) void attend_bf16_kernel(
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

    // per-lane LDS read bases (constant offsets are added per instruction)
    const int k_rd = l32 * L::kPitch + 16 * half;
    const int v_rd = L::kBytes + l32 * L::vPitch + 8 * half;

    Stage<D> st;
    Entry cur{-1, 0.f};
    if (n_sub > 0) {
        cur = list_entry<full>(lrow, wrow, 0, NB);
        load_subtile<D>(st, kh, vh, cur, 0, N, tid);
        stage_store<D>(st, lds, tid);
    }
    __syncthreads();

    for (int u = 0; u < n_sub; ++u) {
        char *cur_stage = lds + (u & 1) * L::stage;
        // prefetch the next sub-tile into registers; it lands while this one is computed
        Entry nxt = cur;
        if (u + 1 < n_sub) {
            if (u & 1) nxt = list_entry<full>(lrow, wrow, (u + 1) >> 1, NB);
            load_subtile<D>(st, kh, vh, nxt, (u + 1) & 1, N, tid);
        }

        const int key0 = cur.j * kBlock + kSub * (u & 1);
        if (cur.j >= 0 && key0 < N) {   // uniform over the workgroup
            // S^T = K Q^T: tile kt holds keys [32kt, 32kt+32) of the sub-tile x this
            // wave's 32 queries; lane (l32, half) holds key 32kt + 8(r/4) + 4half + r%4.
            floatx16 s[KT];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const char *kr = cur_stage + k_rd + kt * 32 * L::kPitch;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const uint4 a = *reinterpret_cast<const uint4 *>(kr + 32 * ks);
                    s[kt] = mfma32(__builtin_bit_cast(bf16x8, a), qf[ks], ks == 0 ? zero16 : s[kt]);
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
            // element e is key 32kt + 16sub + 8(e/4) + 4h + e%4, i.e. V^T slots
            // 8kt + 4sub + h and 8kt + 4sub + h + 2.
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const char *vr = cur_stage + v_rd + dt * 32 * L::vPitch;
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                    for (int sub = 0; sub < 2; ++sub) {
                        const uint2 a0 = *reinterpret_cast<const uint2 *>(vr + 8 * (8 * kt + 4 * sub));
                        const uint2 a1 = *reinterpret_cast<const uint2 *>(vr + 8 * (8 * kt + 4 * sub + 2));
                        const uint4 a = make_uint4(a0.x, a0.y, a1.x, a1.y);
                        o[dt] = mfma32(__builtin_bit_cast(bf16x8, a), pb[kt][sub], o[dt]);
                    }
            }
        }

        if (u + 1 < n_sub) stage_store<D>(st, lds + ((u + 1) & 1) * L::stage, tid);
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
