// diag.hip -- attention mass per key block, for the selection diagnostics
// (gfx950).
//
// AB-Attention page, IBCS paragraph and the opening of section "Три приёма
// AB-Attention": the quality of a block selection is the share of the dense
// attention mass its blocks hold; the best K blocks hold the ideal top-K mass.
// For a query block b' with n valid query rows,
//     M[b', j] = (1/n) sum_i sum_{t in key block j} softmax_t(s q_i . k_t),
// so every row of M sums to one.  Key blocks are 128 tokens, or 4 tokens for
// the fine-grained selection of the page's kernel paragraph.  Not on the
// attention path: it exists to measure how much of M the sampled (or scored)
// blocks keep.
//
// One workgroup of 4 wavefronts per listed query block; wavefront w owns query
// rows [32w, 32w + 32) as the MFMA column of S^T = K Q^T (32x32x16 bf16 MFMA,
// fp32 accumulation, K fragments read straight from global memory).  Pass 1
// walks every key for the row maxima and normalisers; pass 2 walks them again
// and adds the normalised probabilities of each key block, reduced over the
// wavefront's lanes and then over the four wavefronts in LDS.
#include "aba_internal.h"

namespace aba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

template <int D, bool fine>
__global__ __launch_bounds__(256) void block_mass_kernel(const uint16_t *__restrict__ q,
                                                         const uint16_t *__restrict__ k,
                                                         const int32_t *__restrict__ items, int B, int H, int N,
                                                         int N_pad, int NB, int NBk, float scale_log2,
                                                         float *__restrict__ mass)
{
    constexpr int KS = D / 16;
    constexpr int kPart = fine ? kBlock / kFineBlock : kMaxBlocks;   // per-wavefront partial sums kept in LDS
    __shared__ float part[4][kPart];
    const int it = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, half = lane >> 5;
    float *out = mass + (long)it * NBk;

    const int b = items[3 * it], h = items[3 * it + 1], qb = items[3 * it + 2];
    if (b < 0 || b >= B || h < 0 || h >= H || qb < 0 || qb >= NB) {   // an item outside the layer: zeros
        for (int j = tid; j < NBk; j += 256) out[j] = 0.f;
        return;
    }
    const long bh = (long)b * H + h;
    const uint16_t *qh = q + bh * N_pad * D, *kh = k + bh * N_pad * D;
    const int nq = min(kBlock, N - qb * kBlock);
    const int qrow = qb * kBlock + 32 * wave + l32;
    const bool qvalid = qrow < N;

    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (qvalid) raw = *reinterpret_cast<const uint4 *>(qh + (long)qrow * D + 16 * ks + 8 * half);
        qf[ks] = __builtin_bit_cast(bf16x8, raw);
    }

    // S^T for keys [key0, key0 + 32): lane (l32, half) element r is key
    // key0 + 8(r/4) + 4half + r%4 of query l32, in log2 units; keys >= N -> -inf.
    auto tile = [&](int key0, floatx16 &s) {
        const int kr = min(key0 + l32, N - 1);   // rows past N are read from a valid row, then masked
        s = floatx16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint4 raw = *reinterpret_cast<const uint4 *>(kh + (long)kr * D + 16 * ks + 8 * half);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, raw), qf[ks], s, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = key0 + 8 * (r >> 2) + 4 * half + (r & 3);
            s[r] = key < N ? s[r] * scale_log2 : -INFINITY;
        }
    };
    auto pair_sum = [](float x) { return x + __shfl_xor(x, 32, 64); };
    auto pair_max = [](float x) { return fmaxf(x, __shfl_xor(x, 32, 64)); };

    // pass 1: row max and normaliser (exact online rescaling)
    float m = -INFINITY, l = 0.f;
    for (int key0 = 0; key0 < N; key0 += 32) {
        floatx16 s;
        tile(key0, s);
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = pair_max(mx);
        const float m_new = fmaxf(m, mx);
        float add = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) add += __builtin_amdgcn_exp2f(s[r] - m_new);
        l = l * __builtin_amdgcn_exp2f(m - m_new) + pair_sum(add);
        m = m_new;
    }
    const float inv = qvalid ? 1.f / ((float)nq * l) : 0.f;

    // pass 2: normalised probabilities summed per key block
    if (!fine) {
        for (int j = 0; j < NB; ++j) {
            float acc = 0.f;
            for (int key0 = j * kBlock; key0 < min(N, (j + 1) * kBlock); key0 += 32) {
                floatx16 s;
                tile(key0, s);
#pragma unroll
                for (int r = 0; r < 16; ++r) acc += __builtin_amdgcn_exp2f(s[r] - m);
            }
            acc = wave_sum(acc * inv);
            if (lane == 0) part[wave][j] = acc;
        }
        __syncthreads();
        for (int j = tid; j < NBk; j += 256) out[j] = part[0][j] + part[1][j] + part[2][j] + part[3][j];
    } else {
        // 4-token blocks: element r of a 32-key tile is in block key0/4 + 2(r/4) + half;
        // each 128-key stretch fills part[][0..32) and is flushed after a barrier
        for (int j = 0; j < NB; ++j) {
            for (int t = 0; t < kBlock / 32; ++t) {
                const int key0 = j * kBlock + 32 * t;
                float g[4] = {0.f, 0.f, 0.f, 0.f};
                if (key0 < N) {
                    floatx16 s;
                    tile(key0, s);
#pragma unroll
                    for (int r = 0; r < 16; ++r) g[r >> 2] += __builtin_amdgcn_exp2f(s[r] - m);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = g[i] * inv;
#pragma unroll
                    for (int o = 1; o < 32; o <<= 1) x += __shfl_xor(x, o, 64);   // over the 32 query lanes of a half
                    if (l32 == 0) part[wave][8 * t + 2 * i + half] = x;
                }
            }
            __syncthreads();
            const int jj = j * kPart + tid;
            if (tid < kPart && jj < NBk) out[jj] = part[0][tid] + part[1][tid] + part[2][tid] + part[3][tid];
            __syncthreads();
        }
    }
}

}  // namespace

hipError_t launch_block_mass(const void *q, const void *k, int dtype, int B, int H, int N, int N_pad, int D, int NB,
                             int kb, float scale, const int32_t *items, int n_items, float *mass, hipStream_t s)
{
    if (n_items <= 0) return hipSuccess;
    const dim3 grid((unsigned)n_items), block(256);
    const float sl2 = scale * kLog2e;
    const int NBk = (N + kb - 1) / kb;
    const uint16_t *q16 = (const uint16_t *)q, *k16 = (const uint16_t *)k;
    if (dtype != kBF16 || (kb != kBlock && kb != kFineBlock)) return hipErrorInvalidValue;
    if (D == 128 && kb == kBlock)
        block_mass_kernel<128, false><<<grid, block, 0, s>>>(q16, k16, items, B, H, N, N_pad, NB, NBk, sl2, mass);
    else if (D == 128)
        block_mass_kernel<128, true><<<grid, block, 0, s>>>(q16, k16, items, B, H, N, N_pad, NB, NBk, sl2, mass);
    else if (D == 64 && kb == kBlock)
        block_mass_kernel<64, false><<<grid, block, 0, s>>>(q16, k16, items, B, H, N, N_pad, NB, NBk, sl2, mass);
    else if (D == 64)
        block_mass_kernel<64, true><<<grid, block, 0, s>>>(q16, k16, items, B, H, N, N_pad, NB, NBk, sl2, mass);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace aba
