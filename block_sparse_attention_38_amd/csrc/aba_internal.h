// aba_internal.h -- declarations shared by the HIP sources of libaba.so.
// Kernels are written for gfx950 (CDNA4): 64-lane wavefronts, bf16 MFMA,
// 160 KB LDS per CU, 256 CUs in 8 XCDs.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace aba {

constexpr int kBlock = 128;       // tokens per query block (and per coarse key block)
constexpr int kFineBlock = 4;     // tokens per fine-grained key block
constexpr int kMaxBlocks = 1024;  // blocks per sequence the score/sample kernels hold in LDS
constexpr int kMaxFineBlocks = 32768;            // fine key blocks per sequence (N <= 131072)
constexpr int kSampleLdsLimit = 152 * 1024;      // dynamic LDS of the long-row sampler (of 160 KB per CU)
constexpr int kMaxClusters = 8;

enum Dtype : int { kF32 = 0, kBF16 = 1 };

// Host launchers; each returns the HIP status of its launch.
// k-means of every query block; for bf16 the same kernel also pools the keys
// into kbar (key blocks of kb tokens, NBk of them) and sets *pooled.
hipError_t launch_kmeans(const void *q, const void *k, int dtype, int B, int H, int N, int N_pad, int D, int NB, int C,
                         int T, int kb, int NBk, float *cent, float *weight, float *kbar, bool *pooled, hipStream_t s);
hipError_t launch_pool(const void *k, int dtype, int B, int H, int N, int N_pad, int D, int NB, float *kbar,
                       hipStream_t s);
// Draws use the global indices h0 + h and b0 + b (the call may cover a slice of a layer).
// ws: sample_workspace_bytes of device memory (rows of more than 8192 key blocks; else unused).
hipError_t launch_sample(const float *scores, int B, int H, int NBq, int NB, int K, uint64_t seed, int h0, int b0,
                         int cap, int32_t *idx, int32_t *cnt, float *w, void *ws, hipStream_t s);
// Dynamic LDS the sampler needs for rows of NB key blocks and budget K.
size_t sample_lds_bytes(int NB, int K);
// Device bytes launch_sample needs at ws (0 unless rows hold more than 8192 key blocks).
size_t sample_workspace_bytes(int B, int H, int NBq, int NB, int K);
// 4-token key pooling, and the two-pass MFMA scoring of either key block size
// (workspace: per-chunk partial statistics, per-centroid coefficients and the
// split centroid tiles).
hipError_t launch_fine_pool(const void *k, int dtype, int B, int H, int N, int N_pad, int D, int NBk, float *kbar,
                            hipStream_t s);
size_t fine_score_workspace_bytes(int B, int H, int NBq, int NBk);
hipError_t launch_fine_score(const float *cent, const float *weight, const float *kbar, int B, int H, int NBq, int NBk,
                             int C, int D, float scale, void *ws, float *scores, hipStream_t s);
hipError_t launch_attend(const void *q, const void *k, const void *v, int dtype, int B, int H, int N, int N_pad, int D,
                         int NB, float scale, const int32_t *idx, const int32_t *cnt, const float *w, int cap, bool full,
                         void *ws, void *out, hipStream_t s);
// Sparse attention over lists of 4-token key blocks (bf16 with D = 128, or fp32
// with D = 64); same workspace as launch_attend.
hipError_t launch_attend_fine(const void *q, const void *k, const void *v, int dtype, int B, int H, int N, int N_pad,
                              int D, int NBq, int NBk, float scale, const int32_t *idx, const int32_t *cnt,
                              const float *w, int cap, void *ws, void *out, hipStream_t s);
// Attention mass per key block of kb tokens (128 or 4) for the listed query blocks.
hipError_t launch_block_mass(const void *q, const void *k, int dtype, int B, int H, int N, int N_pad, int D, int NB,
                             int kb, float scale, const int32_t *items, int n_items, float *mass, hipStream_t s);
// Device bytes launch_attend needs at ws (the work order, and at head_dim 64 the V^T copy; 0 for fp32).
size_t attend_workspace_bytes(int dtype, int B, int H, int N_pad, int D);
// Sustained bf16 MFMA rate: kMfmaRateBlocks workgroups of 256 threads, each
// wavefront 16 * iters MFMAs on register operands (random bits or zeros); out
// holds one float per thread.
constexpr int kMfmaRateBlocks = 512;
hipError_t launch_mfma_rate(int iters, int random, float *out, hipStream_t s);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// Eight consecutive elements of a row as fp32.
__device__ __forceinline__ void load8(const uint16_t *p, float out[8])
{
    uint4 r = *reinterpret_cast<const uint4 *>(p);
    out[0] = bf16_lo(r.x); out[1] = bf16_hi(r.x);
    out[2] = bf16_lo(r.y); out[3] = bf16_hi(r.y);
    out[4] = bf16_lo(r.z); out[5] = bf16_hi(r.z);
    out[6] = bf16_lo(r.w); out[7] = bf16_hi(r.w);
}
__device__ __forceinline__ void load8(const float *p, float out[8])
{
    float4 a = *reinterpret_cast<const float4 *>(p);
    float4 b = *reinterpret_cast<const float4 *>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X.  Remap the
// hardware id so that every XCD (with its own L2) works through one contiguous
// range of logical ids: heads stay together and neighbouring query blocks of a
// head, which keep overlapping key blocks, share an L2.
__device__ __forceinline__ int xcd_contiguous_id(int hw_id, int n)
{
    constexpr int kXcds = 8;
    const int per = n / kXcds, extra = n % kXcds;
    const int xcd = hw_id % kXcds, k = hw_id / kXcds;
    return xcd * per + (xcd < extra ? xcd : extra) + k;
}

// Cross-lane exchanges without LDS: DPP butterflies inside 16-lane rows
// (quad_perm xor 1, xor 2; row_half_mirror and row_mirror pair the two quads of
// an 8-lane group and the two halves of a row), then v_permlane16_swap between
// rows and v_permlane32_swap between the wavefront's halves.
template <int CTRL> __device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t swap16_u32(uint32_t v, bool second)
{
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return second ? r[1] : r[0];
}
__device__ __forceinline__ uint32_t swap32_u32(uint32_t v, bool second)
{
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return second ? r[1] : r[0];
}

// x[l] + x[l ^ 32] and max(x[l], x[l ^ 32]) in every lane l (one lane swap).
__device__ __forceinline__ float xor32_sum(float x)
{
    return __uint_as_float(swap32_u32(__float_as_uint(x), false)) + __uint_as_float(swap32_u32(__float_as_uint(x), true));
}
__device__ __forceinline__ float xor32_max(float x)
{
    return fmaxf(__uint_as_float(swap32_u32(__float_as_uint(x), false)),
                 __uint_as_float(swap32_u32(__float_as_uint(x), true)));
}

// Sum and maximum over each aligned group of 8 lanes, in every lane of the group
// (the same pairing, hence the same rounding, as xor butterflies over 1, 2, 4).
__device__ __forceinline__ float group8_sum(float x)
{
    x += __uint_as_float(dpp_u32<0xB1>(__float_as_uint(x)));    // quad_perm(1, 0, 3, 2)
    x += __uint_as_float(dpp_u32<0x4E>(__float_as_uint(x)));    // quad_perm(2, 3, 0, 1)
    return x + __uint_as_float(dpp_u32<0x141>(__float_as_uint(x)));   // row_half_mirror
}
__device__ __forceinline__ float group8_max(float x)
{
    x = fmaxf(x, __uint_as_float(dpp_u32<0xB1>(__float_as_uint(x))));
    x = fmaxf(x, __uint_as_float(dpp_u32<0x4E>(__float_as_uint(x))));
    return fmaxf(x, __uint_as_float(dpp_u32<0x141>(__float_as_uint(x))));
}

// op over the 64 lanes of a wavefront, the result in every lane; op must be
// commutative and associative (sum, min, max).  T is 32 or 64 bits wide.
template <typename T, typename Op> __device__ __forceinline__ T wave_allreduce(T x, Op op)
{
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
    auto pull = [](T v, auto f) __attribute__((always_inline)) {
        if constexpr (sizeof(T) == 4) {
            return __builtin_bit_cast(T, f(__builtin_bit_cast(uint32_t, v)));
        } else {
            const uint64_t u = __builtin_bit_cast(uint64_t, v);
            const uint64_t lo = f((uint32_t)u), hi = f((uint32_t)(u >> 32));
            return __builtin_bit_cast(T, lo | (hi << 32));
        }
    };
    x = op(x, pull(x, [](uint32_t v) { return dpp_u32<0xB1>(v); }));    // quad_perm(1, 0, 3, 2)
    x = op(x, pull(x, [](uint32_t v) { return dpp_u32<0x4E>(v); }));    // quad_perm(2, 3, 0, 1)
    x = op(x, pull(x, [](uint32_t v) { return dpp_u32<0x141>(v); }));   // row_half_mirror
    x = op(x, pull(x, [](uint32_t v) { return dpp_u32<0x140>(v); }));   // row_mirror
    x = op(pull(x, [](uint32_t v) { return swap16_u32(v, false); }), pull(x, [](uint32_t v) { return swap16_u32(v, true); }));
    x = op(pull(x, [](uint32_t v) { return swap32_u32(v, false); }), pull(x, [](uint32_t v) { return swap32_u32(v, true); }));
    return x;
}

// Inclusive prefix sum over the 64 lanes of a wavefront (32- or 64-bit integers
// or floats): Hillis-Steele inside each 16-lane row (row_shr 1, 2, 4, 8; lanes
// shifted in from outside the row read 0), then the last lane of rows 0 and 2
// into rows 1 and 3 (row_bcast:15) and the last lane of row 1 into rows 2 and 3
// (row_bcast:31).
template <typename T> __device__ __forceinline__ T wave_incl_scan_dpp(T x)
{
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
    auto step = [&](auto f) __attribute__((always_inline)) {
        if constexpr (sizeof(T) == 4) {
            x = x + __builtin_bit_cast(T, f(__builtin_bit_cast(uint32_t, x)));
        } else {
            const uint64_t u = __builtin_bit_cast(uint64_t, x);
            const uint64_t lo = f((uint32_t)u), hi = f((uint32_t)(u >> 32));
            x = x + __builtin_bit_cast(T, lo | (hi << 32));
        }
    };
#define ABA_DPP_STEP(ctrl, rows) \
    step([](uint32_t v) { return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, rows, 0xF, true); })
    ABA_DPP_STEP(0x111, 0xF);   // row_shr:1
    ABA_DPP_STEP(0x112, 0xF);   // row_shr:2
    ABA_DPP_STEP(0x114, 0xF);   // row_shr:4
    ABA_DPP_STEP(0x118, 0xF);   // row_shr:8
    ABA_DPP_STEP(0x142, 0xA);   // row_bcast:15 into rows 1 and 3
    ABA_DPP_STEP(0x143, 0xC);   // row_bcast:31 into rows 2 and 3
#undef ABA_DPP_STEP
    return x;
}

// The value of x in lane l (l the same in every lane of the wavefront).
template <typename T> __device__ __forceinline__ T lane_value(T x, int l)
{
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
    } else {
        const uint64_t u = __builtin_bit_cast(uint64_t, x);
        const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
        const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
        return __builtin_bit_cast(T, lo | (hi << 32));
    }
}

__device__ __forceinline__ float wave_max(float x)
{
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x)
{
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// ---------------------------------------------------------------------------
// Buffer -> LDS direct loads (used by the attention and 4-token scoring kernels)
// ---------------------------------------------------------------------------
typedef int int4v __attribute__((ext_vector_type(4)));

// Buffer descriptor over one slice of device memory (base, stride 0, size in
// bytes, raw dword access): the loads below address it by byte offset, and the
// hardware range check returns zeros past its end.
__device__ __forceinline__ int4v head_rsrc(const void *base, int bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return int4v{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff)), bytes, 0x00020000};
}

__device__ __forceinline__ uint32_t lds_address(char *p)
{
    return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char *)p);
}

// Direct copy of 16 bytes per lane from a buffer into LDS: lane L's bytes land
// at dst + 16 L (dst is wavefront-uniform; M0 holds its LDS address).  Issued
// as inline assembly: the compiler then does not track these LDS writes, and
// would otherwise wait for every copy in flight before each LDS read it cannot
// prove disjoint from them.  Ordering is explicit instead: a slot is read only
// after wait_loads_and_sync has covered the copies into it, and is refilled
// only after the barrier that follows its last read.
__device__ __forceinline__ void load_lds16(int4v rs, int voff, int soff, char *dst)
{
    const uint32_t m0 = lds_address(dst);
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rs), "s"(soff), "{m0}"(m0)
                 : "memory");
}

// The same with 4 bytes per lane (lane L's bytes land at dst + 4 L).
__device__ __forceinline__ void load_lds4(int4v rs, int voff, int soff, char *dst)
{
    const uint32_t m0 = lds_address(dst);
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(rs), "s"(soff), "{m0}"(m0)
                 : "memory");
}

// Wait until at most n of this wavefront's vector memory operations are in
// flight (they complete in issue order), then meet the other wavefronts: their
// direct loads up to the same point are then in LDS as well.  A bare
// s_barrier: the workgroup fence of __syncthreads would also wait for the loads
// that are meant to stay in flight.  Every LDS read before the barrier has been
// consumed by then.
template <int n> __device__ __forceinline__ void wait_loads_and_sync()
{
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(n) : "memory");
}

// The same for code that also writes LDS with ordinary stores before the
// barrier: those must land (lgkmcnt) before another wavefront reads them.
template <int n> __device__ __forceinline__ void wait_loads_lds_and_sync()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(n) : "memory");
}

}  // namespace aba
