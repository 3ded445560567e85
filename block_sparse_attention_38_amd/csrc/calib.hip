// calib.hip -- sustained rate of the bf16 matrix cores (measurement support).
//
// The bf16 MFMA peak of an MI355X (2.5 PFLOP/s dense) is quoted at a 2.4 GHz
// shader clock.  The clock the chip sustains under a matrix-core load depends
// on the power it draws, and that depends on how many operand bits toggle: a
// loop of nothing but MFMAs on register operands runs close to the quoted peak
// with constant operands and well below it with random ones.  This kernel is
// that loop, so that a measured kernel can be set against what the matrix cores
// sustain on data like its own as well as against the quoted peak.
//
// Two workgroups of four wavefronts per CU (two wavefronts per SIMD, the
// occupancy of the attention kernels); each wavefront runs `iters` rounds of
// 16 v_mfma_f32_32x32x16_bf16 in four independent accumulator chains, with
// operands in registers and no memory access inside the loop.
#include "aba_internal.h"

namespace aba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// A 32-bit integer hash (two multiply-xorshift rounds); only a source of
// operand bits, no statistical quality is needed.
__device__ __forceinline__ uint32_t mix32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, int random, float *__restrict__ out)
{
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // random: values in [-2, 2) with every mantissa bit in play; else 0
            const float x = random ? ((int)(mix32(t * 64u + 8u * i + e) & 0xffffu) - 32768) * (1.f / 16384.f) : 0.f;
            const float y = random ? ((int)(mix32(t * 64u + 32u + 8u * i + e) & 0xffffu) - 32768) * (1.f / 16384.f)
                                   : 0.f;
            a[i][e] = (__bf16)x;
            b[i][e] = (__bf16)y;
        }
    floatx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[k], c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[(k + 1) & 3], c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + 1) & 3], b[k], c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + 2) & 3], b[(k + 3) & 3], c3, 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
    out[t] = s;   // keeps the products live
}

}  // namespace

hipError_t launch_mfma_rate(int iters, int random, float *out, hipStream_t s)
{
    mfma_rate_kernel<<<kMfmaRateBlocks, 256, 0, s>>>(iters, random, out);
    return hipGetLastError();
}

}  // namespace aba
