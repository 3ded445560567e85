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
// bf16 path (the hot path):
//   attend_bf16   one workgroup of 4 wavefronts per (b, h, query block), two
//                 workgroups per CU (two wavefronts per SIMD); wavefront w owns
//                 query rows [32w, 32w + 32).  A kept key block is two 64-key
//                 sub-tiles of K and V rows, each copied by buffer->LDS direct
//                 loads into LDS slots while earlier ones are computed; one
//                 barrier per sub-tile.  Per sub-tile:
//   S^T = K Q^T      32x32x16 bf16 MFMA, K from LDS, Q fragments in registers
//   online softmax   in the exp2 domain; the block's log2(w_j) is added to its
//                    logits, so the weight enters numerator and normaliser; the
//                    running max moves only when it grows by more than 2^8
//   O^T += V^T P^T   32x32x16 bf16 MFMA, P^T straight from the S^T accumulators,
//                    the V^T operand by transposing LDS reads of the row-major
//                    V tile (ds_read_b64_tr_b16, head_dim 128); at head_dim 64
//                    a pre-pass (vt_kernel) writes V^T tiles instead.
// Computing the transposed products makes every lane own one query column, so
// row statistics need a single cross-half exchange (v_permlane32_swap) and the
// rescale of O is a per-lane scalar multiply.  LDS fragment reads are issued
// four MFMAs ahead of their use, the second key tile's probabilities are
// computed between the first tile's PV MFMAs, and the wavefront raises its
// priority while it issues MFMAs, so that the other wavefront of the SIMD
// fills the softmax gaps rather than competing for the matrix pipe.
//
// fp32 path: a plain VALU kernel (pairs of lanes per query row) for fp32
// inputs with head_dim 64.
#include "aba_internal.h"

#include <type_traits>

namespace aba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

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
// A workgroup covers one 128-row query block with four wavefronts of 32 rows
// (one 32x32 MFMA tile of queries each); two workgroups share a CU, so every
// SIMD runs two wavefronts.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// ---------------------------------------------------------------------------
// V^T staging (head_dim 64).  The PV product contracts over keys, so its MFMA
// operand wants each lane's 8 keys of one head dimension contiguous.  A
// pre-pass writes V once per call as, for every (b, h) and 64-key sub-tile s,
// a [D][64] bf16 tile whose row d holds v[64s + .][d] with key order vt_key():
// inside each group of 16 keys, positions 4..7 and 8..11 are exchanged.  Lane
// half h of an MFMA then finds its keys 8(e/4) + 4h + e%4 (e = 0..7, the order
// in which the S^T accumulators hand over P^T) at positions 8h .. 8h+7: one
// 16-byte LDS read.  Keys >= N are written as zero.  The tiles occupy the same
// B*H*N_pad*D elements as v.  At head_dim 128 the kernels read v itself (see
// "Transposing reads of V" below).
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int vt_key(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

template <int D>
__global__ __launch_bounds__(256) void vt_kernel(const uint16_t *__restrict__ v, int N, int N_pad,
                                                 uint16_t *__restrict__ vt)
{
    constexpr int kRow = D + 2;                 // odd word stride: the column reads spread over banks
    constexpr int kChunks = kSub * D / 8;       // 16-byte chunks per tile
    __shared__ uint32_t tile[kSub * kRow / 2];
    const int tiles = N_pad / kSub;
    const int s = blockIdx.x % tiles;
    const long bh = blockIdx.x / tiles;
    const uint16_t *src = v + (bh * N_pad + (long)kSub * s) * D;
    const int valid = N - kSub * s;
    for (int i = threadIdx.x; i < kChunks; i += 256) {
        const int r = i / (D / 8), c = i % (D / 8);
        uint4 x = make_uint4(0, 0, 0, 0);
        if (r < valid) x = *reinterpret_cast<const uint4 *>(src + (long)r * D + 8 * c);
        uint32_t *t = tile + (r * kRow + 8 * c) / 2;
        t[0] = x.x;
        t[1] = x.y;
        t[2] = x.z;
        t[3] = x.w;
    }
    __syncthreads();
    const uint16_t *t16 = reinterpret_cast<const uint16_t *>(tile);
    uint4 *dst = reinterpret_cast<uint4 *>(vt + (bh * N_pad + (long)kSub * s) * D);
    for (int i = threadIdx.x; i < kChunks; i += 256) {
        const int d = i / (kSub / 8), c = i % (kSub / 8);   // row d, positions 8c .. 8c+7
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const int k0 = 16 * (c >> 1) + vt_key(8 * (c & 1) + e);
            const int k1 = 16 * (c >> 1) + vt_key(8 * (c & 1) + e + 1);
            w[e / 2] = (uint32_t)t16[k0 * kRow + d] | ((uint32_t)t16[k1 * kRow + d] << 16);
        }
        dst[i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// LDS layout of one stage, unpadded (one direct global->LDS load fills whole
// rows), with XOR swizzles of the 16-byte chunks:
//   K   [64 keys][D]:  chunk c of row r at c ^ (r % 16), so the 16 rows one
//       16-lane phase of a 128-bit read touches hit 16 different chunks;
//   V   [64 keys][D] (head_dim 128): chunk c of row r at c ^ 4 (r % 4), which
//       keeps the transposing reads below free of bank conflicts;
//   V^T [D][64 keys] (head_dim 64): chunk c of row r at c ^ ((r / 2) % 8);
//       with 128-byte rows, 16 consecutive rows then cover every bank once.
// Three K slots and two V slots: K sub-tiles are loaded two sub-tiles ahead of
// their use and V one and a half (the PV product comes after the softmax),
// which hides the latency of key blocks gathered from beyond the L2.  80 KB at
// D = 128, so two workgroups fill the 160 KB of a CU.
//
// Transposing reads of V (head_dim 128).  ds_read_b64_tr_b16 works in groups of
// 16 lanes: lane m of a group points at 4 consecutive bf16 values, and lane i
// receives value i % 4 of the pieces of lanes 4j + i / 4, j = 0..3 (measured
// with an in-bounds probe).  So if lane m points at row 4 (g / 2) + m / 4 and
// dimensions 32 dt + 16 (g % 2) + 4 (m % 4) (g = lane / 16), lane i receives
// rows 4 (g / 2) + j of dimension 32 dt + 16 (g % 2) + i: for MFMA lane (l32,
// half) the keys 4 half + j of dimension 32 dt + l32, and a second read 8 rows
// further gives keys 8 + 4 half + j -- the order of P^T in the accumulators.
// The row offsets of a k-step are immediates; the swizzle depends only on row
// % 4, which those offsets keep.  Rows of v past N are read through a buffer
// descriptor that ends at row N (the row offset in the range-checked per-lane
// offset), so they arrive as zeros.  No V^T copy of v is made.
template <int D> struct Lds {
    static constexpr int pitch = D * 2;        // K row bytes
    static constexpr int chunks = D / 8;
    static constexpr int kBytes = kSub * pitch;
    static constexpr int vPitch = kSub * 2;    // V^T row bytes
    static constexpr int vBytes = D * vPitch;
    static constexpr int kSlots = 3, vSlots = 2;
    static constexpr int bytes = kSlots * kBytes + vSlots * vBytes;
};
template <int D> __device__ __forceinline__ int k_swz(int r) { return r & (Lds<D>::chunks - 1); }
__device__ __forceinline__ int vt_swz(int r) { return (r >> 1) & 7; }
// row-major V tiles read by transposing LDS reads (D = 128): chunk c of row r at c ^ 4 (r % 4)
__device__ __forceinline__ int vr_swz(int r) { return 4 * (r & 3); }
template <int D> constexpr bool v_rows() { return D == 128; }

// One PV operand (8 bf16) from a row-major V tile: two transposing reads, keys
// p and p + 8 rows below (see the lane layout where the offsets are formed).
template <int D> __device__ __forceinline__ bf16x8 v_frag_tr(const char *p)
{
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)p);
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p + 8 * 2 * D));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Direct loads of one 64-key sub-tile: K rows key0 .. key0+63 into a K slot,
// the matching V rows (D = 128) or V^T tile (D = 64) into a V slot.  Every load
// moves 1024 bytes: whole rows (4 at D = 128) or 8 V^T rows.  The per-lane byte
// offsets inside a sub-tile are precomputed; the sub-tile's own offset is a
// scalar for K and V^T, and part of the range-checked per-lane offset for V
// rows (so rows >= N read as 0).  Rows of K past N are read as they are (they
// lie inside the padded sequence) and masked after the product.  A slot is
// read only after a vmcnt wait and a barrier.
template <int D, int W = kWaves> struct Dma {
    static constexpr int loads = Lds<D>::kBytes / 1024 / W;       // per tensor and wavefront (W wavefronts)
    static constexpr int k_rows = 1024 / Lds<D>::pitch;             // K rows per load
    static constexpr int k_period = 16 / k_rows;                    // loads per K swizzle period
    int k[k_period];
    int v[2];                                                       // V rows: one period; V^T: 2 loads
};

template <int D, int W = kWaves>
__device__ __forceinline__ Dma<D, W> dma_offsets(int wave, int lane)
{
    using L = Lds<D>;
    using O = Dma<D, W>;
    O off;
    const int k0 = O::loads * O::k_rows * wave, v0 = O::loads * 8 * wave;
#pragma unroll
    for (int t = 0; t < O::k_period; ++t) {
        const int r = k0 + O::k_rows * t + lane / L::chunks, pc = lane % L::chunks;
        off.k[t] = r * L::pitch + 16 * (pc ^ k_swz<D>(r));
    }
    if (v_rows<D>()) {
        // a load fills 4 rows: lane L row L / 16 (row % 4 == L / 16), LDS chunk L % 16
        const int r = O::loads * 4 * wave + lane / 16, pc = lane % 16;
        off.v[0] = r * L::pitch + 16 * (pc ^ vr_swz(r));
        off.v[1] = off.v[0];
    } else {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int r = v0 + 8 * t + lane / 8, pc = lane % 8;
            off.v[t] = r * L::vPitch + 16 * (pc ^ vt_swz(r));
        }
    }
    return off;
}

// Issue the direct loads of K rows key0 .. key0+63 into a K slot, or of the
// matching V rows or V^T tile into a V slot (wavefront w fills its share).
template <int D, int W = kWaves>
__device__ __forceinline__ void issue_k(int4v rk, int key0, char *slot, int wave, const Dma<D, W> &off)
{
    using L = Lds<D>;
    using O = Dma<D, W>;
    const int base = key0 * D * 2;
    char *dst = slot + O::loads * 1024 * wave;
#pragma unroll
    for (int t = 0; t < O::loads; ++t)
        load_lds16(rk, off.k[t % O::k_period], base + (t / O::k_period) * 16 * L::pitch, dst + 1024 * t);
}

template <int D, int W = kWaves>
__device__ __forceinline__ void issue_v(int4v rv, int key0, char *slot, int wave, const Dma<D, W> &off)
{
    using L = Lds<D>;
    using O = Dma<D, W>;
    const int base = key0 * D * 2;   // a V^T tile sits where its keys' rows of v do
    char *dst = slot + O::loads * 1024 * wave;
    if (v_rows<D>()) {
        // rows of v itself; the row offset goes in the per-lane offset, which the
        // buffer range check covers, so rows >= N (past the descriptor) read as 0
#pragma unroll
        for (int t = 0; t < O::loads; ++t) load_lds16(rv, off.v[0] + base + t * 4 * L::pitch, 0, dst + 1024 * t);
    } else {
#pragma unroll
        for (int t = 0; t < O::loads; ++t) load_lds16(rv, off.v[t % 2], base + (t / 2) * 16 * L::vPitch, dst + 1024 * t);
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

// ---------------------------------------------------------------------------
// Work order.  The order is cut into 8 contiguous ranges of query blocks.  The
// hardware hands workgroup i to XCD i % 8 and each XCD starts its workgroups in
// increasing i; with xcd_contiguous_id each XCD works through one range, else
// the ranges run one after the other, each spread over all XCDs (mapped_slot).
// A query block's cost is its kept count, which varies several-fold between
// blocks, so every range is reordered by decreasing count (longest first),
// which keeps the tail of the launch short.  The reordering stays inside
// windows of kOrderWindow consecutive query blocks when the histogram has room
// for it (128-token key blocks at up to 32K tokens): the workgroups an XCD runs
// at once then come from neighbouring query blocks of one head, whose lists
// overlap, and share more of its L2.  One workgroup per range: an LDS histogram
// of (window, count), a scan from high counts to low, and an atomic scatter.
// The order inside one count is arbitrary; results do not depend on it (each
// query block is computed by one workgroup, independently of the others).
// ---------------------------------------------------------------------------
// Which workgroup runs which slot of the order.  With xcd_ranges each XCD
// works through one contiguous range of slots (its L2 then sees neighbouring
// query blocks of one head); otherwise slots go round-robin over the XCDs, so
// that all of them work on the same few heads at once.  The second keeps the
// K and V in use inside the MALL when the layer's K and V do not fit there as a
// whole (see attend_xcd_ranges).
__device__ __forceinline__ int mapped_slot(bool xcd_ranges)
{
    return xcd_ranges ? xcd_contiguous_id(blockIdx.x, gridDim.x) : (int)blockIdx.x;
}

constexpr int kOrderThreads = 1024;
constexpr int kOrderBins = kMaxFineBlocks / (kSub / kFineBlock) + 1;   // cost ranks: 0 .. ceil(cap / unit)
constexpr int kOrderWindow = 128;

// cnt[i] entries cost ceil(cnt[i] / unit) units of work (unit = 1 for 128-token
// key blocks, 16 for 4-token key blocks: one 64-key sub-tile).
__global__ __launch_bounds__(kOrderThreads) void order_kernel(const int32_t *__restrict__ cnt, int G, int cap, int unit,
                                                             int32_t *__restrict__ order)
{
    __shared__ int bins[kOrderBins];
    __shared__ int part[kOrderThreads / 64];
    constexpr int kXcds = 8;
    const int x = blockIdx.x, per = G / kXcds, extra = G % kXcds;
    const int start = x * per + (x < extra ? x : extra), n = per + (x < extra ? 1 : 0);
    const int capu = (cap + unit - 1) / unit;
    const int wins = (n + kOrderWindow - 1) / kOrderWindow;
    const bool windowed = (long)wins * (capu + 1) <= kOrderBins;
    const int nb = (windowed ? wins : 1) * (capu + 1), tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    auto key = [&](int i) {   // window, then cost rank (0 for the largest possible cost)
        const int c = cnt[start + i];
        const int u = c <= 0 ? 0 : (c >= cap ? capu : (c + unit - 1) / unit);
        return (windowed ? (i / kOrderWindow) * (capu + 1) : 0) + capu - u;
    };
    for (int b = tid; b < nb; b += kOrderThreads) bins[b] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kOrderThreads) atomicAdd(&bins[key(i)], 1);
    __syncthreads();
    // exclusive scan of bins[0 .. nb): each thread owns a run of consecutive bins
    constexpr int kRun = (kOrderBins + kOrderThreads - 1) / kOrderThreads;
    int run[kRun], sum = 0;
#pragma unroll
    for (int r = 0; r < kRun; ++r) {
        const int b = tid * kRun + r;
        run[r] = b < nb ? bins[b] : 0;
        sum += run[r];
    }
    int incl = sum;   // inclusive scan of the per-thread sums: wavefront, then across wavefronts
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
    }
    if (lane == 63) part[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int v = 0; v < wave; ++v) base += part[v];
    int off = base + incl - sum;
#pragma unroll
    for (int r = 0; r < kRun; ++r) {
        const int b = tid * kRun + r;
        if (b < nb) bins[b] = off;
        off += run[r];
    }
    __syncthreads();
    for (int i = tid; i < n; i += kOrderThreads) order[start + atomicAdd(&bins[key(i)], 1)] = start + i;
}

// The list of a sparse row is read 64 entries at a time into lane-distributed
// registers (lane i: entry 64m + i, already validated and turned into log2 w),
// and an entry is taken with v_readlane: no memory access per entry, so no
// scalar load shares the LDS wait counter with the fragment reads.
struct Window {
    int j;
    float lw;
};

template <bool full>
__device__ __forceinline__ Window load_window(const int32_t *lrow, const float *wrow, int m, int n_list, int NB, int lane)
{
    const int e = 64 * m + lane;
    Window win{-1, 0.f};
    if (!full && e < n_list) {
        const Entry en = list_entry<false>(lrow, wrow, e, NB);
        win.j = en.j;
        win.lw = en.lw;
    }
    return win;
}

template <bool full> __device__ __forceinline__ Entry window_entry(const Window &win, int e)
{
    if (full) return Entry{e, 0.f};
    return Entry{__builtin_amdgcn_readlane(win.j, e & 63),
                 __int_as_float(__builtin_amdgcn_readlane(__float_as_int(win.lw), e & 63))};
}

__device__ __forceinline__ float max2(float a, float b) { return __builtin_fmaxf(a, b); }

// Raw v_max3_f32 / v_max_f32 on values that are never NaN (products of finite
// bf16 operands, or -inf where masked): without the operand canonicalisation
// the compiler adds around fmaxf.
__device__ __forceinline__ float vmax3(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float vmax(float a, float b)
{
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Maximum of the 32 values of two S^T accumulator tiles of one lane: two
// independent v_max3 chains of 16 values each.
__device__ __forceinline__ float tile_max(const floatx16 &a, const floatx16 &b)
{
    float x = vmax3(a[0], a[1], a[2]), y = vmax3(b[0], b[1], b[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
        x = vmax3(x, a[r], a[r + 1]);
        y = vmax3(y, b[r], b[r + 1]);
    }
    return vmax3(vmax(x, a[15]), y, b[15]);
}

// l += p[e - 1] + p[e] for the bf16 probabilities of one pair (e odd): one
// v_dot2 against (1, 1), so the softmax normaliser sums exactly the rounded
// values the PV product multiplies.
__device__ __forceinline__ void row_sum_pair(const bf16x8 &p, int e, float &l)
{
    const bf16x2 pair = {p[e - 1], p[e]};
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    l = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, l, false);
}

// Maximum of x over the lane pair (l, l ^ 32), in every lane.
__device__ __forceinline__ float half_pair_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// The attention of one workgroup: QB query blocks (4 QB wavefronts).  QB = 2
// serves the dense path only: both query blocks take the same full key list,
// so each K and V sub-tile is copied into LDS once for 256 query rows instead
// of 128.  Every wavefront runs exactly the instructions it runs with QB = 1,
// in the same order, so the outputs do not depend on QB.
template <int D, bool full, int QB>
__device__ __forceinline__ void attend_bf16_body(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ vt,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ cnt, const float *__restrict__ w,
    const int32_t *__restrict__ order, uint16_t *__restrict__ out, int N, int N_pad, int NB, int cap,
    float scale_log2, bool xcd_ranges)
{
    using L = Lds<D>;
    constexpr int KS = D / 16;         // k-steps of S^T = K Q^T per 32-key tile
    constexpr int DT = D / 32;         // 32-row tiles of O^T
    constexpr int KT = kSub / 32;      // 32-key tiles per sub-tile
    constexpr int NK = KT * KS;        // K fragments (QK MFMAs) per sub-tile
    constexpr int NV = KT * 2 * DT;    // V^T fragments (PV MFMAs) per sub-tile
    constexpr int PF = 4;              // LDS fragment reads kept in flight ahead of their MFMA
    // every slot is a separate LDS object, so that the compiler can tell the
    // slot being read from the slots whose direct loads are still in flight
    __shared__ __align__(16) char ks0[L::kBytes], ks1[L::kBytes], ks2[L::kBytes];
    __shared__ __align__(16) char vs0[L::vBytes], vs1[L::vBytes];

    static_assert(QB == 1 || (QB == 2 && full), "two query blocks per workgroup only on the dense path");
    constexpr int W = kWaves * QB;     // wavefronts of the workgroup (they share the LDS staging)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qwave = wave % kWaves;   // the wavefront's 32 rows within its query block
    const int l32 = lane & 31, half = lane >> 5;
    // QB = 1: blk = (b*H + h) * NB + query block; sparse lists run longest first
    // within each range of the order (see mapped_slot).  QB = 2: slot = (b*H + h) *
    // ceil(NB / 2) + pair p, query blocks 2p and 2p + 1 of that head.  When NB is
    // odd the head's last pair has no second query block: its wavefronts still
    // copy their share of K and V and meet every barrier, but compute and store
    // nothing.
    const int slot = mapped_slot(xcd_ranges);
    const int blk = QB == 1 ? (full ? slot : order[slot]) : 0;
    const int np = (NB + 1) / 2;
    const long bh = QB == 1 ? blk / NB : slot / np;
    const int qb = QB == 1 ? blk % NB : 2 * (slot % np) + wave / kWaves;
    const bool active = QB == 1 || qb < NB;   // uniform over the wavefront
    const uint16_t *qh = q + bh * N_pad * D;
    const int4v rk = head_rsrc(k + bh * N_pad * D, N_pad * D * 2);
    const int4v rv = head_rsrc(vt + bh * N_pad * D, (v_rows<D>() ? N : N_pad) * D * 2);

    // this lane's query row (the MFMA column l32 of wavefront's tile); padding rows read as zero
    const int qrow = qb * kBlock + 32 * qwave + l32;
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
    float m_run = -INFINITY, l_run0 = 0.f, l_run1 = 0.f;
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

    // Per-lane LDS read offsets; tile offsets are immediates.
    // K fragment i = (kt, ks): row 32kt + l32, logical chunk 2ks + half (row % 16 == l32 % 16).
    int k_rd[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k_rd[ks] = l32 * L::pitch + 16 * ((2 * ks + half) ^ k_swz<D>(l32));
    // V operand i = (ksub = 2 kt + sub, dt).  Row-major V (D = 128): two transposing
    // reads from per-lane bases of each dt (the lane layout above), k-step rows as
    // immediates.  V^T tiles (D = 64): one 16-byte read at row 32dt + l32 (the
    // dimension), logical chunk 4kt + 2sub + half, i.e. positions 32kt + 16sub +
    // 8half .. +7; (row / 2) % 8 == (l32 / 2) % 8, so the tile row 32dt is an
    // immediate offset.
    int v_rd[v_rows<D>() ? DT : KT * 2];
    if (v_rows<D>()) {
        const int g = lane >> 4, m = lane & 15, row0 = 4 * (g >> 1) + (m >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int chunk = 4 * dt + 2 * (g & 1) + ((m & 3) >> 1);
            v_rd[dt] = row0 * L::pitch + 16 * (chunk ^ vr_swz(row0)) + 8 * (m & 1);
        }
    } else {
#pragma unroll
        for (int i = 0; i < KT * 2; ++i) v_rd[i] = l32 * L::vPitch + 16 * ((2 * i + half) ^ vt_swz(l32));
    }
    auto k_frag = [&](const char *st, int i) __attribute__((always_inline)) {
        return __builtin_bit_cast(bf16x8,
                                  *reinterpret_cast<const uint4 *>(st + k_rd[i % KS] + (i / KS) * 32 * L::pitch));
    };
    auto v_frag = [&](const char *st, int i) __attribute__((always_inline)) {
        if (v_rows<D>()) return v_frag_tr<D>(st + v_rd[i % DT] + 16 * (i / DT) * L::pitch);
        return __builtin_bit_cast(bf16x8,
                                  *reinterpret_cast<const uint4 *>(st + v_rd[i / DT] + (i % DT) * 32 * L::vPitch));
    };

    const Dma<D, W> dma = dma_offsets<D, W>(wave, lane);

    // One 64-key sub-tile held in K slot kst and V slot vst (compile-time
    // offsets, so every LDS read address is a per-lane base plus an
    // immediate); lw = log2 w_j.
    auto tile = [&](const char *kst, const char *vst, int key0, float lw) __attribute__((always_inline)) {
        // S^T = K Q^T: s[kt] holds keys [32kt, 32kt+32) of the sub-tile; lane
        // (l32, half) element r is key 32kt + 8(r/4) + 4half + r%4 of query l32.
        floatx16 s[KT];
        bf16x8 kf[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) kf[i] = k_frag(kst, i);
        // each read is issued PF MFMAs ahead of its use; the scheduling
        // fences keep the compiler from pulling reads back next to their use
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            const int kt = i / KS, ks = i % KS;
            s[kt] = mfma32(kf[i % PF], qf[ks], ks == 0 ? zero16 : s[kt]);
            if (i + PF < NK) kf[i % PF] = k_frag(kst, i + PF);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        // the PV operands are read while the softmax runs
        bf16x8 vf[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) vf[i] = v_frag(vst, i);

        if (key0 + kSub > N) {   // ragged end of the sequence: mask padding keys
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (key0 + kt * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= N) s[kt][r] = -INFINITY;
        }
        static_assert(KT == 2, "two 32-key tiles per sub-tile");
        // block weight enters as a logit shift
        const float m_tile = fmaf(half_pair_max(tile_max(s[0], s[1])), scale_log2, lw);
        // lazy rescale: the running max moves only when the tile's max
        // exceeds it by more than the slack (always on the first tile)
        if (__ballot(m_tile > m_run + kRescaleSlack) != 0) {
            asm volatile("s_nop 0");   // keeps this a branch rather than selects
            const float m_new = max2(m_run, m_tile);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run0 *= alpha;
            l_run1 *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        }
        // P^T in bf16 straight from the accumulators; the row sum adds the same
        // bf16-rounded probabilities the PV product uses (numerator and
        // normaliser agree), a pair per dot2 in two chains
        const float bias = lw - m_run;
        bf16x8 pb[KT][2];
        auto prob = [&](int kt, int r) __attribute__((always_inline)) {
            const float pr = __builtin_amdgcn_exp2f(fmaf(s[kt][r], scale_log2, bias));
            pb[kt][r >> 3][r & 7] = (__bf16)pr;
            if (r & 1) row_sum_pair(pb[kt][r >> 3], r & 7, (r & 2) ? l_run1 : l_run0);
        };
#pragma unroll
        for (int r = 0; r < 16; ++r) prob(0, r);
        // O^T += V^T P^T: MFMA (kt, sub, dt) contracts the 16 keys held in
        // accumulator rows [8sub, 8sub+8) of S^T tile kt against V^T rows
        // [32dt, 32dt+32); for lane half h, element e is key 32kt + 16sub +
        // 8(e/4) + 4h + e%4, stored at positions 32kt + 16sub + 8h + e.
        // Tile 1's probabilities are computed between tile 0's MFMAs.
        constexpr int per = 16 / (NV / 2);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            const int ksub = i / DT, dt = i % DT;
            o[dt] = mfma32(vf[i % PF], pb[ksub >> 1][ksub & 1], o[dt]);
            if (i + PF < NV) vf[i % PF] = v_frag(vst, i + PF);
            if (i < NV / 2) {
#pragma unroll
                for (int e = 0; e < per; ++e) prob(1, per * i + e);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
    };

    // Sub-tile u is half u % 2 of list entry u / 2; its K sits in K slot u % 3,
    // its V (rows, or the V^T tile at head_dim 64) in V slot u % 2.  Iteration u
    // issues V(u + 1) and then K(u + 2), computes u, and waits for all but the
    // K(u + 2) loads: K(u + 1) and V(u + 1) are then in LDS.  The entry loop is unrolled three times, so
    // every slot is a compile-time offset.  Branches are uniform over the
    // workgroup; invalid entries and sub-tiles past N load and compute nothing.
    constexpr int KL = Dma<D, W>::loads;
    auto kptr = [&](int sl) __attribute__((always_inline)) { return sl == 0 ? ks0 : (sl == 1 ? ks1 : ks2); };
    auto vptr = [&](int sl) __attribute__((always_inline)) { return sl == 0 ? vs0 : vs1; };
    const Entry none{-1, 0.f};
    Window win = load_window<full>(lrow, wrow, 0, n_list, NB, lane);
    Entry ce = n_list > 0 ? window_entry<full>(win, 0) : none;
    Entry ne = n_list > 1 ? window_entry<full>(win, 1) : none;
    auto hi_valid = [&](const Entry &en) __attribute__((always_inline)) { return en.j >= 0 && en.j * kBlock + kSub < N; };
    if (ce.j >= 0) {
        issue_k<D, W>(rk, ce.j * kBlock, kptr(0), wave, dma);
        issue_v<D, W>(rv, ce.j * kBlock, vptr(0), wave, dma);
    }
    if (hi_valid(ce)) issue_k<D, W>(rk, ce.j * kBlock + kSub, kptr(1), wave, dma);
    // settle the Q loads here, once, rather than before every tile of the loop
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
    if (hi_valid(ce)) wait_loads_and_sync<KL>(); else wait_loads_and_sync<0>();
    auto step = [&](auto e3c, int e) __attribute__((always_inline)) {
        constexpr int E3 = decltype(e3c)::value;             // e % 3
        constexpr int k0 = (2 * E3) % 3, k1 = (2 * E3 + 1) % 3;   // K slots of this entry's halves
        const int e2 = e + 2;
        if (!full && e2 < n_list && (e2 & 63) == 0) win = load_window<full>(lrow, wrow, e2 >> 6, n_list, NB, lane);
        const Entry nn = e2 < n_list ? window_entry<full>(win, e2) : none;
        const bool ce_hi = hi_valid(ce), ne_ok = ne.j >= 0, ne_hi = hi_valid(ne);
        // first half: V of the second half, K of the next entry's first half
        if (ce_hi) issue_v<D, W>(rv, ce.j * kBlock + kSub, vptr(1), wave, dma);
        if (ne_ok) issue_k<D, W>(rk, ne.j * kBlock, kptr((2 * E3 + 2) % 3), wave, dma);
        if (ce.j >= 0 && active) tile(kptr(k0), vptr(0), ce.j * kBlock, ce.lw);
        if (ne_ok) wait_loads_and_sync<KL>(); else wait_loads_and_sync<0>();
        // second half: V of the next entry's first half, K of its second half
        if (ne_ok) issue_v<D, W>(rv, ne.j * kBlock, vptr(0), wave, dma);
        if (ne_hi) issue_k<D, W>(rk, ne.j * kBlock + kSub, kptr((2 * E3 + 3) % 3), wave, dma);
        if (ce_hi && active) tile(kptr(k1), vptr(1), ce.j * kBlock + kSub, ce.lw);
        if (ne_hi) wait_loads_and_sync<KL>(); else wait_loads_and_sync<0>();
        ce = ne;
        ne = nn;
    };
    for (int e = 0; e < n_list; e += 3) {
        step(std::integral_constant<int, 0>{}, e);
        if (e + 1 >= n_list) break;
        step(std::integral_constant<int, 1>{}, e + 1);
        if (e + 2 >= n_list) break;
        step(std::integral_constant<int, 2>{}, e + 2);
    }

    // normalise and store: lane holds dims dt*32 + 8(r/4) + 4half + r%4 of its query
    const float l_lane = l_run0 + l_run1;
    const auto lr = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_lane), __float_as_uint(l_lane), false, false);
    const float lsum = __uint_as_float(lr[0]) + __uint_as_float(lr[1]);
    const float inv = (lsum > 0.f && qvalid) ? 1.f / lsum : 0.f;
    if (!active) return;
    uint16_t *orow = out + (bh * N_pad + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = dt * 32 + 8 * g + 4 * half;
            __bf16 b0 = (__bf16)(o[dt][4 * g + 0] * inv), b1 = (__bf16)(o[dt][4 * g + 1] * inv);
            __bf16 b2 = (__bf16)(o[dt][4 * g + 2] * inv), b3 = (__bf16)(o[dt][4 * g + 3] * inv);
            const uint32_t lo =
                (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
            const uint32_t hi =
                (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
            *reinterpret_cast<uint2 *>(orow + d) = make_uint2(lo, hi);
        }
}


// One query block per workgroup: sparse lists, and dense at head_dim 64.
template <int D, bool full>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attend_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ vt,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ cnt, const float *__restrict__ w,
    const int32_t *__restrict__ order, uint16_t *__restrict__ out, int N, int N_pad, int NB, int cap,
    float scale_log2, bool xcd_ranges)
{
    attend_bf16_body<D, full, 1>(q, k, vt, idx, cnt, w, order, out, N, N_pad, NB, cap, scale_log2, xcd_ranges);
}

// Dense, two query blocks of one head per workgroup: they share the K and V
// staging (the last pair of a head with an odd number of query blocks has one).
template <int D>
__global__ __launch_bounds__(2 * kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attend_dense_pair_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ vt,
    uint16_t *__restrict__ out, int N, int N_pad, int NB, float scale_log2, bool xcd_ranges)
{
    attend_bf16_body<D, true, 2>(q, k, vt, nullptr, nullptr, nullptr, nullptr, out, N, N_pad, NB, NB, scale_log2,
                                 xcd_ranges);
}

// ---------------------------------------------------------------------------
// 4-token key blocks (kernel paragraph: the unit of selection is smaller than
// the compute tile).  A list entry is a key block of 4 tokens; 16 of them fill
// a 64-key sub-tile, gathered by index with direct loads into the same LDS
// ring as above, so the MFMA work per sub-tile is unchanged.  At D = 128 one
// 4-token block of K or V (4 rows) is exactly 1024 bytes, one direct load
// of a wavefront: load t of wavefront w fills block slot 4w + t, its source
// address a scalar (block index x 1024) taken from the list window with
// v_readlane.
//
// V is gathered the same way (a block's 4 rows are also 1 KB) into the
// row-major, swizzled V layout of the 128-token kernel, and read with the same
// transposing reads: the PV operand of lane half h (keys 8(e/4) + 4h + e%4 of
// its S^T accumulators) is the 4 keys of block slot 4 ksub + h at dimension d
// followed by the 4 keys of slot 4 ksub + h + 2.  The partial last block reads
// its rows past N as zeros (range-checked offset, as above).
//
// Weights: an S^T element in row 8(r/4) + 4h + r%4 of 32-key tile kt belongs
// to block slot 8kt + 2(r/4) + h, so each lane needs 8 log2 weights per
// sub-tile, read from the window with v_readlane and selected by lane half.
// The lazy rescale tests an upper bound of the sub-tile's shifted maximum
// (max raw logit x scale + max log2 weight of the sub-tile): still no exp2
// argument exceeds the slack, and the running max can only overshoot by the
// spread of log2 weights (at most 32), harmless in fp32.
// Entries that are invalid or past the list load block 0 and get weight 0
// (log2 w = -inf); a sub-tile with no valid entry is not computed.  Keys past
// N can only sit in the last key block when N % 4 != 0; sub-tiles holding it
// mask those keys explicitly.
// ---------------------------------------------------------------------------
constexpr int kFineSub = kSub / kFineBlock;   // 4-token key blocks per sub-tile


// 64 list entries held lane-distributed: lane i has entry 64m + i as the block
// to load (0 for invalid entries and entries past the list) and its log2
// weight (-inf for those).  Ballots mark the entries that contribute and the
// entries whose block is the partial last block.
struct FineWindow {
    int j;
    float lw;
    uint64_t valid, partial;
};

// Raw list entries of window m, loaded without a branch on their values (index
// clamped into the list; entries past it are dropped by make_fine_window), so
// that both loads are in flight together and nothing waits for them until
// make_fine_window runs.
struct RawWindow {
    int j;
    float w;
};

__device__ __forceinline__ RawWindow load_raw_window(const int32_t *lrow, const float *wrow, int m, int n_list, int lane)
{
    const int e = min(64 * m + lane, n_list - 1);   // n_list >= 1 wherever a window is loaded
    return RawWindow{lrow[e], wrow[e]};
}

__device__ __forceinline__ FineWindow make_fine_window(const RawWindow &raw, int m, int n_list, int NBk, bool ragged,
                                                       int lane)
{
    const int e = 64 * m + lane;
    int j = 0;
    float lw = -INFINITY;
    if (e < n_list && raw.j >= 0 && raw.j < NBk && raw.w > 0.f && raw.w < INFINITY) {
        j = raw.j;
        lw = __log2f(raw.w);
    }
    FineWindow win;
    win.j = j;
    win.lw = lw;
    win.valid = __ballot(lw > -INFINITY);
    win.partial = __ballot(ragged && j == NBk - 1);
    return win;
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attend_fine_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ cnt, const float *__restrict__ w,
    const int32_t *__restrict__ order, uint16_t *__restrict__ out, int N, int N_pad, int NBq, int NBk, int cap,
    float scale_log2, bool xcd_ranges)
{
    static_assert(D == 128, "a 4-token key block of K or V is one 1024-byte direct load at D = 128");
    using L = Lds<D>;
    constexpr int KS = D / 16, DT = D / 32, KT = kSub / 32, NK = KT * KS, NV = KT * 2 * DT, PF = 4;
    constexpr int GB = kFineBlock * D * 2;   // bytes of one 4-token block of K or V
    constexpr int KL = kFineSub / kWaves;    // direct loads per wavefront and tensor per sub-tile
    __shared__ __align__(16) char ks0[L::kBytes], ks1[L::kBytes], ks2[L::kBytes];
    __shared__ __align__(16) char vs0[L::vBytes], vs1[L::vBytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, half = lane >> 5;
    const int slot = mapped_slot(xcd_ranges);
    const int blk = order[slot];
    const int qb = blk % NBq;
    const long bh = blk / NBq;
    const uint16_t *qh = q + bh * N_pad * D;
    const int4v rk = head_rsrc(k + bh * N_pad * D, N_pad * D * 2);
    const int4v rv = head_rsrc(v + bh * N_pad * D, N * D * 2);   // rows >= N read as 0

    const int qrow = qb * kBlock + 32 * wave + l32;
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
    float m_run = -INFINITY, l_run0 = 0.f, l_run1 = 0.f;
    const floatx16 zero16 = {};

    int n_list = cnt[blk];
    n_list = n_list < 0 ? 0 : (n_list > cap ? cap : n_list);
    const int32_t *lrow = idx + (long)blk * cap;
    const float *wrow = w + (long)blk * cap;
    const int n_sub = (n_list + kFineSub - 1) / kFineSub;
    const bool ragged = (N % kFineBlock) != 0;

    int k_rd[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k_rd[ks] = l32 * L::pitch + 16 * ((2 * ks + half) ^ k_swz<D>(l32));
    auto k_frag = [&](const char *st, int i) __attribute__((always_inline)) {
        return __builtin_bit_cast(bf16x8,
                                  *reinterpret_cast<const uint4 *>(st + k_rd[i % KS] + (i / KS) * 32 * L::pitch));
    };
    // V fragment i = (ksub, dt): the keys of block slots 4 ksub + half and
    // 4 ksub + half + 2 at dimension 32 dt + l32, by transposing reads of the
    // row-major V tile (the same addressing as the 128-token kernel)
    int v_rd[DT];
    {
        const int g = lane >> 4, m = lane & 15, row0 = 4 * (g >> 1) + (m >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int chunk = 4 * dt + 2 * (g & 1) + ((m & 3) >> 1);
            v_rd[dt] = row0 * L::pitch + 16 * (chunk ^ vr_swz(row0)) + 8 * (m & 1);
        }
    }
    auto v_frag = [&](const char *st, int i) __attribute__((always_inline)) {
        return v_frag_tr<D>(st + v_rd[i % DT] + 16 * (i / DT) * L::pitch);
    };

    // direct-load source offsets inside a 4-token block of K: lane L fills row
    // L / 16 of the block, LDS chunk L % 16, which holds logical chunk
    // (L % 16) ^ (LDS row % 16), and LDS row % 16 = 4t + L / 16 for load t
    int koff[KL];
#pragma unroll
    for (int t = 0; t < KL; ++t) koff[t] = (lane >> 4) * L::pitch + 16 * ((lane & 15) ^ (4 * t + (lane >> 4)));

    FineWindow win0{0, -INFINITY, 0, 0}, win1{0, -INFINITY, 0, 0};
    if (n_list > 0) win0 = make_fine_window(load_raw_window(lrow, wrow, 0, n_list, lane), 0, n_list, NBk, ragged, lane);
    RawWindow raw{0, 0.f};   // window m + 1, loaded at iteration 4m and turned into a window at 4m + 2
    // block to load for entry 16u + 4 wave + t (sub-tile u, this wavefront's load t)
    auto block_of = [&](int u, int t) __attribute__((always_inline)) {
        const int src = ((u >> 2) & 1) ? win1.j : win0.j;
        return __builtin_amdgcn_readlane(src, 16 * (u & 3) + 4 * wave + t);
    };
    auto issue_k = [&](char *dst, int u) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < KL; ++t) load_lds16(rk, koff[t], block_of(u, t) * GB, dst + (KL * wave + t) * 1024);
    };
    // V rows of a block: LDS row % 4 = L / 16, chunk L % 16 holds logical chunk
    // (L % 16) ^ vr_swz(row); the block's offset goes in the range-checked
    // per-lane offset, so rows >= N (the partial last block) read as 0
    const int voff = (lane >> 4) * L::pitch + 16 * ((lane & 15) ^ vr_swz(lane >> 4));
    auto issue_v = [&](char *dst, int u) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < KL; ++t) load_lds16(rv, voff + block_of(u, t) * GB, 0, dst + (KL * wave + t) * 1024);
    };

    auto tile = [&](const char *kst, const char *vst, int u) __attribute__((always_inline)) {
        const bool odd = (u >> 2) & 1;
        const int base = 16 * (u & 3);
        const float lw_src = odd ? win1.lw : win0.lw;
        // log2 weights of this lane's 8 block slots 8kt + 2i + half
        float lwe[KT][4];
        float lwm = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = base + 8 * kt + 2 * i;
                const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lw_src), e));
                const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lw_src), e + 1));
                lwe[kt][i] = half ? b : a;
                lwm = max2(lwm, lwe[kt][i]);
            }
        lwm = half_pair_max(lwm);

        floatx16 s[KT];
        bf16x8 kf[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) kf[i] = k_frag(kst, i);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            const int kt = i / KS, ks = i % KS;
            s[kt] = mfma32(kf[i % PF], qf[ks], ks == 0 ? zero16 : s[kt]);
            if (i + PF < NK) kf[i % PF] = k_frag(kst, i + PF);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        bf16x8 vf[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) vf[i] = v_frag(vst, i);

        const uint64_t pmask = odd ? win1.partial : win0.partial;
        if ((pmask >> base) & 0xFFFFull) {   // keys past N: the partial last block is in this sub-tile
            const int j_src = odd ? win1.j : win0.j;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int e = base + 8 * kt + 2 * i;
                    const int ja = __builtin_amdgcn_readlane(j_src, e), jb = __builtin_amdgcn_readlane(j_src, e + 1);
                    const int key0 = (half ? jb : ja) * kFineBlock;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (key0 + c >= N) s[kt][4 * i + c] = -INFINITY;
                }
        }
        const float m_tile = fmaf(half_pair_max(tile_max(s[0], s[1])), scale_log2, lwm);
        if (__ballot(m_tile > m_run + kRescaleSlack) != 0) {
            asm volatile("s_nop 0");
            const float m_new = max2(m_run, m_tile);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run0 *= alpha;
            l_run1 *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        }
        float bias[KT][4];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) bias[kt][i] = lwe[kt][i] - m_run;
        bf16x8 pb[KT][2];
        auto prob = [&](int kt, int r) __attribute__((always_inline)) {
            const float pr = __builtin_amdgcn_exp2f(fmaf(s[kt][r], scale_log2, bias[kt][r >> 2]));
            pb[kt][r >> 3][r & 7] = (__bf16)pr;
            if (r & 1) row_sum_pair(pb[kt][r >> 3], r & 7, (r & 2) ? l_run1 : l_run0);
        };
#pragma unroll
        for (int r = 0; r < 16; ++r) prob(0, r);
        constexpr int per = 16 / (NV / 2);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            const int ksub = i / DT, dt = i % DT;
            o[dt] = mfma32(vf[i % PF], pb[ksub >> 1][ksub & 1], o[dt]);
            if (i + PF < NV) vf[i % PF] = v_frag(vst, i + PF);
            if (i < NV / 2) {
#pragma unroll
                for (int e = 0; e < per; ++e) prob(1, per * i + e);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
    };

    // Sub-tile u: K in K slot u % 3, V in V slot u % 2.  Iteration u issues
    // V(u + 1) and K(u + 2), computes u and waits for all but the K(u + 2)
    // loads.  Window m (sub-tiles 4m .. 4m+3) sits in win{m % 2}; the entries of
    // window m + 1 are loaded at iteration 4m and validated at 4m + 2, just
    // before their first use, so the wait the compiler puts before that use
    // finds them long arrived.  Unrolled six times, so that every slot is a
    // compile-time offset.
    auto kptr = [&](int sl) __attribute__((always_inline)) { return sl == 0 ? ks0 : (sl == 1 ? ks1 : ks2); };
    auto vptr = [&](int sl) __attribute__((always_inline)) { return sl == 0 ? vs0 : vs1; };
    auto sub_valid = [&](int u) __attribute__((always_inline)) {
        const uint64_t vm = ((u >> 2) & 1) ? win1.valid : win0.valid;
        return ((vm >> (16 * (u & 3))) & 0xFFFFull) != 0;
    };
    if (n_sub > 0) {
        issue_k(kptr(0), 0);
        issue_v(vptr(0), 0);
    }
    if (n_sub > 1) issue_k(kptr(1), 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
    if (n_sub > 1) wait_loads_and_sync<KL>(); else wait_loads_and_sync<0>();
    auto step = [&](auto u6c, int u) __attribute__((always_inline)) {
        constexpr int U6 = decltype(u6c)::value;   // u % 6
        const int u1 = u + 1, u2 = u + 2;
        if ((u & 3) == 0 && u + 4 < n_sub) raw = load_raw_window(lrow, wrow, (u >> 2) + 1, n_list, lane);
        if ((u & 3) == 2 && u + 2 < n_sub) {   // window (u >> 2) + 1 is first used below, for K(u + 2)
            const FineWindow nw = make_fine_window(raw, (u >> 2) + 1, n_list, NBk, ragged, lane);
            if ((u >> 2) & 1) win0 = nw; else win1 = nw;
        }
        if (u1 < n_sub) issue_v(vptr((U6 + 1) % 2), u1);
        if (u2 < n_sub) issue_k(kptr((U6 + 2) % 3), u2);
        if (sub_valid(u)) tile(kptr(U6 % 3), vptr(U6 % 2), u);
        if (u2 < n_sub) wait_loads_and_sync<KL>(); else wait_loads_and_sync<0>();
    };
    for (int u = 0; u < n_sub; u += 6) {
        step(std::integral_constant<int, 0>{}, u);
        if (u + 1 >= n_sub) break;
        step(std::integral_constant<int, 1>{}, u + 1);
        if (u + 2 >= n_sub) break;
        step(std::integral_constant<int, 2>{}, u + 2);
        if (u + 3 >= n_sub) break;
        step(std::integral_constant<int, 3>{}, u + 3);
        if (u + 4 >= n_sub) break;
        step(std::integral_constant<int, 4>{}, u + 4);
        if (u + 5 >= n_sub) break;
        step(std::integral_constant<int, 5>{}, u + 5);
    }

    const float l_lane = l_run0 + l_run1;
    const auto lr = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_lane), __float_as_uint(l_lane), false, false);
    const float lsum = __uint_as_float(lr[0]) + __uint_as_float(lr[1]);
    const float inv = (lsum > 0.f && qvalid) ? 1.f / lsum : 0.f;
    uint16_t *orow = out + (bh * N_pad + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = dt * 32 + 8 * g + 4 * half;
            __bf16 b0 = (__bf16)(o[dt][4 * g + 0] * inv), b1 = (__bf16)(o[dt][4 * g + 1] * inv);
            __bf16 b2 = (__bf16)(o[dt][4 * g + 2] * inv), b3 = (__bf16)(o[dt][4 * g + 3] * inv);
            const uint32_t lo =
                (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
            const uint32_t hi =
                (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
            *reinterpret_cast<uint2 *>(orow + d) = make_uint2(lo, hi);
        }
}

// fp32 inputs with 4-token key blocks: the fp32 kernel below, with 16 list
// entries gathered into each 64-row key/value tile.
template <int D>
__global__ __launch_bounds__(256) void attend_f32_fine_kernel(const float *__restrict__ q, const float *__restrict__ k,
                                                              const float *__restrict__ v, const int32_t *__restrict__ idx,
                                                              const int32_t *__restrict__ cnt,
                                                              const float *__restrict__ w, float *__restrict__ out,
                                                              int N, int N_pad, int NBq, int NBk, int cap,
                                                              float scale_log2)
{
    constexpr int kTile = 64, HD = D / 2, kChunk = 16;
    __shared__ float4 k_s[kTile][D / 4];
    __shared__ float4 v_s[kTile][D / 4];
    __shared__ float lw_s[kTile];

    const int tid = threadIdx.x;
    const int blk = xcd_contiguous_id(blockIdx.x, gridDim.x);
    const int qb = blk % NBq;
    const long bh = blk / NBq;
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
    int n_list = cnt[blk];
    n_list = n_list < 0 ? 0 : (n_list > cap ? cap : n_list);
    for (int e0 = 0; e0 < n_list; e0 += kTile / kFineBlock) {
        __syncthreads();
        for (int i = tid; i < kTile * D / 4; i += 256) {
            const int rr = i / (D / 4), c = i % (D / 4);
            const int e = e0 + rr / kFineBlock;
            int j = -1;
            float wj = 0.f;
            if (e < n_list) {
                j = idx[(long)blk * cap + e];
                wj = w[(long)blk * cap + e];
                if (j < 0 || j >= NBk || !(wj > 0.f) || !(wj < INFINITY)) j = -1;
            }
            const int key = j * kFineBlock + rr % kFineBlock;
            const bool ok = j >= 0 && key < N;
            k_s[rr][c] = ok ? reinterpret_cast<const float4 *>(kh + (long)key * D)[c] : make_float4(0, 0, 0, 0);
            v_s[rr][c] = ok ? reinterpret_cast<const float4 *>(vh + (long)key * D)[c] : make_float4(0, 0, 0, 0);
            if (c == 0) lw_s[rr] = ok ? __log2f(wj) : -INFINITY;
        }
        __syncthreads();
        for (int c0 = 0; c0 < kTile; c0 += kChunk) {
            float lg[kChunk];
            float cmax = -INFINITY;
#pragma unroll
            for (int tt = 0; tt < kChunk; ++tt) {
                const float *kr = reinterpret_cast<const float *>(&k_s[c0 + tt][0]) + hd * HD;
                float dot = 0.f;
#pragma unroll
                for (int d = 0; d < HD; ++d) dot = fmaf(qv[d], kr[d], dot);
                dot += __shfl_xor(dot, 1, 64);
                const float lw = lw_s[c0 + tt];
                lg[tt] = lw > -INFINITY ? fmaf(dot, scale_log2, lw) : -INFINITY;
                cmax = fmaxf(cmax, lg[tt]);
            }
            if (cmax == -INFINITY) continue;   // nothing in this chunk (the same for every row)
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
    const float inv = (l_run > 0.f && qvalid) ? 1.f / l_run : 0.f;
    float *orow = out + (bh * N_pad + qrow) * D + hd * HD;
#pragma unroll
    for (int d = 0; d < HD; ++d) orow[d] = ov[d] * inv;
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

// XCD-contiguous ranges of the order while the layer's K and V fit in the
// 256 MB MALL as a whole, round-robin slots otherwise.  Measured with the same
// lists: 12 heads of 32K tokens (201 MB of K and V) run 9% faster with the
// ranges; 40 such heads (672 MB) 12% faster round-robin, and 24 heads of 119K
// tokens (1.5 GB) ~10% faster round-robin: once the layer does not fit, eight
// XCDs on eight different heads lose the MALL, all XCDs on the same heads keep it.
static bool attend_xcd_ranges(int B, int H, int N_pad, int D)
{
    constexpr double kMallBytes = 256.0 * 1024 * 1024;
    const double kv_bytes = 2.0 * B * H * N_pad * D * sizeof(uint16_t);
    return kv_bytes <= kMallBytes;
}

// Workspace of the bf16 attention calls: the V^T copy (head_dim 64 only; at 128
// the kernels read v itself), then the work order (sparse lists only).
size_t vt_bytes(int B, int H, int N_pad, int D)
{
    if (v_rows<128>() && D == 128) return 0;
    return ((size_t)B * H * N_pad * D * sizeof(uint16_t) + 255) & ~(size_t)255;
}

template <bool full>
hipError_t launch_attend_t(const void *q, const void *k, const void *v, int dtype, int B, int H, int N, int N_pad,
                           int D, int NB, float scale, const int32_t *idx, const int32_t *cnt, const float *w, int cap,
                           void *ws, void *out, hipStream_t s)
{
    const int G = B * H * NB;
    const dim3 grid((unsigned)G), block(256);
    const float sl2 = scale * kLog2e;
    if (dtype == kBF16 && (D == 128 || D == 64)) {
        uint16_t *vt = static_cast<uint16_t *>(ws);
        int32_t *order = nullptr;
        if (!full) {
            order = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + vt_bytes(B, H, N_pad, D));
            order_kernel<<<dim3(8), dim3(kOrderThreads), 0, s>>>(cnt, G, cap, 1, order);
        }
        if (D == 128 && full) {
            // dense: two query blocks of one head per workgroup share the K and V staging
            attend_dense_pair_kernel<128><<<dim3((unsigned)((long)B * H * ((NB + 1) / 2))), dim3(2 * kThreads), 0, s>>>(
                (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (uint16_t *)out, N, N_pad, NB, sl2,
                attend_xcd_ranges(B, H, N_pad, D));
        } else if (D == 128) {
            attend_bf16_kernel<128, full><<<grid, dim3(kThreads), 0, s>>>(
                (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, idx, cnt, w, order, (uint16_t *)out, N,
                N_pad, NB, cap, sl2, attend_xcd_ranges(B, H, N_pad, D));
        } else {
            vt_kernel<64><<<dim3((unsigned)((long)B * H * (N_pad / kSub))), block, 0, s>>>((const uint16_t *)v, N, N_pad,
                                                                                        vt);
            attend_bf16_kernel<64, full><<<grid, dim3(kThreads), 0, s>>>(
                (const uint16_t *)q, (const uint16_t *)k, vt, idx, cnt, w, order, (uint16_t *)out, N, N_pad, NB, cap, sl2,
                attend_xcd_ranges(B, H, N_pad, D));
        }
    } else if (dtype == kF32 && D == 64) {
        attend_f32_kernel<64, full><<<grid, block, 0, s>>>((const float *)q, (const float *)k, (const float *)v, idx,
                                                          cnt, w, (float *)out, N, N_pad, NB, cap, sl2);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Sparse attention over lists of 4-token key blocks.
hipError_t launch_attend_fine(const void *q, const void *k, const void *v, int dtype, int B, int H, int N, int N_pad,
                              int D, int NBq, int NBk, float scale, const int32_t *idx, const int32_t *cnt,
                              const float *w, int cap, void *ws, void *out, hipStream_t s)
{
    const int G = B * H * NBq;
    const float sl2 = scale * kLog2e;
    if (dtype == kBF16 && D == 128) {
        int32_t *order = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + vt_bytes(B, H, N_pad, D));
        order_kernel<<<dim3(8), dim3(kOrderThreads), 0, s>>>(cnt, G, cap, kFineSub, order);
        attend_fine_kernel<128><<<dim3((unsigned)G), dim3(kThreads), 0, s>>>(
            (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, idx, cnt, w, order, (uint16_t *)out, N,
            N_pad, NBq, NBk, cap, sl2, attend_xcd_ranges(B, H, N_pad, D));
    } else if (dtype == kF32 && D == 64) {
        attend_f32_fine_kernel<64><<<dim3((unsigned)G), dim3(256), 0, s>>>((const float *)q, (const float *)k,
                                                                          (const float *)v, idx, cnt, w, (float *)out,
                                                                          N, N_pad, NBq, NBk, cap, sl2);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_attend(const void *q, const void *k, const void *v, int dtype, int B, int H, int N, int N_pad, int D,
                         int NB, float scale, const int32_t *idx, const int32_t *cnt, const float *w, int cap, bool full,
                         void *ws, void *out, hipStream_t s)
{
    return full ? launch_attend_t<true>(q, k, v, dtype, B, H, N, N_pad, D, NB, scale, idx, cnt, w, cap, ws, out, s)
                : launch_attend_t<false>(q, k, v, dtype, B, H, N, N_pad, D, NB, scale, idx, cnt, w, cap, ws, out, s);
}

size_t attend_workspace_bytes(int dtype, int B, int H, int N_pad, int D)
{
    if (dtype != kBF16) return 0;
    return vt_bytes(B, H, N_pad, D) + (size_t)B * H * (N_pad / kBlock) * sizeof(int32_t);
}

}  // namespace aba
