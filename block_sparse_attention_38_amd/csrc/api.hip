// api.hip -- the C ABI of libaba.so (declared in include/aba.h): argument
// validation, workspace layout and kernel launches.  Host code only; every
// computation runs in the kernels of kmeans.hip, pool_score.hip, fine_score.hip,
// sample.hip, attend.hip, diag.hip and calib.hip.
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/aba.h"
#include "aba_internal.h"

namespace {

thread_local std::string g_last_error;

aba_status fail(aba_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
aba_status fail(aba_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

aba_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return ABA_OK;
    return fail(ABA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// One workspace serves every call, each using it from offset 0 and only for
// the duration of the call: aba_score keeps centroids, weights and pooled keys
// there when the caller does not ask for them (and, for 4-token key blocks, the
// per-chunk softmax statistics of its two-pass scoring), aba_attend and
// aba_attend_full the work order (and at head_dim 64 a V^T staging copy of v),
// aba_sample the per-chunk totals, tops and counts of rows of more than 8192
// key blocks.
struct Workspace {
    size_t cent, weight, kbar, fine, score_total, attend_total, sample_total, total;
};

Workspace workspace_layout(const aba_plan_t &p)
{
    const size_t rows = (size_t)p.batch * p.heads * p.n_blocks;
    const size_t krows = (size_t)p.batch * p.heads * p.n_key_blocks;
    Workspace w;
    w.cent = 0;
    w.weight = align256(rows * p.n_clusters * p.head_dim * sizeof(float));
    w.kbar = w.weight + align256(rows * p.n_clusters * sizeof(float));
    w.fine = w.kbar + align256(krows * p.head_dim * sizeof(float));
    w.score_total = w.fine + align256(aba::fine_score_workspace_bytes(p.batch, p.heads, p.n_blocks, p.n_key_blocks));
    w.attend_total = align256(aba::attend_workspace_bytes(p.dtype, p.batch, p.heads, p.seq_pad, p.head_dim));
    w.sample_total = align256(aba::sample_workspace_bytes(p.batch, p.heads, p.n_blocks, p.n_key_blocks, p.budget));
    w.total = w.score_total > w.attend_total ? w.score_total : w.attend_total;
    w.total = w.total > w.sample_total ? w.total : w.sample_total;
    return w;
}

aba_status check_attend_workspace(const aba_plan_t *p, const void *workspace)
{
    if (!workspace && workspace_layout(*p).attend_total > 0)
        return fail(ABA_E_INVALID, "workspace of %llu bytes is required for bf16 attention",
                    (unsigned long long)p->workspace_bytes);
    return ABA_OK;
}

// A plan must be exactly what aba_plan produces for its own fields.
aba_status check_plan(const aba_plan_t *p)
{
    if (!p) return fail(ABA_E_INVALID, "plan is NULL");
    aba_plan_t ref;
    const aba_status st = aba_plan(&ref, p->batch, p->heads, p->seq_len, p->head_dim, (aba_dtype)p->dtype,
                                   p->n_clusters, p->kmeans_iters, p->budget, p->key_block, p->softmax_scale);
    if (st != ABA_OK) return st;
    if (ref.n_blocks != p->n_blocks || ref.seq_pad != p->seq_pad || ref.list_cap != p->list_cap ||
        ref.block != p->block || ref.n_key_blocks != p->n_key_blocks || ref.workspace_bytes != p->workspace_bytes)
        return fail(ABA_E_INVALID, "plan fields are inconsistent; fill the plan with aba_plan");
    return ABA_OK;
}

// Scratch of aba_attend_noalloc: the attention work order (one int32 per query
// block) of calls whose caller cannot allocate a workspace.  Each GPU the
// library runs on holds its own copy until the process ends; every call on a
// GPU reuses it, so calls that overlap in time on one GPU race.
constexpr size_t kStaticScratchBytes = size_t(1) << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch (the current device's), resolved once
// per device with that device current.  The array's name is only a host-side
// stand-in; kernels get this address.
aba_status static_scratch(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ABA_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(ABA_E_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(ABA_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return ABA_OK;
}

}  // namespace

extern "C" {

aba_status aba_plan(aba_plan_t *p, int32_t batch, int32_t heads, int32_t seq_len, int32_t head_dim, aba_dtype dtype,
                    int32_t n_clusters, int32_t kmeans_iters, int32_t budget, int32_t key_block, float softmax_scale)
{
    g_last_error.clear();
    if (!p) return fail(ABA_E_INVALID, "plan is NULL");
    if (batch < 1 || heads < 1 || seq_len < 1 || head_dim < 1)
        return fail(ABA_E_INVALID, "sizes must be positive (batch=%d heads=%d seq_len=%d head_dim=%d)", batch, heads,
                    seq_len, head_dim);
    if (n_clusters < 1) return fail(ABA_E_INVALID, "n_clusters must be >= 1 (got %d)", n_clusters);
    if (kmeans_iters < 0) return fail(ABA_E_INVALID, "kmeans_iters must be >= 0 (got %d)", kmeans_iters);
    if (budget < 1) return fail(ABA_E_INVALID, "budget must be >= 1 (got %d)", budget);
    if (!(std::isfinite(softmax_scale))) return fail(ABA_E_INVALID, "softmax_scale is not finite");
    if (dtype != ABA_F32 && dtype != ABA_BF16) return fail(ABA_E_INVALID, "unknown dtype %d", (int)dtype);
    if (key_block != ABA_BLOCK && key_block != ABA_FINE_BLOCK)
        return fail(ABA_E_INVALID, "key_block must be %d or %d (got %d)", ABA_BLOCK, ABA_FINE_BLOCK, key_block);
    if (dtype == ABA_BF16 && head_dim != 64 && head_dim != 128)
        return fail(ABA_E_UNSUPPORTED, "bf16 kernels exist for head_dim 64 and 128 (got %d)", head_dim);
    if (dtype == ABA_F32 && head_dim != 64)
        return fail(ABA_E_UNSUPPORTED, "fp32 kernels exist for head_dim 64 (got %d)", head_dim);
    if (n_clusters > ABA_MAX_CLUSTERS)
        return fail(ABA_E_UNSUPPORTED, "at most %d clusters (got %d)", ABA_MAX_CLUSTERS, n_clusters);
    if (kmeans_iters > 64) return fail(ABA_E_UNSUPPORTED, "at most 64 k-means rounds (got %d)", kmeans_iters);
    const int64_t nb = ((int64_t)seq_len + ABA_BLOCK - 1) / ABA_BLOCK;
    if (nb > ABA_MAX_BLOCKS)
        return fail(ABA_E_UNSUPPORTED, "at most %d blocks of %d tokens (got %lld)", ABA_MAX_BLOCKS, ABA_BLOCK,
                    (long long)nb);
    if ((int64_t)batch * heads * nb > 0x7FFFFFFF) return fail(ABA_E_UNSUPPORTED, "batch*heads*blocks exceeds 2^31");
    const int64_t nbk = ((int64_t)seq_len + key_block - 1) / key_block;
    if (key_block == ABA_FINE_BLOCK) {
        if (dtype == ABA_BF16 && head_dim != 128)
            return fail(ABA_E_UNSUPPORTED, "4-token key blocks with bf16 need head_dim 128 (got %d)", head_dim);
        if (nbk > ABA_MAX_KEY_BLOCKS)
            return fail(ABA_E_UNSUPPORTED, "at most %d key blocks of %d tokens (got %lld)", ABA_MAX_KEY_BLOCKS,
                        ABA_FINE_BLOCK, (long long)nbk);
        if ((int64_t)batch * heads * nb * nbk > ((int64_t)1 << 40))
            return fail(ABA_E_UNSUPPORTED, "score matrix of %lld entries is too large",
                        (long long)((int64_t)batch * heads * nb * nbk));
        const size_t lds = aba::sample_lds_bytes((int)nbk, budget);
        if (lds > (size_t)aba::kSampleLdsLimit)
            return fail(ABA_E_UNSUPPORTED, "budget %d over %lld key blocks needs %zu bytes of sampling LDS (limit %d)",
                        budget, (long long)nbk, lds, aba::kSampleLdsLimit);
    }

    std::memset(p, 0, sizeof *p);
    p->batch = batch;
    p->heads = heads;
    p->seq_len = seq_len;
    p->head_dim = head_dim;
    p->block = ABA_BLOCK;
    p->n_blocks = (int32_t)nb;
    p->seq_pad = (int32_t)nb * ABA_BLOCK;
    p->n_clusters = n_clusters;
    p->kmeans_iters = kmeans_iters;
    p->budget = budget;
    p->list_cap = (int32_t)nbk;
    p->dtype = dtype;
    p->softmax_scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
    p->key_block = key_block;
    p->n_key_blocks = (int32_t)nbk;
    p->workspace_bytes = workspace_layout(*p).total;
    return ABA_OK;
}

aba_status aba_score(const aba_plan_t *p, const void *q, const void *k, float *scores, float *centroids,
                     float *cluster_w, float *pooled_k, void *workspace, hipStream_t stream)
{
    g_last_error.clear();
    aba_status st = check_plan(p);
    if (st != ABA_OK) return st;
    if (!q || !k || !scores) return fail(ABA_E_INVALID, "q, k and scores must be non-NULL");
    const bool fine = p->key_block == ABA_FINE_BLOCK;
    if (!workspace)
        return fail(ABA_E_INVALID, "workspace of %llu bytes is required (the scoring passes keep their statistics there)",
                    (unsigned long long)p->workspace_bytes);
    const Workspace lay = workspace_layout(*p);
    char *ws = static_cast<char *>(workspace);
    float *cent = centroids ? centroids : reinterpret_cast<float *>(ws + lay.cent);
    float *wgt = cluster_w ? cluster_w : reinterpret_cast<float *>(ws + lay.weight);
    float *kbar = pooled_k ? pooled_k : reinterpret_cast<float *>(ws + lay.kbar);

    const int B = p->batch, H = p->heads, N = p->seq_len, NP = p->seq_pad, D = p->head_dim, NB = p->n_blocks;
    const int NBk = p->n_key_blocks;
    bool pooled = false;
    st = hip_status(aba::launch_kmeans(q, k, p->dtype, B, H, N, NP, D, NB, p->n_clusters, p->kmeans_iters,
                                       p->key_block, NBk, cent, wgt, kbar, &pooled, stream),
                    "kmeans launch");
    if (st != ABA_OK) return st;
    if (!pooled) {
        st = hip_status(fine ? aba::launch_fine_pool(k, p->dtype, B, H, N, NP, D, NBk, kbar, stream)
                             : aba::launch_pool(k, p->dtype, B, H, N, NP, D, NB, kbar, stream),
                        "pool launch");
        if (st != ABA_OK) return st;
    }
    return hip_status(aba::launch_fine_score(cent, wgt, kbar, B, H, NB, NBk, p->n_clusters, D, p->softmax_scale,
                                             ws + lay.fine, scores, stream),
                      "score launch");
}

aba_status aba_sample(const aba_plan_t *p, const float *scores, uint64_t seed, int32_t head_offset,
                      int32_t batch_offset, int32_t *idx, int32_t *cnt, float *w, void *workspace,
                      hipStream_t stream)
{
    g_last_error.clear();
    aba_status st = check_plan(p);
    if (st != ABA_OK) return st;
    if (!scores || !idx || !cnt || !w) return fail(ABA_E_INVALID, "scores, idx, cnt and w must be non-NULL");
    if (!workspace && workspace_layout(*p).sample_total > 0)
        return fail(ABA_E_INVALID, "workspace of %llu bytes is required to sample rows of %d key blocks",
                    (unsigned long long)p->workspace_bytes, p->n_key_blocks);
    if (head_offset < 0 || batch_offset < 0 || (int64_t)head_offset + p->heads > INT32_MAX ||
        (int64_t)batch_offset + p->batch > INT32_MAX)
        return fail(ABA_E_INVALID, "head_offset (%d) and batch_offset (%d) must be >= 0 and keep the global indices "
                    "below 2^31", head_offset, batch_offset);
    return hip_status(aba::launch_sample(scores, p->batch, p->heads, p->n_blocks, p->n_key_blocks, p->budget, seed,
                                         head_offset, batch_offset, p->list_cap, idx, cnt, w, workspace, stream),
                      "sample launch");
}

aba_status aba_attend(const aba_plan_t *p, const void *q, const void *k, const void *v, const int32_t *idx,
                      const int32_t *cnt, const float *w, void *out, void *workspace, hipStream_t stream)
{
    g_last_error.clear();
    aba_status st = check_plan(p);
    if (st != ABA_OK) return st;
    if (!q || !k || !v || !idx || !cnt || !w || !out)
        return fail(ABA_E_INVALID, "q, k, v, idx, cnt, w and out must be non-NULL");
    st = check_attend_workspace(p, workspace);
    if (st != ABA_OK) return st;
    if (p->key_block == ABA_FINE_BLOCK)
        return hip_status(aba::launch_attend_fine(q, k, v, p->dtype, p->batch, p->heads, p->seq_len, p->seq_pad,
                                                  p->head_dim, p->n_blocks, p->n_key_blocks, p->softmax_scale, idx, cnt,
                                                  w, p->list_cap, workspace, out, stream),
                          "attend launch");
    return hip_status(aba::launch_attend(q, k, v, p->dtype, p->batch, p->heads, p->seq_len, p->seq_pad, p->head_dim,
                                         p->n_blocks, p->softmax_scale, idx, cnt, w, p->list_cap, false, workspace, out,
                                         stream),
                      "attend launch");
}

aba_status aba_attend_full(const aba_plan_t *p, const void *q, const void *k, const void *v, void *out,
                           void *workspace, hipStream_t stream)
{
    g_last_error.clear();
    aba_status st = check_plan(p);
    if (st != ABA_OK) return st;
    if (!q || !k || !v || !out) return fail(ABA_E_INVALID, "q, k, v and out must be non-NULL");
    st = check_attend_workspace(p, workspace);
    if (st != ABA_OK) return st;
    return hip_status(aba::launch_attend(q, k, v, p->dtype, p->batch, p->heads, p->seq_len, p->seq_pad, p->head_dim,
                                         p->n_blocks, p->softmax_scale, nullptr, nullptr, nullptr, p->list_cap, true,
                                         workspace, out, stream),
                      "attend_full launch");
}

aba_status aba_attend_noalloc(const aba_plan_t *p, const void *q, const void *k, const void *v, const int32_t *idx,
                              const int32_t *cnt, const float *w, void *out, hipStream_t stream)
{
    g_last_error.clear();
    aba_status st = check_plan(p);
    if (st != ABA_OK) return st;
    if (!q || !k || !v || !idx || !cnt || !w || !out)
        return fail(ABA_E_INVALID, "q, k, v, idx, cnt, w and out must be non-NULL");
    if (p->dtype == ABA_BF16 && p->head_dim != 128)
        return fail(ABA_E_UNSUPPORTED, "aba_attend_noalloc: bf16 at head_dim %d stages a transposed copy of v; use "
                    "aba_attend with a workspace", p->head_dim);
    const size_t need = workspace_layout(*p).attend_total;
    if (need > kStaticScratchBytes)
        return fail(ABA_E_UNSUPPORTED, "aba_attend_noalloc: the work order of %lld query blocks needs %zu bytes, more "
                    "than the %zu of its static scratch (at most %zu query blocks); use aba_attend with a workspace",
                    (long long)p->batch * p->heads * p->n_blocks, need, kStaticScratchBytes,
                    kStaticScratchBytes / sizeof(int32_t));
    void *ws = nullptr;
    st = static_scratch(&ws);
    if (st != ABA_OK) return st;
    if (p->key_block == ABA_FINE_BLOCK)
        return hip_status(aba::launch_attend_fine(q, k, v, p->dtype, p->batch, p->heads, p->seq_len, p->seq_pad,
                                                  p->head_dim, p->n_blocks, p->n_key_blocks, p->softmax_scale, idx, cnt,
                                                  w, p->list_cap, ws, out, stream),
                          "attend launch");
    return hip_status(aba::launch_attend(q, k, v, p->dtype, p->batch, p->heads, p->seq_len, p->seq_pad, p->head_dim,
                                         p->n_blocks, p->softmax_scale, idx, cnt, w, p->list_cap, false, ws, out,
                                         stream),
                      "attend launch");
}

aba_status aba_block_mass(const aba_plan_t *p, const void *q, const void *k, const int32_t *items, int32_t n_items,
                          float *mass, hipStream_t stream)
{
    g_last_error.clear();
    aba_status st = check_plan(p);
    if (st != ABA_OK) return st;
    if (p->dtype != ABA_BF16) return fail(ABA_E_UNSUPPORTED, "aba_block_mass takes bf16 inputs");
    if (n_items < 0) return fail(ABA_E_INVALID, "n_items must be >= 0");
    if (n_items == 0) return ABA_OK;
    if (!q || !k || !items || !mass) return fail(ABA_E_INVALID, "q, k, items and mass must be non-NULL");
    return hip_status(aba::launch_block_mass(q, k, p->dtype, p->batch, p->heads, p->seq_len, p->seq_pad, p->head_dim,
                                             p->n_blocks, p->key_block, p->softmax_scale, items, n_items, mass, stream),
                      "block_mass launch");
}

aba_status aba_mfma_rate(int32_t iters, int32_t random, float *out, hipStream_t stream)
{
    if (iters < 1 || iters > 1000000) return fail(ABA_E_INVALID, "aba_mfma_rate: iters %d outside 1 .. 10^6", iters);
    if (!out) return fail(ABA_E_INVALID, "aba_mfma_rate: out is null");
    return hip_status(aba::launch_mfma_rate(iters, random, out, stream), "aba_mfma_rate launch");
}

const char *aba_last_error(void) { return g_last_error.c_str(); }

const char *aba_version(void) { return "aba 0.1.0 (gfx950)"; }

}  // extern "C"
