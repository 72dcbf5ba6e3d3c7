// C ABI of libdllm: host-side argument checks, then the launches.  The
// contract of every entry point is documented in include/dllm.h.
#include "common.hpp"

#include <climits>
#include <cmath>
#include <mutex>

using namespace dllm;

// Scratch of dllm_scatter_attention_noalloc: the key-split partials of its
// attention kernels.  The loader gives every GPU the library runs on its own
// copy, held until the process ends.  In host code `scratch` is a host-side
// stand-in for the symbol, not a device address: the device address comes
// from hipGetSymbolAddress, once per device (scratch_on_current_device).
static __device__ __align__(256) unsigned char scratch[DLLM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

// the device address of the current device's scratch array, looked up on the
// first call on that device (with that device current)
int scratch_on_current_device(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return DLLM_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return DLLM_ERANGE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DLLM_EHIP;
        g_scratch_dev[dev] = p;
    }
    *ptr = g_scratch_dev[dev];
    return DLLM_OK;
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

inline int dtype_size(int dt) {
    switch (dt) {
    case DLLM_F32: return 4;
    case DLLM_BF16: return 2;
    case DLLM_E4M3: return 1;
    default: return 0;
    }
}

int check_cache(const dllm_kv_cache *c) {
    if (!c || !c->k || !c->v) return DLLM_EINVAL;
    if (c->B < 1 || c->L < 1 || c->n_kv_heads < 1) return DLLM_ESHAPE;
    if (c->d_head < 16 || c->d_head > 256) return DLLM_ESHAPE;
    const int esz = dtype_size(c->dtype);
    if (!esz) return DLLM_EDTYPE;
    if ((c->d_head * esz) % 16 != 0) return DLLM_EALIGN;
    // the rows of one (sequence, KV head) are addressed with 32-bit offsets
    if ((uint64_t)c->L * c->d_head * esz > 0xFFFFFFFFull) return DLLM_ERANGE;
    if (!aligned16(c->k) || !aligned16(c->v)) return DLLM_EALIGN;
    if (c->dtype == DLLM_E4M3) {
        if (c->d_head % 128 != 0) return DLLM_ESHAPE;
        if (!c->k_scale || !c->v_scale) return DLLM_EINVAL;
    }
    return DLLM_OK;
}

}  // namespace

extern "C" {

const char *dllm_status_str(int status) {
    switch (status) {
    case DLLM_OK: return "ok";
    case DLLM_EINVAL: return "invalid argument";
    case DLLM_EDTYPE: return "unsupported dtype";
    case DLLM_ESHAPE: return "unsupported or inconsistent shape";
    case DLLM_EALIGN: return "pointer or row not 16-byte aligned";
    case DLLM_ERANGE: return "size beyond the supported maximum";
    case DLLM_EHIP: return "HIP runtime or launch failure";
    case DLLM_EWORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
    }
}

int dllm_version(void) { return 100; }

int dllm_cache_init(dllm_kv_cache *cache, int B, int L, int n_kv_heads, int d_head, int dtype,
                    void *k, void *v, float *k_scale, float *v_scale, void *stream) {
    if (!cache) return DLLM_EINVAL;
    dllm_kv_cache c{};
    c.B = B;
    c.L = L;
    c.n_kv_heads = n_kv_heads;
    c.d_head = d_head;
    c.dtype = dtype;
    c.k = k;
    c.v = v;
    c.k_scale = dtype == DLLM_E4M3 ? k_scale : nullptr;
    c.v_scale = dtype == DLLM_E4M3 ? v_scale : nullptr;
    int rc = check_cache(&c);
    if (rc != DLLM_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t rows = (size_t)B * n_kv_heads * L;
    const size_t bytes = rows * d_head * dtype_size(dtype);
    if ((rc = launch_fill_zero(k, bytes, s)) != DLLM_OK) return rc;
    if ((rc = launch_fill_zero(v, bytes, s)) != DLLM_OK) return rc;
    if (dtype == DLLM_E4M3) {
        const size_t sbytes = rows * (d_head / 128) * sizeof(float);
        if ((rc = launch_fill_zero(k_scale, sbytes, s)) != DLLM_OK) return rc;
        if ((rc = launch_fill_zero(v_scale, sbytes, s)) != DLLM_OK) return rc;
    }
    *cache = c;
    return DLLM_OK;
}

int dllm_scatter_kv(const dllm_kv_cache *cache, const void *k_new, const void *v_new,
                    int src_dtype, const int32_t *pos, int n, int32_t *bad_count, void *stream) {
    int rc = check_cache(cache);
    if (rc != DLLM_OK) return rc;
    if (n < 0) return DLLM_EINVAL;
    if (n == 0) return DLLM_OK;
    if (!k_new || !v_new || !pos) return DLLM_EINVAL;
    if (cache->dtype == DLLM_E4M3) {
        if (src_dtype != DLLM_F32 && src_dtype != DLLM_BF16) return DLLM_EDTYPE;
    } else if (src_dtype != cache->dtype) {
        return DLLM_EDTYPE;
    }
    if (!aligned16(k_new) || !aligned16(v_new)) return DLLM_EALIGN;
    return launch_scatter(*cache, k_new, v_new, src_dtype, pos, n, bad_count,
                          static_cast<hipStream_t>(stream));
}

int dllm_sink_rolling_map(int B, int L, int S, int R, const int32_t *end, int32_t *key_idx,
                          int n_keys, void *stream) {
    if (B < 1 || L < 1 || S < 0 || R < 0) return DLLM_EINVAL;
    if (!end || !key_idx) return DLLM_EINVAL;
    if ((int64_t)n_keys < (int64_t)S + R || n_keys < 1) return DLLM_ESHAPE;
    if (B > 65535) return DLLM_ERANGE;
    return launch_sink_rolling(B, L, S, R, end, key_idx, n_keys, static_cast<hipStream_t>(stream));
}

size_t dllm_block_attention_workspace(const dllm_kv_cache *cache, int q_dtype, int Hq, int b,
                                      int n_keys) {
    if (check_cache(cache) != DLLM_OK || Hq < 1 || b < 1 || n_keys < 1) return 0;
    if (Hq % cache->n_kv_heads != 0) return 0;
    // enough for the call with or without a key map
    AttnPlan with_map, without;
    if (plan_attention(*cache, q_dtype, Hq, b, n_keys, true, &with_map) != DLLM_OK) return 0;
    if (plan_attention(*cache, q_dtype, Hq, b, n_keys, false, &without) != DLLM_OK) return 0;
    return with_map.ws_bytes > without.ws_bytes ? with_map.ws_bytes : without.ws_bytes;
}

int dllm_block_attention(const dllm_kv_cache *cache, const void *q, int q_dtype, int Hq, int b,
                         const int32_t *key_idx, int n_keys, float scale, void *out,
                         int out_dtype, float *lse, void *workspace, size_t ws_bytes,
                         void *stream) {
    int rc = check_cache(cache);
    if (rc != DLLM_OK) return rc;
    if (!q || !out) return DLLM_EINVAL;
    if (Hq < 1 || b < 1) return DLLM_ESHAPE;
    if (Hq % cache->n_kv_heads != 0) return DLLM_ESHAPE;
    if (!key_idx) n_keys = cache->L;
    if (n_keys < 1) return DLLM_ESHAPE;
    if (q_dtype != DLLM_F32 && q_dtype != DLLM_BF16) return DLLM_EDTYPE;
    if (out_dtype != DLLM_F32 && out_dtype != DLLM_BF16) return DLLM_EDTYPE;
    if (!(scale >= 0.f) || std::isinf(scale)) return DLLM_EINVAL;
    if (scale == 0.f) scale = 1.0f / std::sqrt((float)cache->d_head);
    if ((int64_t)cache->B * Hq * b > INT32_MAX / 4) return DLLM_ERANGE;
    AttnPlan p;
    if ((rc = plan_attention(*cache, q_dtype, Hq, b, n_keys, key_idx != nullptr, &p)) != DLLM_OK)
        return rc;
    if (p.path != 0 && (!aligned16(q) || !aligned16(out))) return DLLM_EALIGN;
    if (p.ws_bytes > 0 && (!workspace || ws_bytes < p.ws_bytes || !aligned16(workspace)))
        return DLLM_EWORKSPACE;
    return launch_attention(*cache, p, q, q_dtype, Hq, b, key_idx, n_keys, scale, AttnMemo{}, out,
                            out_dtype, lse, workspace, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {
// the checks of dllm_scatter_kv, then those of dllm_block_attention (without
// the workspace's), and the plan; scale and n_keys come back resolved
int check_scatter_attention(const dllm_kv_cache *cache, const void *k_new, const void *v_new,
                            int src_dtype, const int32_t *pos, int n, const void *q, int q_dtype,
                            int Hq, int b, const int32_t *key_idx, int &n_keys, float &scale,
                            void *out, int out_dtype, AttnPlan *p) {
    int rc = check_cache(cache);
    if (rc != DLLM_OK) return rc;
    if (n < 0) return DLLM_EINVAL;
    if (n > 0) {
        if (!k_new || !v_new || !pos) return DLLM_EINVAL;
        if (cache->dtype == DLLM_E4M3) {
            if (src_dtype != DLLM_F32 && src_dtype != DLLM_BF16) return DLLM_EDTYPE;
        } else if (src_dtype != cache->dtype) {
            return DLLM_EDTYPE;
        }
        if (!aligned16(k_new) || !aligned16(v_new)) return DLLM_EALIGN;
    }
    if (!q || !out) return DLLM_EINVAL;
    if (Hq < 1 || b < 1) return DLLM_ESHAPE;
    if (Hq % cache->n_kv_heads != 0) return DLLM_ESHAPE;
    if (!key_idx) n_keys = cache->L;
    if (n_keys < 1) return DLLM_ESHAPE;
    if (q_dtype != DLLM_F32 && q_dtype != DLLM_BF16) return DLLM_EDTYPE;
    if (out_dtype != DLLM_F32 && out_dtype != DLLM_BF16) return DLLM_EDTYPE;
    if (!(scale >= 0.f) || std::isinf(scale)) return DLLM_EINVAL;
    if (scale == 0.f) scale = 1.0f / std::sqrt((float)cache->d_head);
    if ((int64_t)cache->B * Hq * b > INT32_MAX / 4) return DLLM_ERANGE;
    if ((rc = plan_attention(*cache, q_dtype, Hq, b, n_keys, key_idx != nullptr, p)) != DLLM_OK)
        return rc;
    if (p->path != 0 && (!aligned16(q) || !aligned16(out))) return DLLM_EALIGN;
    return DLLM_OK;
}
}  // namespace

extern "C" {

int dllm_scatter_attention(const dllm_kv_cache *cache, const void *k_new, const void *v_new,
                           int src_dtype, const int32_t *pos, int n, int32_t *bad_count,
                           const void *q, int q_dtype, int Hq, int b, const int32_t *key_idx,
                           int n_keys, float scale, void *out, int out_dtype, float *lse,
                           void *workspace, size_t ws_bytes, void *stream) {
    AttnPlan p;
    int rc = check_scatter_attention(cache, k_new, v_new, src_dtype, pos, n, q, q_dtype, Hq, b, key_idx,
                                     n_keys, scale, out, out_dtype, &p);
    if (rc != DLLM_OK) return rc;
    if (p.ws_bytes > 0 && (!workspace || ws_bytes < p.ws_bytes || !aligned16(workspace)))
        return DLLM_EWORKSPACE;
    return launch_scatter_attention(*cache, p, k_new, v_new, src_dtype, pos, n, bad_count, q, q_dtype,
                                    Hq, b, key_idx, n_keys, scale, out, out_dtype, lse, workspace,
                                    static_cast<hipStream_t>(stream));
}

int dllm_scatter_attention_noalloc(const dllm_kv_cache *cache, const void *k_new, const void *v_new,
                                   int src_dtype, const int32_t *pos, int n, int32_t *bad_count,
                                   const void *q, int q_dtype, int Hq, int b, const int32_t *key_idx,
                                   int n_keys, float scale, void *out, int out_dtype, float *lse,
                                   void *stream) {
    AttnPlan p;
    int rc = check_scatter_attention(cache, k_new, v_new, src_dtype, pos, n, q, q_dtype, Hq, b, key_idx,
                                     n_keys, scale, out, out_dtype, &p);
    if (rc != DLLM_OK) return rc;
    if (p.ws_bytes > DLLM_NOALLOC_SCRATCH_BYTES) return DLLM_ERANGE;
    void *ws = nullptr;
    if (p.ws_bytes > 0 && (rc = scratch_on_current_device(&ws)) != DLLM_OK) return rc;
    return launch_scatter_attention(*cache, p, k_new, v_new, src_dtype, pos, n, bad_count, q, q_dtype,
                                    Hq, b, key_idx, n_keys, scale, out, out_dtype, lse, ws,
                                    static_cast<hipStream_t>(stream));
}

int dllm_facache_maps(int B, int L, int blk, const int32_t *start, int32_t *unchanged_idx,
                      int32_t *block_idx, void *stream) {
    if (B < 1 || blk < 1 || L <= blk) return DLLM_ESHAPE;
    if (B > 65535) return DLLM_ERANGE;
    if (!start || !unchanged_idx || !block_idx) return DLLM_EINVAL;
    return launch_facache_maps(B, L, blk, start, unchanged_idx, block_idx,
                               static_cast<hipStream_t>(stream));
}

size_t dllm_facache_merge_workspace(const dllm_kv_cache *cache, int q_dtype, int Hq, int n_q,
                                    int n_keys) {
    if (check_cache(cache) != DLLM_OK || Hq < 1 || n_q < 1 || n_keys < 1) return 0;
    if (Hq % cache->n_kv_heads != 0) return 0;
    AttnPlan with_map, without;
    if (plan_facache(*cache, q_dtype, Hq, n_q, n_keys, true, &with_map) != DLLM_OK) return 0;
    if (plan_facache(*cache, q_dtype, Hq, n_q, n_keys, false, &without) != DLLM_OK) return 0;
    return with_map.ws_bytes > without.ws_bytes ? with_map.ws_bytes : without.ws_bytes;
}

int dllm_facache_merge(const dllm_kv_cache *cache, const void *q, int q_dtype, int Hq, int n_q,
                       const int32_t *key_idx, int n_keys, float scale, const float *memo_o,
                       const float *memo_lse, void *out, int out_dtype, float *lse,
                       void *workspace, size_t ws_bytes, void *stream) {
    int rc = check_cache(cache);
    if (rc != DLLM_OK) return rc;
    if (!q || !out || !memo_o || !memo_lse) return DLLM_EINVAL;
    if (Hq < 1 || n_q < 1) return DLLM_ESHAPE;
    if (Hq % cache->n_kv_heads != 0) return DLLM_ESHAPE;
    if (!key_idx) n_keys = cache->L;
    if (n_keys < 1) return DLLM_ESHAPE;
    if (q_dtype != DLLM_F32 && q_dtype != DLLM_BF16) return DLLM_EDTYPE;
    if (out_dtype != DLLM_F32 && out_dtype != DLLM_BF16) return DLLM_EDTYPE;
    if (!(scale >= 0.f) || std::isinf(scale)) return DLLM_EINVAL;
    if (scale == 0.f) scale = 1.0f / std::sqrt((float)cache->d_head);
    if ((int64_t)cache->B * Hq * n_q > INT32_MAX / 4) return DLLM_ERANGE;
    AttnPlan p;
    if ((rc = plan_facache(*cache, q_dtype, Hq, n_q, n_keys, key_idx != nullptr, &p)) != DLLM_OK)
        return rc;
    if (p.path == 2 && (!aligned16(q) || !aligned16(out) || !aligned16(memo_o)))
        return DLLM_EALIGN;
    if (p.ws_bytes > 0 && (!workspace || ws_bytes < p.ws_bytes || !aligned16(workspace)))
        return DLLM_EWORKSPACE;
    AttnMemo memo;
    memo.o = memo_o;
    memo.lse = memo_lse;
    return launch_attention(*cache, p, q, q_dtype, Hq, n_q, key_idx, n_keys, scale, memo, out,
                            out_dtype, lse, workspace, static_cast<hipStream_t>(stream));
}

int dllm_fp8_quant_rows(const void *x, int dtype, int64_t M, int K, int64_t ld, uint8_t *codes,
                        uint8_t *scales, void *stream) {
    if (dtype != DLLM_F32 && dtype != DLLM_BF16) return DLLM_EDTYPE;
    if (M < 0 || K < 128 || K % 128 != 0 || ld < K) return DLLM_ESHAPE;
    if (M > INT32_MAX) return DLLM_ERANGE;
    if (M == 0) return DLLM_OK;
    if (!x || !codes || !scales) return DLLM_EINVAL;
    if (!aligned16(x) || !aligned16(codes) || (ld * dtype_size(dtype)) % 16 != 0) return DLLM_EALIGN;
    return launch_fp8_quant_rows(x, dtype, ld, M, K, codes, scales, static_cast<hipStream_t>(stream));
}

int dllm_fp8_addnorm_quant(const void *x, const void *residual, const void *gamma, int dtype,
                           float eps, int64_t M, int K, void *residual_out, uint8_t *codes,
                           uint8_t *scales, void *stream) {
    if (dtype != DLLM_F32 && dtype != DLLM_BF16) return DLLM_EDTYPE;
    if (M < 0 || K < 128 || K % 128 != 0 || K > 16384) return DLLM_ESHAPE;
    if (M > INT32_MAX) return DLLM_ERANGE;
    if (!(eps >= 0.f) || std::isinf(eps)) return DLLM_EINVAL;
    if (M == 0) return DLLM_OK;
    if (!x || !gamma || !codes || !scales) return DLLM_EINVAL;
    if (!aligned16(x) || !aligned16(gamma) || !aligned16(codes) || (residual && !aligned16(residual)) ||
        (residual_out && !aligned16(residual_out)))
        return DLLM_EALIGN;
    return launch_fp8_addnorm_quant(x, residual, gamma, dtype, eps, M, K, residual_out, codes, scales,
                                    static_cast<hipStream_t>(stream));
}

int dllm_fp8_quant_weight(const void *w, int dtype, int N, int K, uint8_t *codes, uint8_t *scales,
                          void *stream) {
    if (dtype != DLLM_F32 && dtype != DLLM_BF16) return DLLM_EDTYPE;
    if (N < 128 || K < 128 || N % 128 != 0 || K % 128 != 0) return DLLM_ESHAPE;
    if (!w || !codes || !scales) return DLLM_EINVAL;
    if (!aligned16(w) || !aligned16(codes)) return DLLM_EALIGN;
    return launch_fp8_quant_weight(w, dtype, N, K, codes, scales, static_cast<hipStream_t>(stream));
}

namespace {
int check_fp8_gemm(const uint8_t *a, const uint8_t *a_scale, const uint8_t *b, const uint8_t *b_scale,
                   int M, int N, int K) {
    if (M < 0 || N < 256 || K < 128 || N % 256 != 0 || K % 128 != 0) return DLLM_ESHAPE;
    if (K > 12288) return DLLM_ERANGE;                // the tile's scales are held in LDS
    if (!a || !a_scale || !b || !b_scale) return DLLM_EINVAL;
    if (!aligned16(a) || !aligned16(b)) return DLLM_EALIGN;
    return DLLM_OK;
}
}  // namespace

int dllm_fp8_gemm(const uint8_t *a, const uint8_t *a_scale, const uint8_t *b, const uint8_t *b_scale,
                  int M, int N, int K, void *c, void *stream) {
    int rc = check_fp8_gemm(a, a_scale, b, b_scale, M, N, K);
    if (rc != DLLM_OK) return rc;
    if (M == 0) return DLLM_OK;
    if (!c) return DLLM_EINVAL;
    return launch_fp8_gemm(a, a_scale, b, b_scale, M, N, K, 0, static_cast<uint16_t *>(c), nullptr,
                           nullptr, static_cast<hipStream_t>(stream));
}

int dllm_fp8_gemm_swiglu(const uint8_t *a, const uint8_t *a_scale, const uint8_t *b,
                         const uint8_t *b_scale, int M, int N, int K, uint8_t *out_codes,
                         uint8_t *out_scales, void *stream) {
    int rc = check_fp8_gemm(a, a_scale, b, b_scale, M, N, K);
    if (rc != DLLM_OK) return rc;
    if (M == 0) return DLLM_OK;
    if (!out_codes || !out_scales) return DLLM_EINVAL;
    return launch_fp8_gemm(a, a_scale, b, b_scale, M, N, K, 1, nullptr, out_codes, out_scales,
                           static_cast<hipStream_t>(stream));
}

size_t dllm_vocab_stats_workspace(int64_t N, int64_t V) {
    if (N < 0 || V < 1) return 0;
    return plan_vocab(N, V).ws_bytes;
}

size_t dllm_workspace_size(int which, const dllm_workspace_args *a) {
    if (a == nullptr) return 0;
    switch (which) {
    case DLLM_WS_BLOCK_ATTENTION:
        return dllm_block_attention_workspace(a->cache, a->q_dtype, a->Hq, a->n_q, a->n_keys);
    case DLLM_WS_FACACHE_MERGE:
        return dllm_facache_merge_workspace(a->cache, a->q_dtype, a->Hq, a->n_q, a->n_keys);
    case DLLM_WS_VOCAB_STATS:
        return dllm_vocab_stats_workspace(a->N, a->V);
    default:
        return 0;
    }
}

int dllm_vocab_stats(const void *logits, int dtype, int64_t N, int64_t V, int64_t row_stride,
                     int32_t *argmax, float *maxprob, float *entropy, void *workspace,
                     size_t ws_bytes, void *stream) {
    if (N < 0 || V < 1 || row_stride < V) return DLLM_ESHAPE;
    if (V > INT32_MAX) return DLLM_ERANGE;
    if (dtype != DLLM_F32 && dtype != DLLM_BF16) return DLLM_EDTYPE;
    if (N == 0) return DLLM_OK;
    if (!logits || !argmax || !maxprob || !entropy) return DLLM_EINVAL;
    if (((uintptr_t)logits & (uintptr_t)(dtype_size(dtype) - 1)) != 0) return DLLM_EALIGN;
    const VocabPlan p = plan_vocab(N, V);
    if (p.ws_bytes > 0 && (!workspace || ws_bytes < p.ws_bytes || !aligned16(workspace)))
        return DLLM_EWORKSPACE;
    return launch_vocab(logits, dtype, N, V, row_stride, argmax, maxprob, entropy, p, workspace,
                        static_cast<hipStream_t>(stream));
}

int dllm_stability_reset(int B, int L, int D, int32_t *ring_argmax, float *ring_maxprob,
                         int32_t *ring_step, float *entropy_latest, int32_t *t_write,
                         uint8_t *stable, void *stream) {
    if (B < 1 || L < 1 || D < 1) return DLLM_ESHAPE;
    if (!ring_argmax || !ring_maxprob || !ring_step || !entropy_latest || !t_write || !stable)
        return DLLM_EINVAL;
    return launch_stability_reset(B, L, D, ring_argmax, ring_maxprob, ring_step, entropy_latest,
                                  t_write, stable, static_cast<hipStream_t>(stream));
}

int dllm_stability_mask(int B, int L, int step, int32_t *step_dev, const int32_t *pos, int n,
                        const int32_t *argmax, const float *maxprob, const float *entropy,
                        int32_t *ring_argmax, float *ring_maxprob, int32_t *ring_step,
                        float *entropy_latest, int32_t *t_write, uint8_t *stable,
                        const dllm_stab_params *params, uint8_t *mask, float *conf,
                        int32_t *next_pos, int32_t *count, uint8_t *all_stable, void *stream) {
    if (!params) return DLLM_EINVAL;
    if (B < 1 || L < 1 || step < 0) return DLLM_ESHAPE;
    if (B > 65535) return DLLM_ERANGE;
    if (!pos && n != L && n != 0) return DLLM_ESHAPE;   // NULL list: all L, or none
    if (n < 0 || n > L) return DLLM_ESHAPE;
    const dllm_stab_params &p = *params;
    if (p.K < 1 || p.D < p.K || p.R < 0 || p.vocab < 2) return DLLM_EINVAL;
    if (p.advance_step && !step_dev) return DLLM_EINVAL;   // nothing to advance
    if (p.R_early < 0 || p.T_steps < 0 || p.refresh_every < 0) return DLLM_EINVAL;
    if (!(p.tau == p.tau) || !(p.alpha == p.alpha) || !(p.beta == p.beta) ||
        !(p.conf_thresh == p.conf_thresh))
        return DLLM_EINVAL;
    // the age factor is read from the caller's table whenever beta is not 0
    if (p.beta != 0.0 && (!p.decay || p.n_decay < 1)) return DLLM_EINVAL;
    if (p.beta != 0.0 && ((uintptr_t)p.decay & 7u) != 0) return DLLM_EALIGN;
    if ((n > 0 && (!argmax || !maxprob || !entropy)) || !ring_argmax || !ring_maxprob ||
        !ring_step || !entropy_latest || !t_write || !stable || !mask || !next_pos || !count ||
        !all_stable)
        return DLLM_EINVAL;
    // maximum entropy of a vocab-V distribution, computed once on the host
    const double hmax = std::log((double)p.vocab);
    return launch_stability(B, L, step, step_dev, pos, n, argmax, maxprob, entropy, ring_argmax,
                            ring_maxprob, ring_step, entropy_latest, t_write, stable, p, hmax,
                            mask, conf, next_pos, count, all_stable,
                            static_cast<hipStream_t>(stream));
}

int dllm_confidence_decay(double lambda, int n, double *table) {
    if (!table || n < 1 || !(lambda >= 0.0) || std::isinf(lambda)) return DLLM_EINVAL;
    // the C library's exp of the float64 product, one value per age
    for (int k = 0; k < n; ++k) table[k] = std::exp(-lambda * (double)k);
    return DLLM_OK;
}

int dllm_check_positions(int B, int L, const int32_t *pos, int n, int32_t *bad, int32_t *dup,
                         void *stream) {
    if (B < 1 || L < 1 || n < 0) return DLLM_ESHAPE;
    if (B > 65535 || L > 131072) return DLLM_ERANGE;
    if ((n > 0 && !pos) || !bad || !dup) return DLLM_EINVAL;
    return launch_check_positions(B, L, pos, n, bad, dup, static_cast<hipStream_t>(stream));
}

int dllm_refresh_interval(int T) {
    const int f = (int)std::floor((double)T / 10.0 + 0.5);
    return f < 3 ? 3 : (f > 10 ? 10 : f);
}

int dllm_cache_quotas(int B, const int32_t *len, int64_t budget, double min_frac, int32_t *quota) {
    if (B < 1 || !len || !quota || budget < 0 || !(min_frac >= 0.0)) return DLLM_EINVAL;
    int64_t need = 0;
    for (int b = 0; b < B; ++b) {
        if (len[b] < 0) return DLLM_EINVAL;
        const double m = std::ceil(min_frac * (double)len[b]);
        quota[b] = (int32_t)(m > (double)len[b] ? (double)len[b] : m);
        need += quota[b];
    }
    if (need > budget) return DLLM_ERANGE;
    int64_t left = budget - need;
    for (int b = 0; b < B; ++b) {
        const int64_t extra = std::min<int64_t>((int64_t)len[b] - quota[b], left);
        quota[b] += (int32_t)extra;
        left -= extra;
    }
    return DLLM_OK;
}

int dllm_evict_by_confidence(int B, int L, const float *conf, const int32_t *quota,
                             const int32_t *pos, int n, uint8_t *cached, uint8_t *mask,
                             int32_t *next_pos, int32_t *count, int32_t *evicted, void *stream) {
    if (B < 1 || L < 1) return DLLM_ESHAPE;
    if (B > 65535 || L > 131072) return DLLM_ERANGE;
    if (!pos && n != L && n != 0) return DLLM_ESHAPE;
    if (n < 0 || n > L) return DLLM_ESHAPE;
    if (!conf || !quota || !cached || !mask || !next_pos || !count) return DLLM_EINVAL;
    return launch_evict(B, L, conf, quota, pos, n, cached, mask, next_pos, count, evicted,
                        static_cast<hipStream_t>(stream));
}

int dllm_parallel_width(int w_early, int w_late, int T, int step) {
    if (T <= 1) return w_late;
    const int st = step < T - 1 ? (step < 0 ? 0 : step) : T - 1;
    return w_early - (w_early - w_late) * st / (T - 1);
}

int dllm_self_verify(int B, int L, const int32_t *dec_pos, int n, const float *p_marg,
                     const float *p_joint, int W, double tau, uint8_t *rollback, uint8_t *mask,
                     uint8_t *stable, uint8_t *cached, int32_t *next_pos, int32_t *count,
                     int32_t *n_rollback, int32_t *rb_pos, void *stream) {
    if (B < 1 || L < 1 || n < 0 || n > L) return DLLM_ESHAPE;
    if (B > 65535 || L > 131072) return DLLM_ERANGE;
    if (W < 2 || W > 8 || !(tau >= 0.0)) return DLLM_EINVAL;
    if (n > 0 && (!dec_pos || !p_marg || !p_joint)) return DLLM_EINVAL;
    if (!rollback || !mask || !next_pos || !count) return DLLM_EINVAL;
    return launch_self_verify(B, L, dec_pos, n, p_marg, p_joint, W, tau, rollback, mask, stable, cached,
                              next_pos, count, n_rollback, rb_pos, static_cast<hipStream_t>(stream));
}

}  // extern "C"
