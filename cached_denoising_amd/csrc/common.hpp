// Internal helpers shared by the HIP kernels of libdllm (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "dllm.h"

namespace dllm {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// bfloat16 bits <-> float (exact widening; the low half of the float is zero)
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bfloat16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// float32 -> OCP e4m3fn code, round to nearest even, saturate to +-448.
// Works on the float's bits: the e4m3 value is the float's significand
// shifted right so that 3 fraction bits remain (more for results below the
// e4m3 normal range), rounded half to even on the dropped bits.
__device__ __forceinline__ uint32_t e4m3_rne(float q) {
    const uint32_t u = __float_as_uint(q);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return 0x7fu;                  // NaN
    if (a > 0x43e00000u) return sign | 0x7eu;            // |q| > 448 (incl. inf)
    const int E = (int)(a >> 23) - 127;                  // unbiased exponent
    uint32_t r;
    if (E < -6) {
        // below 2^-6: count units of 2^-9 (the e4m3 subnormal spacing)
        const uint32_t mant = (a >> 23) ? ((a & 0x7fffffu) | 0x800000u) : (a & 0x7fffffu);
        const int sh = (a >> 23) ? (14 - E) : 140;       // q * 2^9 = mant >> sh
        if (sh >= 32) {
            r = 0;
        } else {
            r = mant >> sh;
            const uint32_t rem = mant & ((1u << sh) - 1u);
            const uint32_t half = 1u << (sh - 1);
            if (rem > half || (rem == half && (r & 1u))) ++r;   // r = 8 is 2^-6: code 0x08
        }
    } else {
        // exponent field E + 7 and the top 3 fraction bits, rounded on the other 20
        r = ((uint32_t)(E + 7) << 3) | ((a >> 20) & 7u);
        const uint32_t rem = a & 0xfffffu;
        if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
    }
    return sign | r;
}

// bits 0..3 of x as the low bits of four bytes (four 0/1 flags in one word)
__device__ __forceinline__ uint32_t spread4(uint32_t x) {
    return (x & 1u) | ((x & 2u) << 7) | ((x & 4u) << 14) | ((x & 8u) << 21);
}

// Four consecutive byte flags at p (p 4-aligned when `aligned`): one 32-bit
// store when all four lie below `limit` positions from p, else byte stores.
__device__ __forceinline__ void store_flags4(uint8_t *p, uint32_t bits4, int left, bool aligned) {
    if (left >= 4 && aligned) {
        *reinterpret_cast<uint32_t *>(p) = spread4(bits4);
    } else {
        for (int k = 0; k < 4 && k < left; ++k) p[k] = (uint8_t)((bits4 >> k) & 1u);
    }
}

// cross-lane helpers on a 64-wide wavefront
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, kWave); }
// the lanes of a wave below this one, as a ballot mask
__device__ __forceinline__ uint64_t lanes_below(int lane) { return lane ? (~0ull) >> (64 - lane) : 0ull; }

// Exclusive prefix over a workgroup of NW waves of one int per thread
// (thread order), and the total.  Uses `tmp` (NW ints, not to be reused by
// the caller without a barrier); contains one barrier.
template <int NW>
__device__ __forceinline__ int block_exclusive_scan(int v, int lane, int wave, int *tmp, int &total) {
    int incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) tmp[wave] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
    for (int w = 0; w < NW; ++w) {
        const int t = tmp[w];
        before += w < wave ? t : 0;
        total += t;
    }
    return before + incl - v;
}

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// status of the last launch on this thread
inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? DLLM_OK : DLLM_EHIP;
}

// ---- launchers (one translation unit each) ---------------------------------
int launch_fill_zero(void *p, size_t bytes, hipStream_t s);

int launch_scatter(const dllm_kv_cache &c, const void *k_new, const void *v_new, int src_dtype,
                   const int32_t *pos, int n, int32_t *bad_count, hipStream_t s);

int launch_sink_rolling(int B, int L, int S, int R, const int32_t *end, int32_t *key_idx,
                        int n_keys, hipStream_t s);
int launch_check_positions(int B, int L, const int32_t *pos, int n, int32_t *bad, int32_t *dup,
                           hipStream_t s);
int launch_facache_maps(int B, int L, int b, const int32_t *start, int32_t *unchanged_idx,
                        int32_t *block_idx, hipStream_t s);

struct AttnPlan {
    int path;          // 0: float32 VALU path, 1: MFMA, keys per wave, 2: MFMA, tiles shared by the waves
    int rows;          // query rows per (batch, kv-head): G * b
    int row_tiles;     // 16-row tiles per wave (MFMA path)
    int row_groups;    // workgroups along the rows of one (batch, kv-head)
    int splits;        // key splits across workgroups
    int waves;         // waves per workgroup (MFMA path)
    int tiles_per_wave;// 32-key tiles per wave (path 2: per workgroup, i.e. per split)
    size_t ws_bytes;   // partial-result workspace
};
// A memoized online-softmax state per query row, stored normalised (o = O~/l
// as [rows, d] float, lse = m + ln l as [rows] float, natural log; lse = -inf
// is an empty state).  When given, the attention kernels start each row's
// state from it instead of the empty state.
struct AttnMemo {
    const float *o = nullptr;
    const float *lse = nullptr;
};
// the block's fresh K/V rows, written by the attention kernel itself (see
// launch_scatter_attention); pos == nullptr: none
struct ScatterIn {
    const uint4 *k_new = nullptr, *v_new = nullptr;   // [B, n, Hkv, d] as 16-byte chunks
    const int32_t *pos = nullptr;                     // [B, n]
    int n = 0;
    int32_t *bad = nullptr;
};
int plan_attention(const dllm_kv_cache &c, int q_dtype, int Hq, int b, int n_keys, bool has_map,
                   AttnPlan *p);
// the plan of a call with a memo: the VALU path or the grouped-query layout
int plan_facache(const dllm_kv_cache &c, int q_dtype, int Hq, int n_q, int n_keys, bool has_map,
                 AttnPlan *p);
// the grouped-query layout (path 2), for more than one 32-row group per KV head
void plan_shared(const dllm_kv_cache &c, int Hq, int b, int row_groups32, int n_keys, bool has_map,
                 AttnPlan *p);
int launch_shared_attention(const dllm_kv_cache &c, const AttnPlan &p, const void *q, int Hq, int b,
                            const int32_t *key_idx, int n_keys, float scale, const AttnMemo &memo,
                            void *out, int out_dtype, float *lse, void *ws, hipStream_t s);
// merge of the (m, l, O~) partials of key splits, in split order
int launch_attn_merge(const float *part_o, const float *part_ml, int64_t rows_total, int D,
                      int splits, void *out, int out_dtype, float *lse, hipStream_t s);
// the scatter then the attention, in one launch when the per-wave layout
// takes the call (bf16 cache and rows, no key map)
int launch_scatter_attention(const dllm_kv_cache &c, const AttnPlan &p, const void *k_new,
                             const void *v_new, int src_dtype, const int32_t *pos, int n,
                             int32_t *bad, const void *q, int q_dtype, int Hq, int b,
                             const int32_t *key_idx, int n_keys, float scale, void *out,
                             int out_dtype, float *lse, void *ws, hipStream_t s);
int launch_attention(const dllm_kv_cache &c, const AttnPlan &p, const void *q, int q_dtype, int Hq,
                     int b, const int32_t *key_idx, int n_keys, float scale, const AttnMemo &memo,
                     void *out, int out_dtype, float *lse, void *ws, hipStream_t s);

int launch_self_verify(int B, int L, const int32_t *dec_pos, int n, const float *p_marg,
                       const float *p_joint, int W, double tau, uint8_t *rollback, uint8_t *mask,
                       uint8_t *stable, uint8_t *cached, int32_t *next_pos, int32_t *count,
                       int32_t *n_rollback, int32_t *rb_pos, hipStream_t s);
int launch_evict(int B, int L, const float *conf, const int32_t *quota, const int32_t *pos, int n,
                 uint8_t *cached, uint8_t *mask, int32_t *next_pos, int32_t *count, int32_t *evicted,
                 hipStream_t s);

// per-group FP8 for the FFN
int launch_fp8_quant_rows(const void *x, int dtype, int64_t ld, int64_t M, int K, uint8_t *codes,
                          uint8_t *scales, hipStream_t s);
int launch_fp8_addnorm_quant(const void *x, const void *res, const void *gamma, int dtype, float eps,
                             int64_t M, int K, void *res_out, uint8_t *codes, uint8_t *scales,
                             hipStream_t s);
int launch_fp8_quant_weight(const void *w, int dtype, int N, int K, uint8_t *codes, uint8_t *scales,
                            hipStream_t s);
int launch_fp8_gemm(const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb, int M,
                    int N, int K, int epilogue, uint16_t *c, uint8_t *qc, uint8_t *qs, hipStream_t s);

struct VocabPlan {
    int threads;       // workgroup size: 256, or 512 when there are few rows
    int splits;        // workgroups per row
    int64_t chunk;     // elements per split
    size_t ws_bytes;
};
VocabPlan plan_vocab(int64_t N, int64_t V);
int launch_vocab(const void *logits, int dtype, int64_t N, int64_t V, int64_t stride,
                 int32_t *argmax, float *maxprob, float *entropy, const VocabPlan &p, void *ws,
                 hipStream_t s);

int launch_stability_reset(int B, int L, int D, int32_t *ring_argmax, float *ring_maxprob,
                           int32_t *ring_step, float *entropy_latest, int32_t *t_write,
                           uint8_t *stable, hipStream_t s);
int launch_stability(int B, int L, int step, int32_t *step_dev, const int32_t *pos, int n,
                     const int32_t *argmax,
                     const float *maxprob, const float *entropy, int32_t *ring_argmax,
                     float *ring_maxprob, int32_t *ring_step, float *entropy_latest,
                     int32_t *t_write, uint8_t *stable, const dllm_stab_params &prm, double hmax,
                     uint8_t *mask, float *conf, int32_t *next_pos, int32_t *count,
                     uint8_t *all_stable, hipStream_t s);

}  // namespace dllm
