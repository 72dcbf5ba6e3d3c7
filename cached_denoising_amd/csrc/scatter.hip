// K/V scatter: the recomputed block's fresh rows go to their positions in
// the persistent cache; every other cached row is untouched, so the cache
// afterwards holds what a full recompute would have produced.  [LaCache
// explainer, Methodology 1 (RoPECache) and 3 (inference workflow); SWD
// page, 4.1 and 4.3 (write results back at the masked positions); sinks
// page, 5.1 (index writes instead of concatenation).]
//
// Also the small fill and key-map kernels of the cache set-up.
#include "common.hpp"

namespace dllm {
namespace {

// ---- plain copy: one 16-byte chunk per thread ------------------------------
__global__ __launch_bounds__(256) void scatter_copy_kernel(
    const uint4 *__restrict__ k_new, const uint4 *__restrict__ v_new, uint4 *__restrict__ ck,
    uint4 *__restrict__ cv, const int32_t *__restrict__ pos, int n, int Hkv, int L,
    int chunks_per_row, int64_t total, int32_t *__restrict__ bad) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const int64_t row = t / chunks_per_row;            // (b, j, h) of the fresh rows
    const int c = (int)(t - row * chunks_per_row);
    const int h = (int)(row % Hkv);
    const int64_t bj = row / Hkv;
    const int b = (int)(bj / n);
    // the source row does not depend on the position: issue all three loads together
    const uint4 kw = k_new[t];
    const uint4 vw = v_new[t];
    const int p = pos[bj];
    if (p < 0 || p >= L) {
        if (p != -1 && bad && c == 0 && h == 0) atomicAdd(bad, 1);
        return;
    }
    const int64_t dst = (((int64_t)b * Hkv + h) * L + p) * chunks_per_row + c;
    ck[dst] = kw;
    cv[dst] = vw;
}

// ---- e4m3 quantise: 32 lanes per 128-element group, 4 elements per lane ----
template <int SRC>
__global__ __launch_bounds__(256) void scatter_e4m3_kernel(
    const void *__restrict__ k_new, const void *__restrict__ v_new, uint8_t *__restrict__ ck,
    uint8_t *__restrict__ cv, float *__restrict__ ks, float *__restrict__ vs,
    const int32_t *__restrict__ pos, int n, int Hkv, int L, int d, int64_t n_groups,
    int32_t *__restrict__ bad) {
    const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t grp = gt >> 5;                       // global group id over (b, j, h, g)
    const int l32 = threadIdx.x & 31;
    const bool live = grp < n_groups;
    const int ng = d >> 7;
    const int64_t row = live ? grp / ng : 0;           // (b, j, h)
    const int g = live ? (int)(grp - row * ng) : 0;
    const int h = (int)(row % Hkv);
    const int64_t bj = row / Hkv;
    const int b = (int)(bj / n);
    const int p = live ? pos[bj] : -1;
    const bool ok = live && p >= 0 && p < L;
    if (live && !ok && p != -1 && bad && l32 == 0 && h == 0 && g == 0) atomicAdd(bad, 1);

    // every lane takes part in the shuffles below; dead lanes contribute 0
    const int64_t src = row * d + g * 128 + l32 * 4;
    float xk[4], xv[4];
    if (live) {           // not gated on the position: the loads issue together
        if (SRC == DLLM_BF16) {
            const uint2 wk = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(k_new) + src);
            const uint2 wv = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(v_new) + src);
            xk[0] = bf16lo(wk.x); xk[1] = bf16hi(wk.x); xk[2] = bf16lo(wk.y); xk[3] = bf16hi(wk.y);
            xv[0] = bf16lo(wv.x); xv[1] = bf16hi(wv.x); xv[2] = bf16lo(wv.y); xv[3] = bf16hi(wv.y);
        } else {
            const float4 k0 = *reinterpret_cast<const float4 *>(static_cast<const float *>(k_new) + src);
            const float4 v0 = *reinterpret_cast<const float4 *>(static_cast<const float *>(v_new) + src);
            xk[0] = k0.x; xk[1] = k0.y; xk[2] = k0.z; xk[3] = k0.w;
            xv[0] = v0.x; xv[1] = v0.y; xv[2] = v0.z; xv[3] = v0.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) xk[i] = xv[i] = 0.f;
    }
    if (!ok) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xk[i] = xv[i] = 0.f;
    }
    float ak = 0.f, av = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ak = fmaxf(ak, fabsf(xk[i]));
        av = fmaxf(av, fabsf(xv[i]));
    }
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {                // max over the 32 lanes of the group
        ak = fmaxf(ak, __shfl_xor(ak, o, kWave));
        av = fmaxf(av, __shfl_xor(av, o, kWave));
    }
    if (!ok) return;
    const float sk = ak / 448.0f;                      // IEEE float32 divides
    const float sv = av / 448.0f;
    uint32_t ck4 = 0, cv4 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t ek = ak == 0.f ? 0u : e4m3_rne(xk[i] / sk);
        const uint32_t ev = av == 0.f ? 0u : e4m3_rne(xv[i] / sv);
        ck4 |= ek << (8 * i);
        cv4 |= ev << (8 * i);
    }
    const int64_t drow = ((int64_t)b * Hkv + h) * L + p;
    const int64_t dst = drow * d + g * 128 + l32 * 4;
    *reinterpret_cast<uint32_t *>(ck + dst) = ck4;
    *reinterpret_cast<uint32_t *>(cv + dst) = cv4;
    if (l32 == 0) {
        ks[drow * ng + g] = ak == 0.f ? 0.f : sk;
        vs[drow * ng + g] = av == 0.f ? 0.f : sv;
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4 *__restrict__ p, int64_t n16,
                                                        uint8_t *__restrict__ tail, int ntail) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = i; j < n16; j += stride) p[j] = make_uint4(0, 0, 0, 0);
    if (i < ntail) tail[i] = 0;
}

// sinks [0, min(S, e)) then the newest keys [max(S, e-R), e), then -1
__global__ __launch_bounds__(256) void sink_rolling_kernel(int L, int S, int R,
                                                           const int32_t *__restrict__ end,
                                                           int32_t *__restrict__ key_idx,
                                                           int n_keys) {
    const int b = blockIdx.y;
    int e = end[b];
    e = e < 0 ? 0 : (e > L ? L : e);
    const int ns = S < e ? S : e;
    const int start = (e - R) > S ? (e - R) : S;
    const int nr = e > start ? e - start : 0;
    int32_t *out = key_idx + (int64_t)b * n_keys;
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n_keys; j += gridDim.x * blockDim.x)
        out[j] = j < ns ? j : (j < ns + nr ? start + (j - ns) : -1);
}

// Debug check of a position list: per sequence, the entries outside [0, L)
// (other than the padding -1) and the entries repeating a position already
// seen.  One workgroup per sequence marks each position in an LDS bitset; the
// old word of the atomic OR tells whether the bit was set before.  Which of
// two equal entries counts as the repeat depends on the order of the
// atomics, their number does not.
constexpr int kCheckThreads = 1024;
__global__ __launch_bounds__(kCheckThreads) void check_positions_kernel(int L, const int32_t *__restrict__ pos,
                                                                        int n, int32_t *__restrict__ bad,
                                                                        int32_t *__restrict__ dup) {
    extern __shared__ uint32_t seen[];
    __shared__ int part[2][kCheckThreads / kWave];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int words = (L + 31) >> 5;
    for (int w = tid; w < words; w += kCheckThreads) seen[w] = 0;
    __syncthreads();
    int nb = 0, nd = 0;
    const int32_t *row = pos + (int64_t)b * n;
    for (int j = tid; j < n; j += kCheckThreads) {
        const int p = row[j];
        if (p == -1) continue;
        if (p < 0 || p >= L) { ++nb; continue; }
        const uint32_t bit = 1u << (p & 31);
        if (atomicOr(&seen[p >> 5], bit) & bit) ++nd;
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) {
        nb += __shfl_xor(nb, o, kWave);
        nd += __shfl_xor(nd, o, kWave);
    }
    if (lane == 0) { part[0][wave] = nb; part[1][wave] = nd; }
    __syncthreads();
    if (tid == 0) {
        int tb = 0, td = 0;
        for (int w = 0; w < kCheckThreads / kWave; ++w) { tb += part[0][w]; td += part[1][w]; }
        bad[b] = tb;
        dup[b] = td;
    }
}

// Unchanged and changed key positions of one SAR step [LaCache, problem
// statement and Methodology 1]: only the active block [o, o + b) changes
// within a block's denoising steps.  Both lists ascending, one thread per
// position.
__global__ __launch_bounds__(256) void facache_maps_kernel(int L, int b, const int32_t *__restrict__ start,
                                                           int32_t *__restrict__ unchanged_idx,
                                                           int32_t *__restrict__ block_idx) {
    const int bi = blockIdx.y;
    int o = start[bi];
    o = o < 0 ? 0 : (o > L - b ? L - b : o);
    int32_t *un = unchanged_idx + (int64_t)bi * (L - b);
    int32_t *blk = block_idx + (int64_t)bi * b;
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < L; j += gridDim.x * blockDim.x) {
        if (j < o) un[j] = j;
        else if (j < o + b) blk[j - o] = j;
        else un[j - b] = j;
    }
}

}  // namespace

int launch_facache_maps(int B, int L, int b, const int32_t *start, int32_t *unchanged_idx,
                        int32_t *block_idx, hipStream_t s) {
    const unsigned gx = (unsigned)std::min(cdiv(L, 256), 64);
    facache_maps_kernel<<<dim3(gx, (unsigned)B), dim3(256), 0, s>>>(L, b, start, unchanged_idx,
                                                                     block_idx);
    return launch_status();
}

int launch_fill_zero(void *p, size_t bytes, hipStream_t s) {
    if (bytes == 0) return DLLM_OK;
    const int64_t n16 = (int64_t)(bytes / 16);
    const int ntail = (int)(bytes % 16);
    const int64_t blocks = std::min<int64_t>(std::max<int64_t>(cdiv64(n16, 256), 1), 8192);
    fill_zero_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        static_cast<uint4 *>(p), n16, static_cast<uint8_t *>(p) + n16 * 16, ntail);
    return launch_status();
}

int launch_scatter(const dllm_kv_cache &c, const void *k_new, const void *v_new, int src_dtype,
                   const int32_t *pos, int n, int32_t *bad, hipStream_t s) {
    if (n == 0) return DLLM_OK;
    const int Hkv = c.n_kv_heads, d = c.d_head, L = c.L;
    const int64_t rows = (int64_t)c.B * n * Hkv;
    if (c.dtype == DLLM_E4M3) {
        const int64_t groups = rows * (d / 128);
        const int64_t threads = groups * 32;
        const unsigned blocks = (unsigned)cdiv64(threads, 256);
        if (src_dtype == DLLM_BF16)
            scatter_e4m3_kernel<DLLM_BF16><<<blocks, 256, 0, s>>>(
                k_new, v_new, static_cast<uint8_t *>(c.k), static_cast<uint8_t *>(c.v), c.k_scale,
                c.v_scale, pos, n, Hkv, L, d, groups, bad);
        else
            scatter_e4m3_kernel<DLLM_F32><<<blocks, 256, 0, s>>>(
                k_new, v_new, static_cast<uint8_t *>(c.k), static_cast<uint8_t *>(c.v), c.k_scale,
                c.v_scale, pos, n, Hkv, L, d, groups, bad);
        return launch_status();
    }
    const int esz = c.dtype == DLLM_F32 ? 4 : 2;
    const int cpr = d * esz / 16;
    const int64_t total = rows * cpr;
    scatter_copy_kernel<<<(unsigned)cdiv64(total, 256), 256, 0, s>>>(
        static_cast<const uint4 *>(k_new), static_cast<const uint4 *>(v_new),
        static_cast<uint4 *>(c.k), static_cast<uint4 *>(c.v), pos, n, Hkv, L, cpr, total, bad);
    return launch_status();
}

int launch_check_positions(int B, int L, const int32_t *pos, int n, int32_t *bad, int32_t *dup,
                           hipStream_t s) {
    const size_t shmem = sizeof(uint32_t) * (size_t)((L + 31) / 32);   // <= 16 KB for L <= 131072
    check_positions_kernel<<<dim3((unsigned)B), dim3(kCheckThreads), shmem, s>>>(L, pos, n, bad, dup);
    return launch_status();
}

int launch_sink_rolling(int B, int L, int S, int R, const int32_t *end, int32_t *key_idx,
                        int n_keys, hipStream_t s) {
    const unsigned gx = (unsigned)std::min(cdiv(n_keys, 256), 64);
    sink_rolling_kernel<<<dim3(gx, (unsigned)B), dim3(256), 0, s>>>(L, S, R, end, key_idx, n_keys);
    return launch_status();
}

}  // namespace dllm
