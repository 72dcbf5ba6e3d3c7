// Per-group FP8 for the FFN [LaCache explainer, Methodology 2]: activations
// quantised in 1 x 128 groups and weights in 128 x 128 blocks, the Gate-Up
// and FF-Out products on FP8 matrix cores, the quantisation fused into the
// add & norm before the FFN and into the SwiGLU between the two products.
//
// Each group's scale is a power of two 2^e, stored as its E8M0 code e + 127
// (e the smallest >= -127 with amax <= 448 * 2^e), so that gfx950's
// block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) applies the scales of
// both operands itself: one fp32 accumulator per output element, no
// per-group rescale on the vector ALU.  Dividing by a power of two is exact,
// so a code is RNE_e4m3(x * 2^-e).
//
// Scale layouts: activations [K/128, M] (one byte per row per group, the
// rows of one group contiguous, as one k-step of the product reads them);
// weights [N/128, K/128].
#include "attn_common.hpp"

#include <climits>
#include <type_traits>

namespace dllm {
namespace {

using attn::lds_dma16;
using attn::vm_wait;
using attn::xcd_remap;

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

// smallest e >= -127 with amax <= 448 * 2^e.  For a normal amax = f 2^E,
// f in [1, 2), and 448 = 1.75 * 2^8: e = E - 8 when f <= 1.75 (fraction
// field <= 0x600000), else E - 7; a subnormal amax takes the same rule
// through frexpf.
__device__ __forceinline__ int e8m0_exponent(float amax) {
    if (!(amax > 0.f)) return -127;
    const uint32_t u = __float_as_uint(amax);
    int e;
    if (u >= 0x00800000u) {
        e = (int)(u >> 23) - 127 - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
    } else {
        int E;
        const float f = frexpf(amax, &E);              // amax = f 2^E, f in [0.5, 1)
        e = f <= 0.875f ? E - 9 : E - 8;
    }
    return e < -127 ? -127 : e;
}

// 2^-e for an exponent of e8m0_exponent (-e in [-120, 127]: a normal float)
__device__ __forceinline__ float inv_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// four values already scaled into [-448, 448] -> four e4m3 codes in one word.
// gfx950's v_cvt_pk_fp8_f32 rounds to nearest even; over every float32 in
// [-448, 448] it gives the same codes as the bitwise encoder e4m3_rne (an
// exhaustive check), so the quantisers keep their results bit for bit.
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// 8 values of one group -> 8 codes (two words); the power-of-two scale
// multiplies exactly
__device__ __forceinline__ uint2 encode8(const float *x, int e) {
    const float s = inv_scale(e);
    return make_uint2(cvt4(x[0] * s, x[1] * s, x[2] * s, x[3] * s), cvt4(x[4] * s, x[5] * s, x[6] * s, x[7] * s));
}

template <int DT>
__device__ __forceinline__ void load8(const void *p, int64_t i, float *x) {
    if (DT == DLLM_BF16) {
        const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p) + i);
        const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = bf16lo(a[j]);
            x[2 * j + 1] = bf16hi(a[j]);
        }
    } else {
        const float4 *q = reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
        const float4 u = q[0], v = q[1];
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
        x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
    }
}

__device__ __forceinline__ float max16(float v) {       // over the 16 lanes of a group
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, shfl_xor_f(v, o));
    return v;
}

// ---- activations: 16 lanes per 1 x 128 group, 8 values per lane ------------
template <int DT>
__global__ __launch_bounds__(256) void fp8_quant_rows_kernel(const void *__restrict__ x, int64_t ld,
                                                             int64_t M, int K, uint8_t *__restrict__ codes,
                                                             uint8_t *__restrict__ scales) {
    const int G = K / 128;
    const int64_t grp = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
    const int l16 = threadIdx.x & 15;
    const bool live = grp < M * G;
    const int64_t m = live ? grp / G : 0;
    const int g = live ? (int)(grp - m * G) : 0;
    float v[8];
    if (live) load8<DT>(x, m * ld + g * 128 + l16 * 8, v);
    else
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.f;
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
    a = max16(a);                                      // every lane joins the shuffles
    if (!live) return;
    const int e = e8m0_exponent(a);
    *reinterpret_cast<uint2 *>(codes + m * K + g * 128 + l16 * 8) = encode8(v, e);
    if (l16 == 0) scales[(int64_t)g * M + m] = (uint8_t)(e + 127);
}

// ---- add & RMS norm, then the 1 x 128 groups of the normalised row ----------
// One workgroup per row: r = x + res in fp32, rounded to the stream dtype
// (res_out); y = gamma * r / sqrt(mean(r^2) + eps); the rounded r waits in
// LDS for the second pass.
template <int DT>
__global__ __launch_bounds__(256) void fp8_addnorm_quant_kernel(
    const void *__restrict__ x, const void *__restrict__ res, const void *__restrict__ gamma,
    float eps, int64_t M, int K, void *__restrict__ res_out, uint8_t *__restrict__ codes,
    uint8_t *__restrict__ scales) {
    extern __shared__ float sr[];                      // K floats
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    float ss = 0.f;
    for (int c = tid * 8; c < K; c += 256 * 8) {
        float a[8], b[8];
        load8<DT>(x, m * K + c, a);
        if (res) load8<DT>(res, m * K + c, b);
        else
#pragma unroll
            for (int i = 0; i < 8; ++i) b[i] = 0.f;
        float r[8];
        if (DT == DLLM_BF16) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint16_t lo = f32_to_bf16(a[2 * i] + b[2 * i]);
                const uint16_t hi = f32_to_bf16(a[2 * i + 1] + b[2 * i + 1]);
                w[i] = (uint32_t)lo | ((uint32_t)hi << 16);
                r[2 * i] = bf16_to_f32(lo);
                r[2 * i + 1] = bf16_to_f32(hi);
            }
            if (res_out)
                *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(res_out) + m * K + c) =
                    make_uint4(w[0], w[1], w[2], w[3]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) r[i] = a[i] + b[i];
            if (res_out) {
                float4 *o = reinterpret_cast<float4 *>(static_cast<float *>(res_out) + m * K + c);
                o[0] = make_float4(r[0], r[1], r[2], r[3]);
                o[1] = make_float4(r[4], r[5], r[6], r[7]);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sr[c + i] = r[i];
            ss = fmaf(r[i], r[i], ss);
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += shfl_xor_f(ss, o);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    ss = (red[0] + red[1]) + (red[2] + red[3]);
    const float inv = 1.0f / sqrtf(ss / (float)K + eps);
    const int G = K / 128;
    const int l16 = tid & 15;
    // groups in rounds of 16 (one per 16 lanes); every lane of a round's waves
    // joins the shuffles
    for (int g0 = 0; g0 < G; g0 += 16) {
        const int g = g0 + (tid >> 4);
        const bool live = g < G;
        float y[8], gm[8];
        float a = 0.f;
        if (live) {
            load8<DT>(gamma, g * 128 + l16 * 8, gm);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                y[i] = sr[g * 128 + l16 * 8 + i] * inv * gm[i];
                a = fmaxf(a, fabsf(y[i]));
            }
        }
        a = max16(a);
        if (!live) continue;
        const int e = e8m0_exponent(a);
        *reinterpret_cast<uint2 *>(codes + m * K + g * 128 + l16 * 8) = encode8(y, e);
        if (l16 == 0) scales[(int64_t)g * M + m] = (uint8_t)(e + 127);
    }
}

// ---- weights: one workgroup per 128 x 128 block, 64 values per thread -------
template <int DT>
__global__ __launch_bounds__(256) void fp8_quant_weight_kernel(const void *__restrict__ w, int N, int K,
                                                               uint8_t *__restrict__ codes,
                                                               uint8_t *__restrict__ scales) {
    __shared__ float red[4];
    const int kb = K / 128;
    const int bn = blockIdx.x / kb, bk = blockIdx.x % kb;
    const int tid = threadIdx.x;
    const int r = tid >> 1, h = tid & 1;               // row of the block, half of the row
    const int64_t base = (int64_t)(bn * 128 + r) * K + bk * 128 + h * 64;
    float v[64];
#pragma unroll
    for (int j = 0; j < 8; ++j) load8<DT>(w, base + j * 8, v + j * 8);
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) a = fmaxf(a, fabsf(v[i]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, shfl_xor_f(a, o));
    if ((tid & 63) == 0) red[tid >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int e = e8m0_exponent(a);
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<uint2 *>(codes + base + j * 8) = encode8(v + j * 8, e);
    if (tid == 0) scales[blockIdx.x] = (uint8_t)(e + 127);
}

// ---- the product: C = dequant(A) dequant(B)^T -------------------------------
// A [M, K] codes with scales [K/128, M]; B [N, K] codes with scales
// [N/128, K/128]; fp32 accumulation.  A workgroup of 4 waves owns a 256 x 256
// tile, each wave 128 x 128 (4 x 4 tiles of 32 x 32), and walks K in slices
// of 64 through a ring of four LDS stages (A and B, 16 KB each per stage),
// filled by direct-to-LDS loads four slices ahead of use.  The operands of
// slice h + 1 are read into registers while the products of slice h run on
// the registers read one slice earlier, so the matrix cores never wait for
// an LDS read, and the one barrier per slice only confirms that slice h + 1
// has landed and that slice h's stage is free for its refill.  In LDS a
// 64-byte row keeps its four 16-byte chunks XOR-swizzled (swz) so that a
// read phase of 16 rows at one logical chunk hits all 64 banks once.
//
// Operands of v_mfma_scale_f32_32x32x64_f8f6f4: lane l holds 32 bytes of
// row l % 32 (A) or of column l % 32 (B), K bytes 32 (l / 32) .. +31 of the
// 64-byte k-chunk; the same lane half and byte on both sides is the same K
// index.  Each lane also passes its row's (column's) E8M0 scale, one per
// 128-wide group, so both scales multiply inside the instruction.  Lane l,
// register i of the result holds row 8 (i / 4) + 4 (l / 32) + i % 4,
// column l % 32.
//
// EPI 0 writes C in bf16.  EPI 1 is SwiGLU with the 1 x 128 quantisation of
// its output: B's rows come in pairs of 128-row blocks (gate block j, then
// up block j).  Wave wn takes gate features 64 wn .. +63 of the block and
// the matching up features, so silu(gate) * up is formed in its own
// registers, and it computes C^T (A operand = the weight rows, B operand =
// the token rows): lane l then holds token l % 32 of each token tile and, in
// register i, feature 8 (i / 4) + 4 (l / 32) + i % 4 of each feature tile, so
// a token's 64 values of the wave are in two lanes (one swap gives their
// maximum), four neighbouring features pack into one word of codes, and the
// two waves of a block exchange one partial maximum per token.  It writes
// codes of [M, N/2] with scales [N/256, M].
constexpr int kBM = 256, kBN = 256, kBK = 128;         // kBK: one scale group
constexpr int kHK = 64;                                // K width of one LDS stage
constexpr int kStages = 4;
constexpr int kSliceBytes = kBM * kHK;                 // one operand tile of one stage: 16 KB
constexpr int kGemmLds = kStages * 2 * kSliceBytes;    // 128 KB
constexpr int kGemmMaxK = 12288;                       // the scales of 96 groups fit beside them
constexpr int kGemmSmem = kGemmLds + (kGemmMaxK / kBK) * (256 + 2);
static_assert(kGemmSmem <= attn::kLdsBytes, "LDS of one workgroup");

// the block-scaled product with byte `sel` (0..3) of sa as A's scale
__device__ __forceinline__ f32x16_t mfma_scaled(const i32x8_t &a, const i32x8_t &b, const f32x16_t &c,
                                                int sa, int sel, int sb) {
    switch (sel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 1, sa, 0, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 2, sa, 0, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 3, sa, 0, sb);
    }
}

// the block-scaled product with byte `sel` (0..3) of sb as B's scale
__device__ __forceinline__ f32x16_t mfma_scaled_b(const i32x8_t &a, const i32x8_t &b, const f32x16_t &c,
                                                  int sa, int sb, int sel) {
    switch (sel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 1, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 2, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 3, sb);
    }
}

// LDS byte offset of 16-byte chunk c (0..3) of stage row r.  A read phase of
// 16 lanes takes rows r .. r + 15 at one logical chunk, and the 64 banks span
// 256 bytes, i.e. four 64-byte rows: rows of equal r % 4 share a quarter of
// the bank window, so the four rows of each residue need distinct chunks:
// c ^ ((r >> 2) & 3).
__device__ __forceinline__ int swz(int r, int c) { return r * kHK + ((c ^ ((r >> 2) & 3)) << 4); }

// one slice's operands of one wave, and the E8M0 scales of its group
struct GemmOps {
    i32x8_t a[4], b[4];
    int sa, sb, su;
};

template <int EPI>
__global__ __launch_bounds__(256, 1) void fp8_gemm_kernel(
    const uint8_t *__restrict__ a, const uint8_t *__restrict__ sa, const uint8_t *__restrict__ b,
    const uint8_t *__restrict__ sb, int M, int N, int K, int tiles_m, int tiles_n,
    uint16_t *__restrict__ c, uint8_t *__restrict__ qc, uint8_t *__restrict__ qs) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kGemmSmem];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, lh = lane >> 5;

    // tile order: the 8 XCDs each take one contiguous run of the logical
    // order, which walks groups of 8 tile rows column by column, so the
    // tiles in flight on one XCD share A rows and B columns in its L2
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int per_group = 8 * tiles_n;
    const int grp = lid / per_group, first_m = grp * 8;
    const int gsize = min(tiles_m - first_m, 8);
    const int in_g = lid - grp * per_group;
    const int tm = first_m + in_g % gsize, tn = in_g / gsize;
    const int m0 = tm * kBM, n0 = tn * kBN;
    const int ksteps = K / kBK;

    // direct-to-LDS loads of slice h: wave w issues 1 KB loads u = 0..3 of
    // each tile; load u covers stage rows 16 (4 w + u) .. +15, lane i row
    // r = 16 (4 w + u) + i / 4, stored slot i % 4, which holds logical chunk
    // (i % 4) ^ ((r >> 2) & 3) = (i % 4) ^ ((i / 16) & 3).  Each lane's byte
    // offset from the slice's wave-uniform base is fixed for the whole loop.
    const int H = K / kHK;
    const int lchunk = (lane & 3) ^ ((lane >> 4) & 3);
    uint32_t offa[4], offb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = 16 * (4 * wave + u) + (lane >> 2);
        offa[u] = (uint32_t)(min(r, M - 1 - m0) * K + lchunk * 16);   // rows past M read row M - 1, never stored
        offb[u] = (uint32_t)(r * K + lchunk * 16);
    }
    const uint8_t *abase = a + (int64_t)m0 * K, *bbase = b + (int64_t)n0 * K;
    const uint32_t smem_lds = attn::lds_addr(smem);
    auto issue = [&](int h) {
        const uint32_t st = smem_lds + (uint32_t)((h & (kStages - 1)) * 2 * kSliceBytes);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            lds_dma16<false>(abase + h * kHK, offa[u], st + (4 * wave + u) * 1024);
            lds_dma16<false>(bbase + h * kHK, offb[u], st + kSliceBytes + (4 * wave + u) * 1024);
        }
    };
    // All E8M0 scales of the tile wait in LDS, read once in a prologue: the A
    // scales of group g at ssa + 256 g, packed so that the word at
    // 128 wm + 4 l32 holds the scales of this lane's row in row tiles 0..3
    // (the MFMA's op_sel picks the byte), the B scales of the wave's 128
    // columns at ssb[ksteps wn + g].  The loop then issues no global load
    // the compiler sees, so it places no wait of its own (one would also wait
    // for the direct-to-LDS loads in flight, which it cannot see).
    unsigned char *ssa = smem + kGemmLds;
    unsigned char *ssb = ssa + ksteps * 256;
#pragma unroll
    for (int h = 0; h < kStages - 1; ++h)               // the first slices load under the prologue
        if (h < H) issue(h);
    {
        // thread t reads row m0 + t of every group (256 threads read one
        // group's 256 contiguous bytes together), 16 groups' loads in flight
        const int wq = tid >> 7, rq = (tid >> 5) & 3, lq = tid & 31;   // tid = 128 wm + 32 rt + l32
        const uint8_t *src = sa + min(m0 + tid, M - 1);
        unsigned char *dst = ssa + wq * 128 + lq * 4 + rq;
        for (int k0 = 0; k0 < ksteps; k0 += 16) {
            uint8_t v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (k0 + j < ksteps) v[j] = src[(int64_t)(k0 + j) * M];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (k0 + j < ksteps) dst[(k0 + j) * 256] = v[j];
        }
        if (tid < 2 * ksteps)
            ssb[tid] = sb[(int64_t)((n0 >> 7) + tid / ksteps) * ksteps + tid % ksteps];
    }

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // B tile row of operand tile t: EPI 0 the wave's 128 rows; EPI 1 its
    // gate rows 64 wn .. +63 (t = 0, 1) and up rows 128 + 64 wn .. +63
    auto brow = [&](int t) { return EPI == 1 ? (t < 2 ? 64 * wn + 32 * t : 64 + 64 * wn + 32 * t) : 128 * wn + 32 * t; };
    // operand pair t of slice h (t = 0..3: A tile t; 4..7: B tile t - 4)
    auto read_pair = [&](int h, int t, GemmOps &o) {
        const unsigned char *st = smem + (h & (kStages - 1)) * 2 * kSliceBytes;
        const int tt = t & 3;
        const int r = t < 4 ? wm * 128 + tt * 32 + l32 : brow(tt) + l32;
        const unsigned char *base = t < 4 ? st : st + kSliceBytes;
        const uint4 x0 = *reinterpret_cast<const uint4 *>(base + swz(r, 2 * lh));
        const uint4 x1 = *reinterpret_cast<const uint4 *>(base + swz(r, 2 * lh + 1));
        const i32x8_t v = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        if (t < 4) o.a[tt] = v;
        else o.b[tt] = v;
    };
    // EPI 0: the scale of the wave's 128 B rows; EPI 1: of the gate block
    // (sb) and of the up block (su)
    auto read_scales = [&](int h, GemmOps &o) {
        const int g = h >> 1;
        o.sa = *reinterpret_cast<const int *>(ssa + g * 256 + wm * 128 + l32 * 4);
        o.sb = ssb[(EPI == 1 ? 0 : wn) * ksteps + g];
        o.su = EPI == 1 ? (int)ssb[ksteps + g] : 0;
    };
    auto product = [&](int i, const GemmOps &o) {
        if (EPI == 1) {
            // C^T: acc[ft][tt], feature tile ft (gate 0, 1; up 2, 3) by token tile tt
            const int tt = i >> 2, ft = i & 3;
            acc[ft][tt] = mfma_scaled_b(o.b[ft], o.a[tt], acc[ft][tt], ft < 2 ? o.sb : o.su, o.sa, tt);
        } else {
            const int rt = i >> 2, ct = i & 3;
            acc[rt][ct] = mfma_scaled(o.a[rt], o.b[ct], acc[rt][ct], o.sa, rt, o.sb);
        }
    };
    // one slice: confirm slice h + 1 and free slice h's stage (a barrier
    // after this wave's own loads of h + 1 and its reads of h), then the 16
    // products of slice h with the reads of slice h + 1 and the refill of
    // slice h + 4 interleaved between them.  MORE: a slice h + 1 exists;
    // REFILL: a slice h + 4 exists; `ahead`: slices loaded after h + 1.
    auto slice = [&](auto more_t, auto refill_t, int h, int ahead, const GemmOps &cur, GemmOps &nxt) {
        constexpr bool MORE = decltype(more_t)::value, REFILL = decltype(refill_t)::value;
        if (MORE) {
            if (ahead >= 2) vm_wait<16>();
            else if (ahead == 1) vm_wait<8>();
            else vm_wait<0>();
            __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
            asm volatile("s_barrier" ::: "memory");
            read_scales(h + 1, nxt);
        }
        const uint32_t st = smem_lds + (uint32_t)((h & (kStages - 1)) * 2 * kSliceBytes);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            product(i, cur);
            if (MORE && i < 8) read_pair(h + 1, i, nxt);
            if (REFILL && i >= 8 && i < 12) {
                const int u = i - 8;
                lds_dma16<false>(abase + (h + kStages) * kHK, offa[u], st + (4 * wave + u) * 1024);
                lds_dma16<false>(bbase + (h + kStages) * kHK, offb[u], st + kSliceBytes + (4 * wave + u) * 1024);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using T = std::true_type;
    using F = std::false_type;

    GemmOps o0, o1;
    vm_wait<0>();
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
    asm volatile("s_barrier" ::: "memory");
    read_scales(0, o0);
#pragma unroll
    for (int t = 0; t < 8; ++t) read_pair(0, t, o0);
    if (kStages - 1 < H) issue(kStages - 1);
    // H is even (K is a multiple of 128), so slice h reads o0 for even h
    int h = 0;
    for (; h < H - kStages; h += 2) {
        slice(T{}, T{}, h, 2, o0, o1);
        slice(T{}, T{}, h + 1, 2, o1, o0);
    }
    for (; h < H - 2; h += 2) {                        // at most once: slices H - 4, H - 3
        slice(T{}, F{}, h, min(H - 1, h + 3) - (h + 1), o0, o1);
        slice(T{}, F{}, h + 1, min(H - 1, h + 4) - (h + 2), o1, o0);
    }
    slice(T{}, F{}, h, 0, o0, o1);                     // h = H - 2
    slice(F{}, F{}, h + 1, 0, o1, o0);

    // ---- epilogues: the tile leaves through LDS (the stages are free once
    // every wave is past its last step) so that global stores are 16 bytes
    // per lane along the output rows
    __syncthreads();
    if (EPI == 0) {
        // each wave's 128 x 128 bf16 block, row-major, 16-byte chunks of a row
        // XOR-swizzled by the row's low 4 bits
        unsigned char *blk = smem + wave * (128 * 256);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = rt * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
                    const int col = ct * 32 + l32;
                    *reinterpret_cast<uint16_t *>(blk + r * 256 + ((((col >> 3) ^ (r & 15)) << 4) | ((col & 7) << 1))) =
                        f32_to_bf16(acc[rt][ct][i]);
                }
        __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));   // this wave's writes
        // 16 lanes per row, 4 rows per pass
#pragma unroll
        for (int p = 0; p < 32; ++p) {
            const int r = p * 4 + (lane >> 4), ch = lane & 15;
            const uint4 v = *reinterpret_cast<const uint4 *>(blk + r * 256 + ((ch ^ (r & 15)) << 4));
            const int row = m0 + wm * 128 + r;
            if (row < M)
                *reinterpret_cast<uint4 *>(c + (int64_t)row * N + n0 + wn * 128 + ch * 8) = v;
        }
    } else {
        // silu(gate) * up of this wave's 64 features (ft = 0, 1; up in
        // ft + 2) of its 128 tokens, each token's partial maximum over them
        // (a lane's 32 values, then lanes l and l ^ 32), the partner wave's
        // partial maximum through LDS, the exponent and the codes.  Lane
        // (l32, lh) holds token 32 tt + l32, features 32 ft + 8 q + 4 lh + j
        // in register 4 q + j: four neighbouring features make one word.
        float h[2][4][16];
        float pm[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            float v = 0.f;
#pragma unroll
            for (int ft = 0; ft < 2; ++ft)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float g = acc[ft][tt][i], u = acc[ft + 2][tt][i];
                    h[ft][tt][i] = __fdividef(g, 1.0f + __expf(-g)) * u;
                    v = fmaxf(v, fabsf(h[ft][tt][i]));
                }
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
            pm[tt] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        float *xm = reinterpret_cast<float *>(smem) + wm * 256;       // [wn][128 tokens]
        if (lh == 0) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) xm[wn * 128 + 32 * tt + l32] = pm[tt];
        }
        __syncthreads();
        // the codes wait in LDS: [128 tokens][64 codes] per wave, the four
        // 16-byte chunks of a token's row XOR-swizzled by (row / 4) % 4
        unsigned char *qb = smem + 4096 + wave * 8192;
        int ex[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const float full = fmaxf(pm[tt], xm[(wn ^ 1) * 128 + 32 * tt + l32]);
            ex[tt] = e8m0_exponent(full);
            const float sc = inv_scale(ex[tt]);
            const int r = 32 * tt + l32;
#pragma unroll
            for (int ft = 0; ft < 2; ++ft)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t w = cvt4(h[ft][tt][4 * q] * sc, h[ft][tt][4 * q + 1] * sc,
                                            h[ft][tt][4 * q + 2] * sc, h[ft][tt][4 * q + 3] * sc);
                    const int col = 32 * ft + 8 * q + 4 * lh;             // byte of the token's 64
                    *reinterpret_cast<uint32_t *>(qb + r * 64 + ((((col >> 4) ^ ((r >> 2) & 3))) << 4) + (col & 15)) = w;
                }
        }
        __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));   // this wave's writes
        // the wave's 128 tokens x 64 codes: 4 lanes per token, 16 tokens per pass
        const int half_n = N >> 1;
        const int tbase = m0 + wm * 128;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int r = p * 16 + (lane >> 2), ch = lane & 3;
            const uint4 v = *reinterpret_cast<const uint4 *>(qb + r * 64 + ((ch ^ ((r >> 2) & 3)) << 4));
            if (tbase + r < M)
                *reinterpret_cast<uint4 *>(qc + (int64_t)(tbase + r) * half_n + (n0 >> 1) + 64 * wn + ch * 16) = v;
        }
        if (wn == 0 && lh == 0) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
                if (tbase + 32 * tt + l32 < M) qs[(int64_t)(n0 >> 8) * M + tbase + 32 * tt + l32] = (uint8_t)(ex[tt] + 127);
        }
    }
}

}  // namespace

int launch_fp8_quant_rows(const void *x, int dtype, int64_t ld, int64_t M, int K, uint8_t *codes,
                          uint8_t *scales, hipStream_t s) {
    if (M == 0) return DLLM_OK;
    const int64_t threads = M * (K / 128) * 16;
    const unsigned blocks = (unsigned)cdiv64(threads, 256);
    if (dtype == DLLM_BF16)
        fp8_quant_rows_kernel<DLLM_BF16><<<blocks, 256, 0, s>>>(x, ld, M, K, codes, scales);
    else
        fp8_quant_rows_kernel<DLLM_F32><<<blocks, 256, 0, s>>>(x, ld, M, K, codes, scales);
    return launch_status();
}

int launch_fp8_addnorm_quant(const void *x, const void *res, const void *gamma, int dtype, float eps,
                             int64_t M, int K, void *res_out, uint8_t *codes, uint8_t *scales,
                             hipStream_t s) {
    if (M == 0) return DLLM_OK;
    const size_t lds = (size_t)K * sizeof(float);
    if (dtype == DLLM_BF16)
        fp8_addnorm_quant_kernel<DLLM_BF16><<<(unsigned)M, 256, lds, s>>>(x, res, gamma, eps, M, K, res_out,
                                                                          codes, scales);
    else
        fp8_addnorm_quant_kernel<DLLM_F32><<<(unsigned)M, 256, lds, s>>>(x, res, gamma, eps, M, K, res_out,
                                                                         codes, scales);
    return launch_status();
}

int launch_fp8_quant_weight(const void *w, int dtype, int N, int K, uint8_t *codes, uint8_t *scales,
                            hipStream_t s) {
    const unsigned blocks = (unsigned)((N / 128) * (K / 128));
    if (dtype == DLLM_BF16)
        fp8_quant_weight_kernel<DLLM_BF16><<<blocks, 256, 0, s>>>(w, N, K, codes, scales);
    else
        fp8_quant_weight_kernel<DLLM_F32><<<blocks, 256, 0, s>>>(w, N, K, codes, scales);
    return launch_status();
}

int launch_fp8_gemm(const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb, int M,
                    int N, int K, int epilogue, uint16_t *c, uint8_t *qc, uint8_t *qs, hipStream_t s) {
    const int tiles_m = cdiv(M, kBM), tiles_n = N / kBN;
    const int64_t blocks = (int64_t)tiles_m * tiles_n;
    if (blocks > INT_MAX) return DLLM_ERANGE;
    if (epilogue == 0)
        fp8_gemm_kernel<0><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a, sa, b, sb, M, N, K, tiles_m,
                                                                        tiles_n, c, qc, qs);
    else
        fp8_gemm_kernel<1><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a, sa, b, sb, M, N, K, tiles_m,
                                                                        tiles_n, c, qc, qs);
    return launch_status();
}

}  // namespace dllm
