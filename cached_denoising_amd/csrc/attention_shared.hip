// Block attention for grouped queries: the same product as the per-wave MFMA
// path, out = softmax(q K^T * scale) V over the selected keys with no causal
// mask [LaCache explainer, problem statement and Methodology 1; attention-
// sinks page, 2.1 and 2.3], laid out for shapes where several 32-row groups
// of queries read each KV head (G query heads times b block queries > 32).
//
// A workgroup of NRG (2 or 4) waves owns one (sequence, KV head, row chunk,
// key split); wave w owns 32 rows of the chunk, and every wave walks the same
// key tiles.  Each 32-key tile's K rows, V rows and (e4m3) per-key scales are
// loaded once per workgroup, straight from HBM into a ring of LDS stages
// (global_load_lds, no registers), the loads of one tile spread over the
// waves.  Per tile a wave waits for its own loads, then one workgroup
// barrier makes the whole tile visible and frees the stage the previous tile
// used, which the next tile's loads then fill.  Each wave then forms
// S^T = K Q^T with its queries held in registers for the whole walk:
//   bf16 cache: A = K rows (16-byte chunks XOR-swizzled so that a read phase
//     hits distinct banks) and B = the queries on v_mfma_f32_16x16x32_bf16;
//   e4m3 cache: A = the K codes as they landed in the ring and B = the
//     queries split exactly into two e4m3 parts, hi + lo, each with a power-
//     of-two scale per 32 dimensions, on the block-scaled
//     v_mfma_scale_f32_16x16x128_f8f6f4 (two products per 16x16 tile, at
//     twice the rate of bf16, so the product costs what the bf16 one does
//     and the K tile is never widened); the per-key K scale then multiplies
//     the scores.
// It runs the base-2 online softmax with the lazy max, and accumulates
// O^T += V^T P^T with V^T read transposed from a row-major bf16 V tile (an
// e4m3 V tile is widened exactly to bf16 once per workgroup, and its per-key
// scale multiplies P).  Compared with one wave per key run,
// the K/V bytes cross L2 once per workgroup instead of once per row group,
// and the query rows are loaded once.  Key splits write (m, l, O~) partials
// for the merge kernel of the per-wave path.  With a memoized state per row
// (FACache [LaCache, Methodology 1]: the state of the unchanged keys), the
// rows start from it instead of the empty state, so only the changed keys
// are walked.
#include "attn_common.hpp"

#include <climits>
#include <type_traits>

namespace dllm {
namespace {

using namespace attn;

constexpr int kNS = 4;                 // LDS ring stages (bf16): three tiles in flight while one is used
constexpr int kNS8 = 4;                // LDS ring stages (e4m3): K of one tile is read from the ring
                                       // while the next is widened and one more is in flight (a fifth
                                       // or sixth stage measured no faster)
constexpr int kTableKeys = 2048;       // key indices of one split held in LDS (with a key map)

// XOR swizzle of the 16-byte chunks of K row kappa in LDS.  One 8-lane phase
// of an A-operand read touches rows 4t + {0..3} and 8 + 4t + {0..3} (plus a
// multiple of 16) at one logical chunk; the swizzle sends those 8 rows to 8
// distinct 16-byte bank groups.
__device__ __forceinline__ int kswz(int kappa) { return (kappa & 3) | ((kappa >> 1) & 4); }
// The same for 256-byte rows (bf16, d = 128), read in 16-lane phases over the
// 64 banks: a phase touches rows {0..3, 8..11, 16..19, 24..27} + 4t at one
// logical chunk, and these 16 rows go to 16 distinct 16-byte bank groups.
__device__ __forceinline__ int kswz16(int kappa) { return (kappa & 3) | ((kappa >> 1) & 12); }
// The same for 128-byte e4m3 K rows read as the A operand of the 16x16x128
// product: a 16-lane phase reads rows {0..3, 8..11, 16..19, 24..27} + 4t at
// one logical chunk; the row parity picks the 128-byte half of the 256-byte
// bank line and this swizzle the 16-byte bank group within it, so the 16 rows
// hit 16 distinct bank groups.
__device__ __forceinline__ int kswz8(int kappa) { return ((kappa >> 1) & 1) | ((kappa >> 2) & 6); }
// V rows of 256 bytes: a 32-lane phase of the transposed reads touches rows
// {0..3, 8..11} (+4) at logical chunks {2dt, 2dt+1}; bits 1..3 separate those
// 8 rows, bit 0 separates neighbouring rows for the widening's writes.
__device__ __forceinline__ int vswz16(int rho) { return 2 * ((rho & 3) | ((rho >> 1) & 4)) | (rho & 1); }
__device__ __forceinline__ int vswz_bf16(int rho) { return vswz<DLLM_BF16>(rho); }
__device__ __forceinline__ int vswz_e4m3(int rho) { return vswz<DLLM_E4M3>(rho); }

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, MAXN]
template <int MAXN>
__device__ __forceinline__ void vm_wait_upto(int n) {
    if constexpr (MAXN <= 0) {
        vm_wait<0>();
    } else {
        if (n >= MAXN) vm_wait<MAXN>();
        else vm_wait_upto<MAXN - 1>(n);
    }
}

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
constexpr int kE8M0One = 127;          // E8M0 code of the scale 1.0

// Block exponent of a 32-value query block with largest magnitude a: the
// block divided by 2^e lies in [128, 256) at its largest (e4m3 holds up to
// 448), clamped so that e and e - 4 are E8M0 scales; 0 for an all-zero block.
__device__ __forceinline__ int query_block_exp(float a) {
    if (!(a > 0.f)) return 0;
    const int ex = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;   // floor(log2 a); -127 if subnormal
    return min(max(ex - 7, -123), 127);
}

// The queries as the B operand of the block-scaled 16x16x128 e4m3 product.
// Lane (l16, g) holds dims 32g .. 32g+31 of row l16 (w: 32 bf16 values); its
// bytes 0..15 belong to scale block g/2 and bytes 16..31 to block 2 + g/2,
// and it supplies the scale of block g of its row (the operand's scale
// layout: a block's scale sits in the lane of its row plus 16 times the block
// index).  Each value x of a block with exponent e is split exactly into
// x = hi * 2^e + lo * 2^(e-4): hi = x / 2^e rounded to e4m3, lo = the rest
// times 16, which has at most 4 significant bits when x has bf16's 8 (values
// more than 13 binades below the block's largest lose bits of lo, an error
// below 2^-17 of the block's largest).  p[0] / p[1] hold hi / lo, sc[0] /
// sc[1] their E8M0 scales.
__device__ __forceinline__ void split_query(const uint4 (&w)[4], int g, i32x8_t (&p)[2], int (&sc)[2]) {
    float x[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t u[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[8 * c + 2 * k] = __uint_as_float(u[k] << 16);
            x[8 * c + 2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
        }
    }
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        a0 = fmaxf(a0, fabsf(x[j]));
        a1 = fmaxf(a1, fabsf(x[16 + j]));
    }
    // lanes g and g^1 hold the two halves of blocks g/2 and 2 + g/2
    a0 = fmaxf(a0, __shfl_xor(a0, 16));
    a1 = fmaxf(a1, __shfl_xor(a1, 16));
    const int e0 = query_block_exp(a0), e1 = query_block_exp(a1);
    // block g's largest value: first halves of lane groups 2g, 2g+1 (g < 2)
    // or second halves of groups 2(g-2), 2(g-2)+1
    const int src = (threadIdx.x & 15) + 32 * (g & 1);
    const float b0 = __shfl(a0, src), b1 = __shfl(a1, src);
    const int es = query_block_exp(g < 2 ? b0 : b1);
    sc[0] = es + 127;
    sc[1] = es - 4 + 127;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        const int e = d < 4 ? e0 : e1;
        float xs[4], lo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) xs[k] = ldexpf(x[4 * d + k], -e);
        int hw = __builtin_amdgcn_cvt_pk_fp8_f32(xs[0], xs[1], 0, false);
        hw = __builtin_amdgcn_cvt_pk_fp8_f32(xs[2], xs[3], hw, true);
        lo[0] = (xs[0] - __builtin_amdgcn_cvt_f32_fp8(hw, 0)) * 16.f;
        lo[1] = (xs[1] - __builtin_amdgcn_cvt_f32_fp8(hw, 1)) * 16.f;
        lo[2] = (xs[2] - __builtin_amdgcn_cvt_f32_fp8(hw, 2)) * 16.f;
        lo[3] = (xs[3] - __builtin_amdgcn_cvt_f32_fp8(hw, 3)) * 16.f;
        int lw = __builtin_amdgcn_cvt_pk_fp8_f32(lo[0], lo[1], 0, false);
        lw = __builtin_amdgcn_cvt_pk_fp8_f32(lo[2], lo[3], lw, true);
        p[0][d] = hw;
        p[1][d] = lw;
    }
}

// Workgroup barrier of the LDS ring.  This wave's LDS reads are complete
// (lgkmcnt 0) so the stage they read may be refilled; the vector-memory
// counter is left alone, so the tiles still in flight stay in flight.  The
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
    asm volatile("s_barrier" ::: "memory");
}

template <int D, int KVDT, bool MAP, bool NT, int NRG>
__global__ __launch_bounds__(NRG * kWave, 2) void attn_shared_kernel(
    const void *__restrict__ ck, const void *__restrict__ cv, const float *__restrict__ ksc,
    const float *__restrict__ vsc, const uint16_t *__restrict__ q, int Hq, int Hkv, int L, int b,
    int G, const int32_t *__restrict__ key_idx, int n_keys, float scale_log2, int row_chunks,
    int splits, int tiles_per_split, int64_t rows_total, const float *__restrict__ memo_o,
    const float *__restrict__ memo_lse, void *__restrict__ out, int out_dtype,
    float *__restrict__ lse, float *__restrict__ part_o, float *__restrict__ part_ml) {
    constexpr int RT = 2;                  // 16-row MFMA tiles per wave: 32 rows
    constexpr int NC = D / 32;             // k-chunks of the first product
    constexpr int NDT = D / 16;            // dim tiles of the second product
    constexpr bool E4 = KVDT == DLLM_E4M3;
    // e4m3 V tiles are widened to bf16 once per workgroup, into one of two
    // converted stages, and e4m3 K tiles are read where they landed; bf16
    // tiles are read where they landed
    constexpr bool CONV = E4;
    constexpr int NS = E4 ? kNS8 : kNS;    // ring stages
    constexpr int ESZ = E4 ? 1 : 2;
    constexpr int ROWB = D * ESZ;          // bytes of one cached row
    constexpr int CPR = ROWB / 16;         // 16-byte chunks per cached row
    constexpr int RPI = 64 / CPR;          // rows per 1 KB direct-to-LDS load
    constexpr int TB = 32 * ROWB;          // bytes of one K (or V) tile as cached
    constexpr int NK = TB / 1024;          // loads per K tile (as many for V)
    static_assert(NK % NRG == 0, "every wave issues the same loads");
    static_assert(!E4 || D == 128, "e4m3 rows are one 128-element scale group");
    constexpr int LW = 2 * NK / NRG + (E4 ? 1 : 0);    // loads each wave issues per tile
    constexpr int STAGE = 2 * TB + (E4 ? 256 : 0);
    constexpr int BROW = D * 2;            // bytes of one bf16 row
    constexpr int CTB = 32 * BROW;         // one bf16 K (or V) tile
    // swizzles of the bf16 operand tiles, and of the ring stages as loaded
    // (the operand tiles themselves for bf16; e4m3 K read as the fp8 operand,
    // e4m3 V read linearly for widening)
    auto kswz_b = [](int r) { return BROW == 256 ? kswz16(r) : kswz(r); };
    auto vswz_b = [](int r) { return BROW == 256 ? vswz16(r) : vswz_bf16(r); };
    auto kswz_r = [&](int r) { return E4 ? kswz8(r) : kswz_b(r); };
    auto vswz_r = [&](int r) { return CONV ? vswz_e4m3(r) : vswz_b(r); };
    constexpr int CSTAGE = CONV ? CTB + 3 * 128 : 0;   // V + per-key kfac, bias, vfac
    constexpr int TAB = MAP ? kTableKeys * 4 : 0;
    // the two converted stages first, so that both lie within the 64 KB
    // immediate offset of an LDS read from one base register: with the tile
    // loop unrolled by two, every operand read of a converted stage is a
    // loop-invariant register plus a constant
    constexpr int OFF_RING = 2 * CSTAGE;
    constexpr int OFF_TAB = OFF_RING + NS * STAGE;
    constexpr int SMEM = OFF_TAB + TAB;
    static_assert(TB % 1024 == 0 && CPR <= 16, "tile layout");
    static_assert(SMEM <= kLdsBytes, "LDS of one workgroup");
    static_assert((NS - 2) * LW < 64, "vmcnt range");

    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
    const int l16 = lane & 15;
    const int g = lane >> 4;

    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int split = lid % splits;
    int rest = lid / splits;
    const int rc = rest % row_chunks;
    rest /= row_chunks;
    const int kvh = rest % Hkv;
    const int bi = rest / Hkv;
    const int M = G * b;                   // rows of this (sequence, KV head)
    const int row0 = (rc * NRG + wave) * 32;

    const int64_t kv_base = ((int64_t)bi * Hkv + kvh) * L;
    const int n_tiles = (n_keys + 31) / 32;
    const int t_begin = split * tiles_per_split;
    const int nt = max(0, min(n_tiles, t_begin + tiles_per_split) - t_begin);

    // this split's key indices (with a map; nt * 32 <= kTableKeys), then the
    // index of tile-local key kappa is one LDS read, or arithmetic without one
    int *tab = reinterpret_cast<int *>(smem + OFF_TAB);
    if (MAP) {
        const int32_t *kmap = key_idx + (int64_t)bi * n_keys;
        for (int j = threadIdx.x; j < nt * 32; j += NRG * kWave)
            tab[j] = key_at(kmap, n_keys, L, t_begin * 32 + j);
        __syncthreads();
    }
    auto key_of = [&](int kt, int kappa) -> int {
        if (MAP) return tab[(kt - t_begin) * 32 + kappa];
        return kt * 32 + kappa < n_keys ? kt * 32 + kappa : -1;
    };

    // this wave's queries (loaded after the first tiles): bf16 rows in the
    // bf16 product's layout, or (e4m3) their two e4m3 parts and scales
    uint4 qreg[RT][NC];
    i32x8_t q8[RT][2];
    int qsc[RT][2];

    // ---- loads of tile kt into ring stage `slot`: every wave issues NK/NRG
    // of the K tile's 1 KB loads, as many of the V tile's, and (e4m3) the
    // scales of 64/NRG lanes, so every wave has LW loads per tile in flight.
    // The rows' key indices are looked up first (keys_of) and the loads
    // issued later (issue), so a key-table read is not waited for on its own.
    struct TileKeys {
        int k[NK / NRG], v[NK / NRG], s;
    };
    auto keys_of = [&](int kt, TileKeys &tk) {
#pragma unroll
        for (int u = 0; u < NK / NRG; ++u) {
            const int j = wave * (NK / NRG) + u;
            tk.k[u] = key_of(kt, (j * 64 + lane) / CPR);
            tk.v[u] = key_of(kt, RPI * j + lane / CPR);
        }
        tk.s = E4 ? key_of(kt, lane & 31) : 0;
    };
    // wave-uniform bases of this (sequence, KV head)'s rows; a lane's load is
    // one 32-bit byte offset from them (the rows of one (sequence, KV head)
    // span less than 4 GiB)
    const unsigned char *kbase = static_cast<const unsigned char *>(ck) + kv_base * ROWB;
    const unsigned char *vbase = static_cast<const unsigned char *>(cv) + kv_base * ROWB;
    const uint32_t smem_lds = lds_addr(smem);
    auto issue = [&](const TileKeys &tk, int slot) {
        const uint32_t st = smem_lds + (uint32_t)(OFF_RING + slot * STAGE);
#pragma unroll
        for (int u = 0; u < NK / NRG; ++u) {
            // chunk position p of the tile: row p / CPR, stored slot p % CPR
            // holds the row's chunk (p % CPR) ^ kswz(row)
            const int j = wave * (NK / NRG) + u;
            const int p = j * 64 + lane;
            const int r = p / CPR, sl = p % CPR;
            const int kk = tk.k[u];
            const uint32_t off = (uint32_t)(kk < 0 ? 0 : kk) * ROWB + (uint32_t)(sl ^ kswz_r(r)) * 16;
            lds_dma16<NT>(kbase, off, st + j * 1024);
        }
#pragma unroll
        for (int u = 0; u < NK / NRG; ++u) {
            // V row rho, stored slot lane % CPR holds chunk (lane % CPR) ^ vswz(rho)
            const int jv = wave * (NK / NRG) + u;
            const int rho = RPI * jv + lane / CPR;
            const int chunk = (lane % CPR) ^ vswz_r(rho);
            const int kk = tk.v[u];
            const uint32_t off = (uint32_t)(kk < 0 ? 0 : kk) * ROWB + (uint32_t)chunk * 16;
            lds_dma16<NT>(vbase, off, st + TB + jv * 1024);
        }
        if (E4) {
            // lanes 0..31: K scales of keys 0..31; lanes 32..63: V scales;
            // this wave writes lanes [64 w / NRG, 64 (w + 1) / NRG), all of
            // one kind
            const int lo = wave * (64 / NRG);
            if (lane >= lo && lane < lo + 64 / NRG) {
                const int kk = tk.s;
                const float *sbase = (lo < 32 ? ksc : vsc) + kv_base;
                lds_dma4(sbase, (uint32_t)(kk < 0 ? 0 : kk) * 4, st + 2 * TB);
            }
        }
    };
    auto issue_tile = [&](int kt, int slot) {
        TileKeys tk;
        keys_of(kt, tk);
        issue(tk, slot);
    };

    // ---- e4m3: widen the V rows of tile kt (ring stage `slot`) into
    // converted stage `cslot`, the whole workgroup sharing the work: each
    // 16-code chunk becomes two bf16 chunks in the layout the transposed
    // reads expect (the bf16 vswz).  Threads 0..31 also write the per-key
    // factors: kfac = K scale * scale * log2(e), the mask bias (0, or -inf for
    // a missing key) and vfac = V scale.  Split in a read half and a write
    // half, so the reads can be issued early.
    constexpr int NCH = 32 * CPR;          // 16-code chunks per V tile
    constexpr int PER = CONV ? (NCH + NRG * kWave - 1) / (NRG * kWave) : 1;
    struct ConvIn {
        uint4 w[PER];
        float ks, vs;
        bool present;
    };
    auto convert_read = [&](int kt, int slot, ConvIn &ci_) {
        if constexpr (CONV) {
            const unsigned char *st = smem + OFF_RING + slot * STAGE;
#pragma unroll
            for (int it = 0; it < PER; ++it) {
                const int idx = threadIdx.x + it * NRG * kWave;
                if (PER * NRG * kWave == NCH || idx < NCH)
                    ci_.w[it] = *reinterpret_cast<const uint4 *>(st + TB + idx * 16);
            }
            const int kap = threadIdx.x & 31;
            const float *sc = reinterpret_cast<const float *>(st + 2 * TB);
            ci_.ks = sc[kap];
            ci_.vs = sc[32 + kap];
            ci_.present = key_of(kt, kap) >= 0;
        } else {
            (void)kt; (void)slot; (void)ci_;
        }
    };
    auto convert_write = [&](int cslot, const ConvIn &ci_) {
        if constexpr (CONV) {
            unsigned char *cs = smem + cslot * CSTAGE;
#pragma unroll
            for (int it = 0; it < PER; ++it) {
                const int idx = threadIdx.x + it * NRG * kWave;
                if (PER * NRG * kWave != NCH && idx >= NCH) break;
                const int r = idx / CPR, sl = idx % CPR;
                const int gc = sl ^ vswz_r(r);         // the row's chunk in slot sl
                const int sw = vswz_b(r);
                unsigned char *row = cs + r * BROW;
                const uint4 w = ci_.w[it];
                *reinterpret_cast<uint4 *>(row + ((2 * gc) ^ sw) * 16) = e4m3x8_to_bf16(w.x, w.y);
                *reinterpret_cast<uint4 *>(row + ((2 * gc + 1) ^ sw) * 16) = e4m3x8_to_bf16(w.z, w.w);
            }
            float *fac = reinterpret_cast<float *>(cs + CTB);
            if (threadIdx.x < 32) {
                fac[threadIdx.x] = ci_.ks * scale_log2;
                fac[32 + threadIdx.x] = ci_.present ? 0.f : kNegInf;
                fac[64 + threadIdx.x] = ci_.vs;
            }
        } else {
            (void)cslot; (void)ci_;
        }
    };

    f32x4_t o[NDT][RT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) o[dt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m[RT], l[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) { m[rt] = kMinit; l[rt] = 0.f; }

    // e4m3 K operands of the tile being computed (loaded one step ahead):
    // lane (l16, g) holds dims 32g .. 32g+31 of key 8(l16/4) + 4t + l16%4 of
    // half t, the codes as cached, with the queries' parts on the same dims
    uint4 k8[2][2];
    auto load_k8 = [&](const unsigned char *kb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int kappa = 8 * (l16 >> 2) + 4 * t + (l16 & 3);
            const unsigned char *krow = kb + kappa * ROWB;
#pragma unroll
            for (int c = 0; c < 2; ++c)
                k8[t][c] = *reinterpret_cast<const uint4 *>(krow + ((2 * g + c) ^ kswz8(kappa)) * 16);
        }
    };

    // ---- one tile: kb / vb are its bf16 K and V rows (chunk-swizzled; e4m3:
    // K in k8, V widened), fac its per-key factors and tile_full whether all
    // its keys are present (converted tiles only)
    auto compute = [&](int kt, const unsigned char *kb, const unsigned char *vb, const float *fac,
                       bool tile_full, auto &&side) {
        // factors of the keys 8g .. 8g+7 this lane holds in S^T
        float kfac[8], kbias[8], vfac[8];
        bool full = true;
        uint32_t present = ~0u;
        if (CONV) {
            full = tile_full;
            const float4 *f4 = reinterpret_cast<const float4 *>(fac);
            const float4 a0 = f4[2 * g], a1 = f4[2 * g + 1];
            const float4 c0 = f4[16 + 2 * g], c1 = f4[16 + 2 * g + 1];
            kfac[0] = a0.x; kfac[1] = a0.y; kfac[2] = a0.z; kfac[3] = a0.w;
            kfac[4] = a1.x; kfac[5] = a1.y; kfac[6] = a1.z; kfac[7] = a1.w;
            vfac[0] = c0.x; vfac[1] = c0.y; vfac[2] = c0.z; vfac[3] = c0.w;
            vfac[4] = c1.x; vfac[5] = c1.y; vfac[6] = c1.z; vfac[7] = c1.w;
            if (!full) {
                // the mask bias of missing keys, read only for tiles that have
                // some (a full tile never reads kbias, so no zeros are kept)
                const float4 b0 = f4[8 + 2 * g], b1 = f4[8 + 2 * g + 1];
                kbias[0] = b0.x; kbias[1] = b0.y; kbias[2] = b0.z; kbias[3] = b0.w;
                kbias[4] = b1.x; kbias[5] = b1.y; kbias[6] = b1.z; kbias[7] = b1.w;
            }
        } else {
            // keys present in the tile (bit kappa; lanes 32..63 repeat 0..31)
            present = (uint32_t)__ballot(key_of(kt, lane & 31) >= 0);
            full = present == 0xffffffffu;
        }
        // K operands of both 16-key halves: slot l16 of half t is key
        // 8(l16/4) + 4t + l16%4, so S^T leaves keys 8g .. 8g+7 of one row in a lane
        f32x4_t sacc[RT][2];
        if constexpr (E4) {
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const i32x8_t a = {(int)k8[t][0].x, (int)k8[t][0].y, (int)k8[t][0].z, (int)k8[t][0].w,
                                   (int)k8[t][1].x, (int)k8[t][1].y, (int)k8[t][1].z, (int)k8[t][1].w};
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    sacc[rt][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        a, q8[rt][0], z, 0, 0, 0, kE8M0One, 0, qsc[rt][0]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    sacc[rt][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        a, q8[rt][1], sacc[rt][t], 0, 0, 0, kE8M0One, 0, qsc[rt][1]);
            }
        } else {
            uint4 ka[2][NC];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int kappa = 8 * (l16 >> 2) + 4 * t + (l16 & 3);
                const unsigned char *krow = kb + kappa * BROW;
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    ka[t][c] = *reinterpret_cast<const uint4 *>(krow + ((c * 4 + g) ^ kswz_b(kappa)) * 16);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) sacc[rt][0] = sacc[rt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        sacc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, ka[t][c]), __builtin_bit_cast(bf16x8_t, qreg[rt][c]),
                            sacc[rt][t], 0, 0, 0);
        }

        side();      // independent work (the next tile's widening) under the products

        // V^T operands, read transposed from the row-major bf16 tile once the
        // score products are issued (they take the K operands' registers), in
        // flight during the softmax: local lane j reads row 8g + 4h + j/4,
        // dims dt*16 + 4(j%4) .. +3; lane i then holds keys 8g+4h .. +3 at
        // dim dt*16 + i
        uint4 vop[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int r0 = 8 * g + (l16 >> 2), r1 = r0 + 4;
            const int cl = 2 * dt + ((l16 & 3) >> 1);
            const uint2 lo = lds_tr16(vb + r0 * BROW + (cl ^ vswz_b(r0)) * 16 + 8 * (l16 & 1));
            const uint2 hi = lds_tr16(vb + r1 * BROW + (cl ^ vswz_b(r1)) * 16 + 8 * (l16 & 1));
            vop[dt] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }

        // scores in base 2 relative to the running max, y = x - m, and their
        // row maxima for both row tiles first, so the rare rescale is one
        // branch per tile and the rest of the tile is one straight block for
        // the scheduler.  The subtraction is folded into the scaling FMA, and
        // a tile with missing keys sets theirs to -inf afterwards.
        float y[RT][8], ymx[RT];
        bool lgrow = false;
        auto scores = [&](int rt, float *xo) {
            const f32x4_t s0 = sacc[rt][0], s1 = sacc[rt][1];
            const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
            if (CONV) {
                // the key biases again from the tile's factors (written for
                // every tile, 0 for a present key), so that a full tile keeps
                // none in registers for this rare path
                const float4 *f4 = reinterpret_cast<const float4 *>(fac);
                const float4 b0 = f4[8 + 2 * g], b1 = f4[8 + 2 * g + 1];
                const float kb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) xo[e] = fmaf(sv[e], kfac[e], kb[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) xo[e] = sv[e] * scale_log2;
                if (!full) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (!((present >> (8 * g + e)) & 1u)) xo[e] = kNegInf;
                }
            }
        };
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const f32x4_t s0 = sacc[rt][0], s1 = sacc[rt][1];
            const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
            for (int e = 0; e < 8; ++e) y[rt][e] = fmaf(sv[e], CONV ? kfac[e] : scale_log2, -m[rt]);
        }
        if (!full) {
            // missing keys (wave-uniform test): -inf
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool miss = CONV ? kbias[e] != 0.f : !((present >> (8 * g + e)) & 1u);
                    if (miss) y[rt][e] = kNegInf;
                }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float v = vmax(vmax(y[rt][0], y[rt][1]), y[rt][2]);
            v = vmax(vmax(v, y[rt][3]), y[rt][4]);
            v = vmax(vmax(v, y[rt][5]), y[rt][6]);
            ymx[rt] = vmax(v, y[rt][7]);       // this lane's 8 keys of the row
            lgrow = lgrow || ymx[rt] > kLazy;
        }
        // the reference max moves only when a tile's max exceeds it by more
        // than kLazy, so the O rescale is rare.  A row's max exceeds it only
        // if one of its four lanes' maxima does, so the row maxima are formed
        // only when some lane of the wave sees such a key.  The rescale
        // recomputes the scores from the products: y is relative to the old
        // max, which is still the finite start value before a row's first key.
        if (__ballot(lgrow)) {
            bool grow[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) grow[rt] = group4_max(ymx[rt]) > kLazy;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if (grow[rt]) {
                    float x[8];
                    scores(rt, x);
                    float v = x[0];
#pragma unroll
                    for (int e = 1; e < 8; ++e) v = vmax(v, x[e]);
                    const float mx = group4_max(v);
                    const float corr = __builtin_amdgcn_exp2f(m[rt] - mx);
                    l[rt] *= corr;
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) o[dt][rt] *= corr;
                    m[rt] = mx;
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[rt][e] = x[e] - mx;
                }
            }
        }
        Frag pf[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float p[8], ps = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = __builtin_amdgcn_exp2f(y[rt][e]);
                ps += p[e];
            }
            l[rt] += ps;
            if (CONV) {
#pragma unroll
                for (int e = 0; e < 8; ++e) p[e] *= vfac[e];
            }
            pf[rt].u = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                  pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
        }

        // ---- O^T += V^T P^T.  The wave raises its issue priority over its
        // products, so that the other wave of the SIMD, in its vector phase,
        // fills the matrix cores' gaps instead of delaying the products
        // (about 1 % on the long-context step, same box, interleaved)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vop[dt]),
                                                                    pf[rt].v, o[dt][rt], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
    };
    auto ring = [&](int slot) { return smem + OFF_RING + slot * STAGE; };
    auto cstage = [&](int cslot) { return smem + cslot * CSTAGE; };

    // ---- the pipeline: NS - 1 tiles in flight.  bf16: per tile, wait for
    // this wave's loads of it, one barrier (the tile is complete, every wave
    // is done with the stage the next load refills), refill, compute from the
    // ring.  e4m3: per tile, wait for the next tile's loads, one barrier,
    // refill the stage the previous tile used, read the next tile's V rows
    // for widening, compute this one (K from the ring, V from its converted
    // stage) and write the next one's widened V under the score products.
#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
        if (i < nt) issue_tile(t_begin + i, i);

    uint4 qraw[RT][4];                     // e4m3: dims 32g .. 32g+31 of each row
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = row0 + rt * 16 + l16;
        const int gq = r / b, i = r - gq * b;
        const uint16_t *qrow = q + (((int64_t)bi * Hq + kvh * G + gq) * b + i) * D;
        if constexpr (E4) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                qraw[rt][c] = make_uint4(0, 0, 0, 0);
                if (r < M) qraw[rt][c] = *reinterpret_cast<const uint4 *>(qrow + 32 * g + 8 * c);
            }
        } else {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                qreg[rt][c] = make_uint4(0, 0, 0, 0);
                if (r < M) qreg[rt][c] = *reinterpret_cast<const uint4 *>(qrow + chunk_dim<DLLM_BF16>(c, g));
            }
        }
    }
    // A memoized state (FACache) starts the rows of split 0: O~ = memo_o,
    // m = memo_lse in base 2 and l = 1, the 1 counted in lane group 0 only
    // (the row sum adds the four groups); an empty memo (-inf) stays empty.
    // Its loads go straight into the accumulators, beside the queries'.
    const bool memo = memo_lse != nullptr && split == 0;
    float mlse[RT];
    if (memo) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int r = row0 + rt * 16 + l16;
            mlse[rt] = kNegInf;
            if (r < M) {
                const int gq = r / b, i = r - gq * b;
                const int64_t orow = ((int64_t)bi * Hq + kvh * G + gq) * b + i;
                mlse[rt] = memo_lse[orow];
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const float4 v = *reinterpret_cast<const float4 *>(memo_o + orow * D + dt * 16 + 4 * g);
                    o[dt][rt] = f32x4_t{v.x, v.y, v.z, v.w};
                }
            }
        }
    }
    // The queries, the memo and the first tiles land together.  Waiting for
    // every load here also tells the compiler the query registers are ready,
    // so it adds no wait of its own inside the loop.
    vm_wait<0>();
    if (memo) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (mlse[rt] == kNegInf) {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) o[dt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            } else {
                m[rt] = mlse[rt] * kLog2e;
                l[rt] = g == 0 ? 1.f : 0.f;
            }
        }
    }
    if constexpr (E4) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) split_query(qraw[rt], g, q8[rt], qsc[rt]);
    }
    if (CONV && nt > 0) {
        ring_barrier();
        ConvIn c0;
        convert_read(t_begin, 0, c0);
        convert_write(0, c0);
    }

    // Which tiles of the split have all 32 keys: arithmetic without a map;
    // with one (at most 64 tiles), lane j checks tile j's table entries once.
    uint64_t fullmask = 0;
    if (CONV && MAP) {
        bool f = true;
        if (lane < nt) {
            const int4 *t4 = reinterpret_cast<const int4 *>(tab + lane * 32);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int4 v = t4[j];
                f = f && v.x >= 0 && v.y >= 0 && v.z >= 0 && v.w >= 0;
            }
        }
        fullmask = __ballot(f);
    }
    auto tile_full = [&](int i) -> bool {
        if (MAP) return (fullmask >> i) & 1ull;
        return (t_begin + i + 1) * 32 <= n_keys;
    };

    // one e4m3 step (slot = i % NS): wait for the next tile's loads, one
    // barrier (every wave is done with the previous tile's ring stage and
    // with the converted stage the next tile is widened into), read the next
    // tile's V rows, compute this tile (its K operands and the refill's key
    // indices were read during the previous step) and issue the refill and
    // write the widened rows under its score products; then read the next
    // tile's K operands (its loads are complete and visible since this
    // step's barrier) and the next refill's key indices (the table does not
    // change), so neither is waited for after the next barrier.
    // The converted stage of tile i is i % 2, a compile-time constant `par`.
    TileKeys tk;
    auto conv_step = [&](int i, auto par, auto wait) {
        constexpr int P = decltype(par)::value;
        const int slot = i % NS;
        __builtin_amdgcn_sched_barrier(0);
        wait();
        ring_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const bool refill = i + NS - 1 < nt;
        const bool next = i + 1 < nt;
        const int nslot = slot + 1 == NS ? 0 : slot + 1;
        ConvIn cn;
        if (next) convert_read(t_begin + i + 1, nslot, cn);
        const unsigned char *cs = cstage(P);
        compute(t_begin + i, nullptr, cs, reinterpret_cast<const float *>(cs + CTB), tile_full(i), [&] {
            if (refill) issue(tk, slot == 0 ? NS - 1 : slot - 1);
            if (next) convert_write(P ^ 1, cn);
        });
        if (next) load_k8(ring(nslot));
        if (i + NS < nt) keys_of(t_begin + i + NS, tk);
    };
    // tiles issued after the next one
    auto conv_wait = [&](int i) {
        return [=] { vm_wait_upto<(NS - 3) * LW>(max(0, min(NS - 3, nt - 2 - i)) * LW); };
    };
    int i = 0;
    if (CONV) {
        if (nt > 0) load_k8(ring(0));
        if (NS - 1 < nt) keys_of(t_begin + NS - 1, tk);
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        for (; i + 1 < nt; i += 2) {
            conv_step(i, P0{}, conv_wait(i));
            conv_step(i + 1, P1{}, conv_wait(i + 1));
        }
        if (i < nt) conv_step(i, P0{}, conv_wait(i));
    }
    for (; !CONV && i < nt; ++i) {
        {
            // tiles issued after this one
            const int ahead = min(NS - 2, nt - 1 - i);
            __builtin_amdgcn_sched_barrier(0);
            vm_wait_upto<(NS - 2) * LW>(ahead * LW);
            ring_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (i + NS - 1 < nt) issue_tile(t_begin + i + NS - 1, (i + NS - 1) % NS);
            const unsigned char *st = ring(i % NS);
            compute(t_begin + i, st, st + TB, nullptr, true, [] {});
        }
    }

    // ---- row sums over the 4 lane groups, then this wave's rows out.  The
    // rows' offsets are formed again here from an opaque copy of the lane
    // index, so the compiler does not keep the prologue's across the loop.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) l[rt] = group4_sum(l[rt]);
    int l16e = l16;
    asm volatile("" : "+v"(l16e));
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = row0 + rt * 16 + l16e;
        if (r >= M) continue;
        const int gq = r / b, i = r - gq * b;
        const int64_t orow = ((int64_t)bi * Hq + kvh * G + gq) * b + i;
        if (splits == 1) {
            const float inv = l[rt] > 0.f ? 1.0f / l[rt] : 0.f;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const f32x4_t v = o[dt][rt] * inv;
                const int64_t off = orow * D + dt * 16 + 4 * g;
                if (out_dtype == DLLM_F32) {
                    *reinterpret_cast<float4 *>(static_cast<float *>(out) + off) =
                        make_float4(v[0], v[1], v[2], v[3]);
                } else {
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + off) =
                        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                }
            }
            if (lse && g == 0) lse[orow] = l[rt] > 0.f ? m[rt] * kLn2 + logf(l[rt]) : kNegInf;
        } else {
            const int64_t prow = (int64_t)split * rows_total + orow;
#pragma unroll
            // the output's precision: bf16 partials for a bf16 output, else fp32
            for (int dt = 0; dt < NDT; ++dt) {
                const f32x4_t v = o[dt][rt];
                if (out_dtype == DLLM_F32)
                    *reinterpret_cast<float4 *>(part_o + prow * D + dt * 16 + 4 * g) =
                        make_float4(v[0], v[1], v[2], v[3]);
                else
                    *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(part_o) + prow * D + dt * 16 + 4 * g) =
                        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
            if (g == 0) {
                part_ml[prow * 2 + 0] = m[rt];
                part_ml[prow * 2 + 1] = l[rt];
            }
        }
    }
}

template <int D, int KVDT, bool MAP, bool NT, int NRG>
int launch_shared(const dllm_kv_cache &c, const AttnPlan &p, const void *q, int Hq, int b,
                  const int32_t *key_idx, int n_keys, float scale, const AttnMemo &memo, void *out,
                  int out_dtype, float *lse, void *ws, hipStream_t s) {
    const int G = Hq / c.n_kv_heads;
    const int64_t rows_total = (int64_t)c.B * Hq * b;
    const int64_t blocks = (int64_t)c.B * c.n_kv_heads * p.row_groups * p.splits;
    if (blocks > INT_MAX) return DLLM_ERANGE;
    if (MAP && p.tiles_per_wave * 32 > kTableKeys) return DLLM_ESHAPE;   // the key table holds them
    float *part_o = nullptr, *part_ml = nullptr;
    if (p.splits > 1) {
        part_o = static_cast<float *>(ws);
        part_ml = part_o + (int64_t)p.splits * rows_total * D;
    }
    attn_shared_kernel<D, KVDT, MAP, NT, NRG><<<dim3((unsigned)blocks), dim3(NRG * kWave), 0, s>>>(
        c.k, c.v, c.k_scale, c.v_scale, static_cast<const uint16_t *>(q), Hq, c.n_kv_heads, c.L,
        b, G, key_idx, n_keys, scale * kLog2e, p.row_groups, p.splits, p.tiles_per_wave, rows_total,
        memo.o, memo.lse, out, out_dtype, lse, part_o, part_ml);
    int rc = launch_status();
    if (rc != DLLM_OK || p.splits == 1) return rc;
    return launch_attn_merge(part_o, part_ml, rows_total, D, p.splits, out, out_dtype, lse, s);
}

}  // namespace

void plan_shared(const dllm_kv_cache &c, int Hq, int b, int row_groups32, int n_keys, bool has_map,
                 AttnPlan *p) {
    // waves per workgroup: one per 32-row group of the KV head, 2 or 4.  Two
    // 4-wave workgroups per CU (a KV head's row chunks on one XCD) measured
    // ahead of one 8-wave workgroup: the two run out of step, so one's
    // softmax overlaps the other's products (74 against 78 us at longctx).
    const int nrg = row_groups32 >= 3 ? 4 : 2;
    p->path = 2;
    p->row_tiles = 2;
    p->waves = nrg;
    p->row_groups = (row_groups32 + nrg - 1) / nrg;      // row chunks of nrg groups
    const int64_t units = (int64_t)c.B * c.n_kv_heads * p->row_groups;
    const int n_tiles = (n_keys + 31) / 32;
    // two waves per SIMD: 2048 / nrg workgroups fill the chip; splits keep
    // at least 4 tiles each and, with a map, fit the LDS key table
    const int64_t want = 2048 / nrg;
    int64_t splits = std::max<int64_t>(1, (want + units - 1) / units);
    splits = std::min<int64_t>(splits, std::max(1, n_tiles / 4));
    if (has_map) splits = std::max<int64_t>(splits, ((int64_t)n_tiles * 32 + kTableKeys - 1) / kTableKeys);
    int tps = (int)((n_tiles + splits - 1) / splits);
    splits = (n_tiles + tps - 1) / tps;                   // no empty split
    p->splits = (int)splits;
    p->tiles_per_wave = tps;                              // tiles per split
    p->ws_bytes = splits > 1 ? (size_t)splits * c.B * Hq * b * (c.d_head + 2) * sizeof(float) : 0;
}

int launch_shared_attention(const dllm_kv_cache &c, const AttnPlan &p, const void *q, int Hq, int b,
                            const int32_t *key_idx, int n_keys, float scale, const AttnMemo &memo,
                            void *out, int out_dtype, float *lse, void *ws, hipStream_t s) {
    const bool e4 = c.dtype == DLLM_E4M3;
    const bool map = key_idx != nullptr;
    // stream K/V past the caches when one workgroup reads each tile
    const bool nt = p.row_groups == 1;
    auto go = [&](auto dd, auto kv, auto mp) -> int {
        constexpr int DD = decltype(dd)::value, KV = decltype(kv)::value;
        constexpr bool MP = decltype(mp)::value;
        auto pick = [&](auto ntv) -> int {
            constexpr bool NTV = decltype(ntv)::value;
            if (p.waves == 2)
                return launch_shared<DD, KV, MP, NTV, 2>(c, p, q, Hq, b, key_idx, n_keys, scale, memo,
                                                         out, out_dtype, lse, ws, s);
            if (p.waves == 4)
                return launch_shared<DD, KV, MP, NTV, 4>(c, p, q, Hq, b, key_idx, n_keys, scale, memo,
                                                         out, out_dtype, lse, ws, s);
            return DLLM_ESHAPE;
        };
        return nt ? pick(std::true_type{}) : pick(std::false_type{});
    };
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    using KB = std::integral_constant<int, DLLM_BF16>;
    using KE = std::integral_constant<int, DLLM_E4M3>;
    if (c.d_head == 128) {
        if (e4) return map ? go(I128{}, KE{}, std::true_type{}) : go(I128{}, KE{}, std::false_type{});
        return map ? go(I128{}, KB{}, std::true_type{}) : go(I128{}, KB{}, std::false_type{});
    }
    if (e4 || c.d_head != 64) return DLLM_ESHAPE;
    return map ? go(I64{}, KB{}, std::true_type{}) : go(I64{}, KB{}, std::false_type{});
}

}  // namespace dllm
