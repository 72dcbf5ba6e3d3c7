// Block attention for grouped queries: the same product as the per-wave MFMA
// path, out = softmax(q K^T * scale) V over the selected keys with no causal
// mask [LaCache explainer, problem statement and Methodology 1; attention-
// sinks page, 2.1 and 2.3], laid out for shapes where several 32-row groups
// of queries read each KV head (G query heads times b block queries > 32).
//
// A workgroup of NRG (2 or 4) waves owns one (sequence, KV head, row chunk,
// key split); wave w owns 32 rows of the chunk, and every wave walks the same
// key tiles.  Each 32-key tile's K rows, V rows and (e4m3) per-key scales are
// loaded once per workgroup, straight from HBM into a ring of kNS LDS stages
// (global_load_lds, no registers), the loads of one tile spread over the
// waves.  Per tile a wave waits for its own loads, then one workgroup
// barrier makes the whole tile visible and frees the stage the previous tile
// used, which the next tile's loads then fill.  Each wave then reads
//     A = K rows (16-byte chunks XOR-swizzled so that a read phase hits
//         distinct banks), widened e4m3 -> bf16 exactly,
//     B = its queries, held in registers for the whole walk,
// for S^T = K Q^T on v_mfma_f32_16x16x32_bf16, runs the base-2 online
// softmax with the lazy max, and accumulates O^T += V^T P^T with V^T read
// transposed from the row-major V tile.  Compared with one wave per key run,
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

constexpr int kNS = 4;                 // LDS ring stages: three tiles in flight while one is used
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
    // e4m3 tiles are widened to bf16 once per workgroup, into one of two
    // converted stages; bf16 tiles are read where they landed
    constexpr bool CONV = E4;
    constexpr int ESZ = E4 ? 1 : 2;
    constexpr int ROWB = D * ESZ;          // bytes of one cached row
    constexpr int CPR = ROWB / 16;         // 16-byte chunks per cached row
    constexpr int RPI = 64 / CPR;          // rows per 1 KB direct-to-LDS load
    constexpr int TB = 32 * ROWB;          // bytes of one K (or V) tile as cached
    constexpr int NK = TB / 1024;          // loads per K tile (as many for V)
    static_assert(NK % NRG == 0, "every wave issues the same loads");
    constexpr int LW = 2 * NK / NRG + (E4 ? 1 : 0);    // loads each wave issues per tile
    constexpr int STAGE = 2 * TB + (E4 ? 256 : 0);
    constexpr int BROW = D * 2;            // bytes of one bf16 row
    constexpr int CTB = 32 * BROW;         // one bf16 K (or V) tile
    // swizzles of the bf16 operand tiles, and of the ring stages as loaded
    // (the operand tiles themselves for bf16; read linearly for widening)
    auto kswz_b = [](int r) { return BROW == 256 ? kswz16(r) : kswz(r); };
    auto vswz_b = [](int r) { return BROW == 256 ? vswz16(r) : vswz_bf16(r); };
    auto kswz_r = [&](int r) { return CONV ? kswz(r) : kswz_b(r); };
    auto vswz_r = [&](int r) { return CONV ? vswz_e4m3(r) : vswz_b(r); };
    constexpr int CSTAGE = CONV ? 2 * CTB + 3 * 128 + 16 : 0;   // + per-key kfac, bias, vfac; full flag
    constexpr int TAB = MAP ? kTableKeys * 4 : 0;
    // the two converted stages first, so that both lie within the 64 KB
    // immediate offset of an LDS read from one base register: with the tile
    // loop unrolled by two, every operand read of a converted stage is a
    // loop-invariant register plus a constant
    constexpr int OFF_RING = 2 * CSTAGE;
    constexpr int OFF_TAB = OFF_RING + kNS * STAGE;
    constexpr int SMEM = OFF_TAB + TAB;
    static_assert(TB % 1024 == 0 && CPR <= 16, "tile layout");
    static_assert(SMEM <= kLdsBytes, "LDS of one workgroup");
    static_assert((kNS - 2) * LW < 64, "vmcnt range");

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

    uint4 qreg[RT][NC];                    // this wave's queries (loaded after the first tiles)

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
    auto issue = [&](const TileKeys &tk, int slot) {
        unsigned char *st = smem + OFF_RING + slot * STAGE;
#pragma unroll
        for (int u = 0; u < NK / NRG; ++u) {
            // chunk position p of the tile: row p / CPR, stored slot p % CPR
            // holds the row's chunk (p % CPR) ^ kswz(row)
            const int j = wave * (NK / NRG) + u;
            const int p = j * 64 + lane;
            const int r = p / CPR, sl = p % CPR;
            const int kk = tk.k[u];
            const unsigned char *src = static_cast<const unsigned char *>(ck) +
                                       (kv_base + (kk < 0 ? 0 : kk)) * ROWB + (sl ^ kswz_r(r)) * 16;
            lds_dma16<NT>(src, st + j * 1024);
        }
#pragma unroll
        for (int u = 0; u < NK / NRG; ++u) {
            // V row rho, stored slot lane % CPR holds chunk (lane % CPR) ^ vswz(rho)
            const int jv = wave * (NK / NRG) + u;
            const int rho = RPI * jv + lane / CPR;
            const int chunk = (lane % CPR) ^ vswz_r(rho);
            const int kk = tk.v[u];
            const unsigned char *src = static_cast<const unsigned char *>(cv) +
                                       (kv_base + (kk < 0 ? 0 : kk)) * ROWB + chunk * 16;
            lds_dma16<NT>(src, st + TB + jv * 1024);
        }
        if (E4) {
            // lanes 0..31: K scales of keys 0..31; lanes 32..63: V scales;
            // this wave writes lanes [64 w / NRG, 64 (w + 1) / NRG)
            const int lo = wave * (64 / NRG);
            if (lane >= lo && lane < lo + 64 / NRG) {
                const int kk = tk.s;
                const float *src = (lane < 32 ? ksc : vsc) + kv_base + (kk < 0 ? 0 : kk);
                lds_dma4(src, st + 2 * TB);
            }
        }
    };
    auto issue_tile = [&](int kt, int slot) {
        TileKeys tk;
        keys_of(kt, tk);
        issue(tk, slot);
    };

    // ---- e4m3: widen tile kt (ring stage `slot`) into converted stage
    // `cslot`, the whole workgroup sharing the work: each 16-code chunk
    // becomes two bf16 chunks in the bf16 layouts the reads expect (K chunks
    // swizzled by kswz, V chunks by the bf16 vswz).  Threads 0..31 also
    // write the per-key factors: kfac = K scale * scale * log2(e), the mask
    // bias (0, or -inf for a missing key) and vfac = V scale, and wave 0
    // whether all 32 keys are present.  Split in a read half and a write
    // half, so the reads can be issued early.
    constexpr int NCH = 32 * CPR;          // 16-code chunks per K (or V) tile
    constexpr int PER = CONV ? (2 * NCH + NRG * kWave - 1) / (NRG * kWave) : 1;
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
                if (PER * NRG * kWave == 2 * NCH || idx < 2 * NCH)
                    ci_.w[it] = *reinterpret_cast<const uint4 *>(st + idx * 16);   // K chunks, then V chunks
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
                if (PER * NRG * kWave != 2 * NCH && idx >= 2 * NCH) break;
                const bool isv = idx >= NCH;
                const int ci = isv ? idx - NCH : idx;
                const int r = ci / CPR, sl = ci % CPR;
                const int gc = sl ^ (isv ? vswz_r(r) : kswz_r(r));   // the row's chunk in slot sl
                const int sw = isv ? vswz_b(r) : kswz_b(r);
                unsigned char *row = cs + (isv ? CTB : 0) + r * BROW;
                const uint4 w = ci_.w[it];
                *reinterpret_cast<uint4 *>(row + ((2 * gc) ^ sw) * 16) = e4m3x8_to_bf16(w.x, w.y);
                *reinterpret_cast<uint4 *>(row + ((2 * gc + 1) ^ sw) * 16) = e4m3x8_to_bf16(w.z, w.w);
            }
            float *fac = reinterpret_cast<float *>(cs + 2 * CTB);
            if (threadIdx.x < 32) {
                fac[threadIdx.x] = ci_.ks * scale_log2;
                fac[32 + threadIdx.x] = ci_.present ? 0.f : kNegInf;
                fac[64 + threadIdx.x] = ci_.vs;
            }
            if (wave == 0) {
                // lanes 32..63 repeat keys 0..31
                const bool all = __ballot(ci_.present) == ~0ull;
                if (lane == 0) reinterpret_cast<int *>(fac)[96] = all ? 1 : 0;
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

    // ---- one tile: kb / vb are its bf16 K and V rows (chunk-swizzled), fac
    // its per-key factors (converted tiles only)
    auto compute = [&](int kt, const unsigned char *kb, const unsigned char *vb, const float *fac,
                       auto &&side) {
        // factors of the keys 8g .. 8g+7 this lane holds in S^T
        float kfac[8], kbias[8], vfac[8];
        bool full = true;
        uint32_t present = ~0u;
        if (CONV) {
            full = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int *>(fac)[96]) != 0;
            const float4 *f4 = reinterpret_cast<const float4 *>(fac);
            const float4 a0 = f4[2 * g], a1 = f4[2 * g + 1];
            const float4 b0 = f4[8 + 2 * g], b1 = f4[8 + 2 * g + 1];
            const float4 c0 = f4[16 + 2 * g], c1 = f4[16 + 2 * g + 1];
            kfac[0] = a0.x; kfac[1] = a0.y; kfac[2] = a0.z; kfac[3] = a0.w;
            kfac[4] = a1.x; kfac[5] = a1.y; kfac[6] = a1.z; kfac[7] = a1.w;
            kbias[0] = b0.x; kbias[1] = b0.y; kbias[2] = b0.z; kbias[3] = b0.w;
            kbias[4] = b1.x; kbias[5] = b1.y; kbias[6] = b1.z; kbias[7] = b1.w;
            vfac[0] = c0.x; vfac[1] = c0.y; vfac[2] = c0.z; vfac[3] = c0.w;
            vfac[4] = c1.x; vfac[5] = c1.y; vfac[6] = c1.z; vfac[7] = c1.w;
        } else {
            // keys present in the tile (bit kappa; lanes 32..63 repeat 0..31)
            present = (uint32_t)__ballot(key_of(kt, lane & 31) >= 0);
            full = present == 0xffffffffu;
        }
        // K operands of both 16-key halves: slot l16 of half t is key
        // 8(l16/4) + 4t + l16%4, so S^T leaves keys 8g .. 8g+7 of one row in a lane
        uint4 ka[2][NC];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int kappa = 8 * (l16 >> 2) + 4 * t + (l16 & 3);
            const unsigned char *krow = kb + kappa * BROW;
#pragma unroll
            for (int c = 0; c < NC; ++c)
                ka[t][c] = *reinterpret_cast<const uint4 *>(krow + ((c * 4 + g) ^ kswz_b(kappa)) * 16);
        }
        f32x4_t sacc[RT][2];
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
        // the scheduler.  A tile with every key present folds the subtraction
        // into the scaling FMA; one with missing keys adds their -inf bias.
        float y[RT][8], ymx[RT];
        auto scores = [&](int rt, float *xo) {
            const f32x4_t s0 = sacc[rt][0], s1 = sacc[rt][1];
            const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
            if (CONV) {
#pragma unroll
                for (int e = 0; e < 8; ++e) xo[e] = fmaf(sv[e], kfac[e], kbias[e]);
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
            if (full) {
                const f32x4_t s0 = sacc[rt][0], s1 = sacc[rt][1];
                const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
                for (int e = 0; e < 8; ++e) y[rt][e] = fmaf(sv[e], CONV ? kfac[e] : scale_log2, -m[rt]);
            } else {
                float x[8];
                scores(rt, x);
#pragma unroll
                for (int e = 0; e < 8; ++e) y[rt][e] = x[e] - m[rt];
            }
            float v = fmaxf(fmaxf(y[rt][0], y[rt][1]), y[rt][2]);
            v = fmaxf(fmaxf(v, y[rt][3]), y[rt][4]);
            v = fmaxf(fmaxf(v, y[rt][5]), y[rt][6]);
            v = fmaxf(v, y[rt][7]);
            ymx[rt] = group4_max(v);
        }
        // the reference max moves only when a tile's max exceeds it by more
        // than kLazy, so the O rescale is rare.  The rescale recomputes the
        // scores from the products: y is relative to the old max, which is
        // still the finite start value before a row's first key.
        bool grow[RT], any = false;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            grow[rt] = ymx[rt] > kLazy;
            any = any || grow[rt];
        }
        if (__ballot(any)) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if (grow[rt]) {
                    float x[8];
                    scores(rt, x);
                    float v = x[0];
#pragma unroll
                    for (int e = 1; e < 8; ++e) v = fmaxf(v, x[e]);
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

        // ---- O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vop[dt]),
                                                                    pf[rt].v, o[dt][rt], 0, 0, 0);
    };
    auto ring = [&](int slot) { return smem + OFF_RING + slot * STAGE; };
    auto cstage = [&](int cslot) { return smem + cslot * CSTAGE; };

    // ---- the pipeline.  bf16: kNS - 1 tiles in flight; per tile, wait for
    // this wave's loads of it, one barrier (the tile is complete, every wave
    // is done with the stage the next load refills), refill, compute.
    // e4m3: kNS tiles in flight; per tile, wait for the next tile's loads,
    // one barrier, refill the stage the (already widened) tile used, widen
    // the next tile, compute this one from its converted stage.
    const int pro = CONV ? kNS : kNS - 1;
#pragma unroll
    for (int i = 0; i < kNS; ++i)
        if (i < pro && i < nt) issue_tile(t_begin + i, i);

#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = row0 + rt * 16 + l16;
        const int gq = r / b, i = r - gq * b;
        const uint16_t *qrow = q + (((int64_t)bi * Hq + kvh * G + gq) * b + i) * D;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            qreg[rt][c] = make_uint4(0, 0, 0, 0);
            if (r < M) qreg[rt][c] = *reinterpret_cast<const uint4 *>(qrow + chunk_dim<DLLM_BF16>(c, g));
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
    if (CONV && nt > 0) {
        ring_barrier();
        ConvIn c0;
        convert_read(t_begin, 0, c0);
        convert_write(0, c0);
    }

    // one e4m3 step: wait for the next tile's loads, one barrier, refill the
    // stage this tile used, read the next tile for widening, compute this
    // one and write the next one back under its first product (slot = i % kNS).
    // The converted stage of tile i is i % 2, a compile-time constant `par`.
    auto conv_step = [&](int i, auto par, auto wait) {
        constexpr int P = decltype(par)::value;
        const int slot = i % kNS;
        __builtin_amdgcn_sched_barrier(0);
        wait();
        ring_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // the refill's key indices and the next tile's raw chunks are read
        // now; the refill is issued and the widening written back under this
        // tile's first product
        const bool refill = i + kNS < nt;
        TileKeys tk;
        if (refill) keys_of(t_begin + i + kNS, tk);
        const bool next = i + 1 < nt;
        ConvIn cn;
        if (next) convert_read(t_begin + i + 1, (slot + 1) % kNS, cn);
        const unsigned char *cs = cstage(P);
        compute(t_begin + i, cs, cs + CTB, reinterpret_cast<const float *>(cs + 2 * CTB), [&] {
            if (refill) issue(tk, slot);
            if (next) convert_write(P ^ 1, cn);
        });
    };
    // tiles issued after the next one
    auto conv_wait = [&](int i) {
        return [=] { vm_wait_upto<(kNS - 2) * LW>(max(0, min(kNS - 2, nt - 2 - i)) * LW); };
    };
    int i = 0;
    if (CONV) {
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
            const int ahead = min(kNS - 2, nt - 1 - i);
            __builtin_amdgcn_sched_barrier(0);
            vm_wait_upto<(kNS - 2) * LW>(ahead * LW);
            ring_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (i + kNS - 1 < nt) issue_tile(t_begin + i + kNS - 1, (i + kNS - 1) % kNS);
            const unsigned char *st = ring(i % kNS);
            compute(t_begin + i, st, st + TB, nullptr, [] {});
        }
    }

    // ---- row sums over the 4 lane groups, then this wave's rows out
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) l[rt] = group4_sum(l[rt]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = row0 + rt * 16 + l16;
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
