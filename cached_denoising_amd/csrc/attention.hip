// Block attention: the queries of the active block attend to the selected
// cached keys with no causal mask, out = softmax(q K^T * scale) V.
// [LaCache explainer, problem statement (bidirectional attention over the
// whole context within a SAR block) and Methodology 1 (FlashAttention's
// online-softmax state m, l, O~); attention-sinks page, 2.1 (the score
// matrix Q K^T / sqrt(d_k), softmax, times V) and 2.3 (fixed key set).]
//
// MFMA path (bf16 queries; bf16 or e4m3 cache; d = 64 or 128):
//   A workgroup of NW = 4 or 8 waves owns one (sequence, KV head, row
//   group, key split); few (sequence, KV head) pairs get more waves per
//   workgroup rather than more key splits, so short contexts need no merge.
//   Each wave keeps the next key tile in flight while it computes one.  The rows are the G query heads sharing the KV head times the
//   block's queries.  Each wave walks its own run of 32-key tiles:
//     S^T (keys x rows) = K . Q^T     on v_mfma_f32_16x16x32_bf16, K straight
//                                      from HBM into the A operand
//     online softmax in base 2        per row, state (m, l) in registers
//     O^T (dims x rows) += V^T . P^T  V rows staged as stored in a per-wave
//                                      LDS tile, read back transposed with
//                                      ds_read_b64_tr_b16 / _tr_b8
//   The two key tiles of a 32-key step are loaded in an interleaved order so
//   that the S^T accumulator of a lane holds 8 consecutive keys of one row:
//   exactly the P^T operand the second product needs, with no shuffles.
//   e4m3 codes widen to bf16 exactly (e4m3 is a subset of bf16) with
//   v_cvt_scalef32_pk_bf16_fp8; the per-key float32 scales multiply the
//   scores (K) and the probabilities (V) in float32.
//   The waves merge through LDS in a fixed binary tree; key splits across
//   workgroups write (m, l, O~) partials merged by a second kernel.
// VALU path (float32 queries and cache, any d <= 256): one wave per query.
#include "attn_common.hpp"

#include <climits>
#include <type_traits>

namespace dllm {
namespace {

using namespace attn;

constexpr int kMapTableTiles = 256;    // 32-key tiles of key indices a workgroup's LDS table holds
constexpr int kStages = 2;             // key tiles per wave in the load pipeline (4 measured no faster)

// LDS of one MFMA workgroup: the staged queries, kStages V tiles per wave
// and, with a key map, the workgroup's table of key indices
constexpr int attn_stage_bytes(int D, int esz, int RT, int NW, bool map) {
    return 16 * RT * (D * 2 + 16) + NW * kStages * 32 * D * esz + (map ? kMapTableTiles * 32 * 4 : 0);
}
// the staging area, or the waves' exchange of O~ at the end if that is larger
constexpr int attn_smem_bytes(int D, int esz, int RT, int NW, bool map) {
    return attn_stage_bytes(D, esz, RT, NW, map) > NW * 16 * RT * (D + 4) * 4
               ? attn_stage_bytes(D, esz, RT, NW, map)
               : NW * 16 * RT * (D + 4) * 4;
}

template <int D, int KVDT, int RT, bool MAP, bool NT, int NW>
__global__ __launch_bounds__(NW * kWave, 2) void attn_mfma_kernel(
    const void *__restrict__ ck, const void *__restrict__ cv, const float *__restrict__ ksc,
    const float *__restrict__ vsc, const uint16_t *__restrict__ q, int Hq, int Hkv, int L, int b,
    int G, const int32_t *__restrict__ key_idx, int n_keys, float scale_log2, int row_groups,
    int splits, int tiles_per_wave, int64_t rows_total, void *__restrict__ out, int out_dtype,
    float *__restrict__ lse, float *__restrict__ part_o, float *__restrict__ part_ml, ScatterIn sc) {
    constexpr int NC = D / 32;           // k-chunks of the first product
    constexpr int NDT = D / 16;          // dim tiles of the second product
    constexpr int ROWS = 16 * RT;        // rows per workgroup
    constexpr int ESZ = KVDT == DLLM_E4M3 ? 1 : 2;
    constexpr int ROWB = D * ESZ;        // bytes of one cached row
    constexpr int CPR = ROWB / 16;       // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;        // rows per wave-wide 16-byte load
    constexpr int VIT = 32 / RPI;        // loads per 32-key V tile
    constexpr int QSTR = D * 2 + 16;     // LDS row stride of Q: 16 rows of one read hit distinct banks
    constexpr int QBYTES = ROWS * QSTR;
    constexpr int VTILE = 32 * ROWB;     // one V tile in LDS
    constexpr int MT = kMapTableTiles / NW;                      // table tiles per wave
    constexpr int TAB = MAP ? kMapTableTiles * 32 * 4 : 0;       // per-wave key index tables
    constexpr int S = kStages;
    constexpr int BST = D + 4;                                   // exchange row stride (floats)
    constexpr int SMEM = attn_smem_bytes(D, ESZ, RT, NW, MAP);
    static_assert(S >= 2 && S <= 4, "pipeline depth");
    static_assert(attn_stage_bytes(D, ESZ, RT, NW, MAP) == QBYTES + NW * S * VTILE + TAB, "LDS layout");
    static_assert(SMEM <= kLdsBytes, "LDS of one workgroup");
    static_assert(SMEM >= NW * ROWS * BST * 4, "the exchange fits");

    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
    __shared__ float sm_ml[NW][ROWS][2];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
    const int l16 = lane & 15;
    const int g = lane >> 4;

    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int rg = lid % row_groups;
    int rest = lid / row_groups;
    const int split = rest % splits;
    rest /= splits;
    const int kvh = rest % Hkv;
    const int bi = rest / Hkv;
    const int M = G * b;                 // rows of this (sequence, KV head)

    const int64_t kv_base = ((int64_t)bi * Hkv + kvh) * L;
    const int32_t *kmap = MAP ? key_idx + (int64_t)bi * n_keys : nullptr;

    // ---- queries: the B operand of S^T = K Q^T.  All waves of the workgroup
    // use the same rows, so they are staged once in LDS; rows past M are
    // zero.  Their loads go out first and are written to LDS after the first
    // key tiles' loads, so the two latencies overlap.
    unsigned char *qs = smem;
    constexpr int QN = ROWS * (D / 8);                   // 16-byte chunks of the staged rows
    constexpr int QIT = (QN + NW * kWave - 1) / (NW * kWave);
    uint4 qv[QIT];
#pragma unroll
    for (int it = 0; it < QIT; ++it) {
        const int idx = threadIdx.x + it * NW * kWave;
        const int r = idx / (D / 8), c8 = idx % (D / 8);
        const int rr = rg * ROWS + r;
        qv[it] = make_uint4(0, 0, 0, 0);
        if (idx < QN && rr < M) {
            const int gq = rr / b, i = rr - gq * b;
            qv[it] = *reinterpret_cast<const uint4 *>(q + (((int64_t)bi * Hq + kvh * G + gq) * b + i) * D + c8 * 8);
        }
    }

    // ---- with the block's fresh rows (bf16 cache, no key map): this
    // workgroup first writes the rows whose positions fall in its own key
    // range into the cache, exactly as the scatter would, and every wave
    // waits for the stores before any tile load, so its loads see them; no
    // other workgroup reads these keys in this call
    if constexpr (KVDT == DLLM_BF16 && !MAP) {
        if (sc.pos) {
            const int key_lo = split * NW * tiles_per_wave * 32;
            const int key_hi = key_lo + NW * tiles_per_wave * 32;
            for (int idx = threadIdx.x; idx < sc.n * CPR; idx += NW * kWave) {
                const int j = idx / CPR, c = idx - (idx / CPR) * CPR;
                const int64_t src = (((int64_t)bi * sc.n + j) * Hkv + kvh) * CPR + c;
                const uint4 kw = sc.k_new[src];
                const uint4 vw = sc.v_new[src];
                const int p = sc.pos[(int64_t)bi * sc.n + j];
                if (p < 0 || p >= L) {
                    if (p != -1 && sc.bad && c == 0 && kvh == 0 && split == 0) atomicAdd(sc.bad, 1);
                    continue;
                }
                if (p < key_lo || p >= key_hi) continue;
                // through the kernel's own cache pointers, so the tile loads
                // below stay ordered after these stores
                const_cast<uint4 *>(static_cast<const uint4 *>(ck))[(kv_base + p) * CPR + c] = kw;
                const_cast<uint4 *>(static_cast<const uint4 *>(cv))[(kv_base + p) * CPR + c] = vw;
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }

    f32x4_t o[NDT][RT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) o[dt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m[RT], l[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) { m[rt] = kMinit; l[rt] = 0.f; }

    unsigned char *vbase = smem + QBYTES + wave * S * VTILE;
    const int n_tiles = (n_keys + 31) / 32;
    const int t_begin = (split * NW + wave) * tiles_per_wave;
    const int t_end = min(n_tiles, t_begin + tiles_per_wave);

    // Software pipeline, S - 1 tiles deep.  While tile t is computed, tiles
    // t+1 .. t+S-1 are in flight: their K rows into the other register sets,
    // their V rows straight from HBM into the wave's other LDS buffers
    // (global_load_lds_dwordx4, no registers).  Direct-to-LDS loads fill 1 KB per instruction in lane
    // order, so the V rows are unpadded and their 16-byte chunks are
    // XOR-swizzled per row instead, which keeps the transposed reads of one
    // 16-lane group on distinct banks.
    constexpr int KR = KVDT == DLLM_E4M3 ? NC / 2 : NC;   // 16-byte K loads per 16-key half
    // vector-memory loads issued for one tile, in order: the map index,
    // K rows, V rows, e4m3 scales
    constexpr int LOADS = 2 * KR + VIT + (KVDT == DLLM_E4M3 ? 2 : 0);
    struct Tile {
        uint4 kr[2][KR];      // K rows as loaded (A operand of S^T = K Q^T)
        int kl;               // key index of tile-local key lane % 32 (-1: none)
        float kfl, vsl;       // its score factor and (e4m3) value scale
    };

    // With a key map, this wave's indices are copied once into its LDS table
    // (tiles_per_wave <= MT); without one, key j of the selection is position
    // j.  Either way the index of tile-local key kappa is cheap.
    int *ktab = reinterpret_cast<int *>(smem + QBYTES + NW * S * VTILE) + wave * MT * 32;
    if (MAP) {
        for (int j = lane; j < (t_end - t_begin) * 32; j += kWave)
            ktab[j] = key_at(kmap, n_keys, L, t_begin * 32 + j);
        __builtin_amdgcn_s_waitcnt(0);           // the table is in LDS before it is read
        __builtin_amdgcn_wave_barrier();
    }
    auto key_of = [&](int kt, int kappa) -> int {
        if (MAP) return ktab[(kt - t_begin) * 32 + kappa];
        return kt * 32 + kappa < n_keys ? kt * 32 + kappa : -1;
    };
    // the key whose rows tile-local key kappa loads: itself, or for a missing
    // key (past the selection, -1 in the map) an in-range one, whose score
    // is masked
    auto key_ld = [&](int kt, int kappa) -> uint32_t {
        if (MAP) return (uint32_t)max(ktab[(kt - t_begin) * 32 + kappa], 0);
        return (uint32_t)min(kt * 32 + kappa, n_keys - 1);
    };
    // 32-bit byte offsets from the wave-uniform bases of this (sequence, KV
    // head)'s rows, which span less than 4 GiB
    const unsigned char *ckrows = static_cast<const unsigned char *>(ck) + kv_base * ROWB;
    const unsigned char *cvrows = static_cast<const unsigned char *>(cv) + kv_base * ROWB;
    auto issue = [&](int kt, Tile &T, unsigned char *vbuf) {
        T.kl = key_of(kt, lane & 31);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            // slot l16 of half t is key 8(l16/4) + 4t + l16%4
            const uint32_t koff = key_ld(kt, 8 * (l16 >> 2) + 4 * t + (l16 & 3)) * ROWB;
#pragma unroll
            for (int cc = 0; cc < KR; ++cc) {
                const int cd = KVDT == DLLM_E4M3 ? 2 * cc : cc;
                T.kr[t][cc] = *reinterpret_cast<const uint4 *>(ckrows + koff + chunk_dim<KVDT>(cd, g) * ESZ);
            }
        }
#pragma unroll
        for (int u = 0; u < VIT; ++u) {
            // this lane fills chunk slot lane % CPR of row RPI*u + lane / CPR
            const int rho = RPI * u + lane / CPR;
            const int chunk = (lane % CPR) ^ vswz<KVDT>(rho);
            const uint32_t off = key_ld(kt, rho) * ROWB + (uint32_t)chunk * 16;
            lds_dma16<NT>(cvrows, off, lds_addr(vbuf) + u * 1024);
        }
        T.kfl = scale_log2;
        T.vsl = 1.f;
        if (KVDT == DLLM_E4M3) {
            const int64_t rr = kv_base + key_ld(kt, lane & 31);
            T.kfl = scale_log2 * ksc[rr];
            T.vsl = vsc[rr];
        }
    };

    // the B operands of S^T, the same for every tile: read once from LDS
    uint4 qreg[RT][NC];
    auto compute = [&](int kt, const Tile &T, const unsigned char *vt) {
        // per-key factors of the keys this lane holds in S^T (8g .. 8g+7), and
        // whether every key of the tile is present (then nothing is masked)
        const bool full = MAP ? (__ballot(T.kl >= 0) == ~0ull) : (kt * 32 + 32 <= n_keys);
        float kfac[8], vfac[8];
        if (KVDT == DLLM_E4M3) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kfac[e] = __shfl(T.kfl, 8 * g + e, kWave);
                vfac[e] = __shfl(T.vsl, 8 * g + e, kWave);
            }
        }
        bool kval[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) kval[e] = true;
        if (!full) {
#pragma unroll
            for (int e = 0; e < 8; ++e) kval[e] = key_of(kt, 8 * g + e) >= 0;
        }
        // K operand of half t, k-chunk c: the loaded bf16 rows as they are, or
        // 8 e4m3 codes widened exactly to bf16
        auto kop = [&](int t, int c) -> bf16x8_t {
            if (KVDT == DLLM_E4M3) {
                const uint4 w = T.kr[t][c >> 1];
                return __builtin_bit_cast(bf16x8_t, (c & 1) ? e4m3x8_to_bf16(w.z, w.w) : e4m3x8_to_bf16(w.x, w.y));
            }
            return __builtin_bit_cast(bf16x8_t, T.kr[t][c]);
        };

        // ---- per row tile: S^T = K Q^T, then the online softmax per row
        // (row = rt*16 + l16) over keys 8g..8g+7 of this lane, in base 2.  The
        // reference max m moves only when a tile's max exceeds it by more than
        // kLazy, so probabilities stay below 2^kLazy and the rescale of O is
        // rare.  m starts at a finite sentinel, so a row without keys yet gives
        // exp2(-inf) = 0, never NaN.
        Frag pf[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                Frag qf;
                qf.u = qreg[rt][c];
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop(0, c), qf.v, s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop(1, c), qf.v, s1, 0, 0, 0);
            }
            const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
            float x[8];
            float mx;
            // a full tile (wave-uniform) masks nothing
            if (KVDT == DLLM_E4M3) {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = sv[e] * kfac[e];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = sv[e];
            }
            if (!full) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (!kval[e]) x[e] = kNegInf;
            }
            mx = x[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) mx = vmax(mx, x[e]);
            // one positive scale for every key (bf16): the max of the raw scores
            if (KVDT != DLLM_E4M3) mx *= scale_log2;
            // the row's max exceeds m + kLazy only if one of its four lanes'
            // does, so the lane maxima are tested first and the row maxima
            // formed only when some lane of the wave sees such a key
            if (__ballot(mx > m[rt] + kLazy)) {
                mx = group4_max(mx);
                if (mx > m[rt] + kLazy) {
                    const float corr = __builtin_amdgcn_exp2f(m[rt] - mx);
                    l[rt] *= corr;
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) o[dt][rt] *= corr;
                    m[rt] = mx;
                }
            }
            const float mref = m[rt];
            float p[8], ps = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a = KVDT == DLLM_E4M3 ? x[e] - mref : fmaf(x[e], scale_log2, -mref);
                p[e] = __builtin_amdgcn_exp2f(a);
                ps += p[e];
            }
            l[rt] += ps;
            if (KVDT == DLLM_E4M3) {
#pragma unroll
                for (int e = 0; e < 8; ++e) p[e] *= vfac[e];
            }
            pf[rt].u = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                  pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
        }

        // ---- O^T += V^T P^T, V^T read from the row-major tile by LDS transpose reads
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            Frag vf;
            if (KVDT == DLLM_E4M3) {
                // local lane j reads row 8g + j/2, codes dt*16 + 8(j%2) .. +7; lane i
                // then holds codes of keys 8g .. 8g+7 at dim dt*16 + i
                const int rho = 8 * g + (l16 >> 1);
                const uint2 c8 = lds_tr8(vt + rho * ROWB + (dt ^ vswz<KVDT>(rho)) * 16 + 8 * (l16 & 1));
                vf.u = e4m3x8_to_bf16(c8.x, c8.y);
            } else {
                // two reads of 4 keys each: local lane j reads row 8g + 4h + j/4,
                // dims dt*16 + 4(j%4) .. +3; lane i then holds keys 8g+4h .. +3 at dim dt*16 + i
                const int r0 = 8 * g + (l16 >> 2), r1 = r0 + 4;
                const int cl = 2 * dt + ((l16 & 3) >> 1);            // logical chunk
                const uint2 lo = lds_tr16(vt + r0 * ROWB + (cl ^ vswz<KVDT>(r0)) * 16 + 8 * (l16 & 1));
                const uint2 hi = lds_tr16(vt + r1 * ROWB + (cl ^ vswz<KVDT>(r1)) * 16 + 8 * (l16 & 1));
                vf.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf.v, pf[rt].v, o[dt][rt], 0, 0, 0);
        }
    };

    // wait until only the loads of the `ahead` tiles issued after this one
    // are outstanding; the scheduling barriers keep every load of a later
    // tile on the far side of the wait
    auto wait_tile = [&](int ahead) {
        __builtin_amdgcn_sched_barrier(0);
        if (ahead <= 0) vm_wait<0>();
        else if (S == 2 || ahead == 1) vm_wait<LOADS>();
        else if (ahead == 2) vm_wait<(S > 2 ? 2 : 1) * LOADS>();
        else vm_wait<(S > 2 ? 3 : 1) * LOADS>();
        __builtin_amdgcn_sched_barrier(0);
    };
    // tile t of this wave's run uses register set and V buffer (t - t_begin) % S
    Tile T[S];
#pragma unroll
    for (int i = 0; i < S - 1; ++i)
        if (t_begin + i < t_end) issue(t_begin + i, T[i], vbase + i * VTILE);
    __builtin_amdgcn_sched_barrier(0);
    // the queries into LDS (their loads were issued before the tiles')
#pragma unroll
    for (int it = 0; it < QIT; ++it) {
        const int idx = threadIdx.x + it * NW * kWave;
        if (idx < QN) *reinterpret_cast<uint4 *>(qs + (idx / (D / 8)) * QSTR + (idx % (D / 8)) * 16) = qv[it];
    }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < NC; ++c)
            qreg[rt][c] = *reinterpret_cast<const uint4 *>(qs + (rt * 16 + l16) * QSTR + chunk_dim<KVDT>(c, g) * 2);
    for (int kt = t_begin; kt < t_end; kt += S) {
#pragma unroll
        for (int j = 0; j < S; ++j) {
            const int t = kt + j;
            if (t >= t_end) break;
            const int jn = (j + S - 1) % S;
            if (t + S - 1 < t_end) issue(t + S - 1, T[jn], vbase + jn * VTILE);
            wait_tile(min(S - 1, t_end - 1 - t));
            compute(t, T[j], vbase + j * VTILE);
        }
    }

    // ---- row sums over the 4 lane groups
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) l[rt] = group4_sum(l[rt]);

    // ---- merge the waves through LDS in one exchange: once every wave is
    // done with the staging area, each stores its unnormalised O~ and its
    // (m, l) per row there; after one more barrier every thread combines
    // one (row, 4 dims) over the waves in order, each wave's share scaled by
    // 2^(m_w - M) with M the row's largest m, and writes the result (or this
    // split's partial).  m starts finite, so a wave without keys adds 0.
    float *buf = reinterpret_cast<float *>(smem);       // [NW][ROWS][BST] floats
    __syncthreads();
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const f32x4_t v = o[dt][rt];
            *reinterpret_cast<float4 *>(buf + (wave * ROWS + rt * 16 + l16) * BST + dt * 16 + 4 * g) =
                make_float4(v[0], v[1], v[2], v[3]);
        }
    if (g == 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            sm_ml[wave][rt * 16 + l16][0] = m[rt];
            sm_ml[wave][rt * 16 + l16][1] = l[rt];
        }
    }
    __syncthreads();
    constexpr int Q4 = D / 4;
    for (int idx = threadIdx.x; idx < ROWS * Q4; idx += NW * kWave) {
        const int r = idx / Q4, c = (idx % Q4) * 4;
        const int rr = rg * ROWS + r;
        if (rr >= M) continue;
        float mw[NW], mm = kMinit;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            mw[w] = sm_ml[w][r][0];
            mm = fmaxf(mm, mw[w]);
        }
        float lt = 0.f;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = __builtin_amdgcn_exp2f(mw[w] - mm);
            lt += sm_ml[w][r][1] * f;
            const float4 v = *reinterpret_cast<const float4 *>(buf + (w * ROWS + r) * BST + c);
            acc += f32x4_t{v.x, v.y, v.z, v.w} * f;
        }
        const int gq = rr / b, i = rr - gq * b;
        const int64_t orow = ((int64_t)bi * Hq + kvh * G + gq) * b + i;
        if (splits == 1) {
            const float inv = lt > 0.f ? 1.0f / lt : 0.f;
            const f32x4_t v = acc * inv;
            const int64_t off = orow * D + c;
            if (out_dtype == DLLM_F32)
                *reinterpret_cast<float4 *>(static_cast<float *>(out) + off) = make_float4(v[0], v[1], v[2], v[3]);
            else
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + off) =
                    make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            if (lse && c == 0) lse[orow] = lt > 0.f ? mm * kLn2 + logf(lt) : kNegInf;
        } else {
            // partial of this split: unnormalised O~, running max (base 2), sum,
            // O~ in the output's precision (bf16 partials for a bf16 output)
            const int64_t prow = (int64_t)split * rows_total + orow;
            if (out_dtype == DLLM_F32)
                *reinterpret_cast<float4 *>(part_o + prow * D + c) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            else
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(part_o) + prow * D + c) =
                    make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
            if (c == 0) {
                part_ml[prow * 2 + 0] = mm;
                part_ml[prow * 2 + 1] = lt;
            }
        }
    }
}

// Merge of the key splits: one thread per (row, 8 dims), splits in order.
// The partial O~ is stored in the output's precision (bf16 for a bf16 output,
// which halves the split traffic; fp32 for an fp32 output); m and l are fp32.
// With up to kU splits every load of a thread is issued in one round; more
// splits take two passes (the maxima, then the sums) of kU splits at a time.
template <int kU>
__device__ __forceinline__ void merge_load(const float *__restrict__ part_o, const float *__restrict__ part_ml,
                                           int64_t rows_total, int D, int splits, int s0, int64_t row, int c,
                                           int out_dtype, float *ms, float *ls, float (*v)[8]) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        ms[u] = kNegInf;
        ls[u] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = 0.f;
        if (s0 + u < splits) {
            const int64_t pr = (int64_t)(s0 + u) * rows_total + row;
            const float2 ml = *reinterpret_cast<const float2 *>(part_ml + pr * 2);
            ms[u] = ml.x;
            ls[u] = ml.y;
            if (out_dtype == DLLM_F32) {
                const float4 a = *reinterpret_cast<const float4 *>(part_o + pr * D + c);
                const float4 b = *reinterpret_cast<const float4 *>(part_o + pr * D + c + 4);
                v[u][0] = a.x; v[u][1] = a.y; v[u][2] = a.z; v[u][3] = a.w;
                v[u][4] = b.x; v[u][5] = b.y; v[u][6] = b.z; v[u][7] = b.w;
            } else {
                const uint4 h = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(part_o) + pr * D + c);
                v[u][0] = bf16lo(h.x); v[u][1] = bf16hi(h.x); v[u][2] = bf16lo(h.y); v[u][3] = bf16hi(h.y);
                v[u][4] = bf16lo(h.z); v[u][5] = bf16hi(h.z); v[u][6] = bf16lo(h.w); v[u][7] = bf16hi(h.w);
            }
        }
    }
}

__global__ __launch_bounds__(256) void attn_merge_kernel(
    const float *__restrict__ part_o, const float *__restrict__ part_ml, int64_t rows_total, int D,
    int splits, void *__restrict__ out, int out_dtype, float *__restrict__ lse) {
    constexpr int kU = 8;                  // splits whose loads are in flight together
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int q8 = D / 8;
    if (t >= rows_total * q8) return;
    const int64_t row = t / q8;
    const int c = (int)(t - row * q8) * 8;
    float ms[kU], ls[kU], v[kU][8];
    float mm = kNegInf;
    if (splits <= kU) {
        merge_load<kU>(part_o, part_ml, rows_total, D, splits, 0, row, c, out_dtype, ms, ls, v);
#pragma unroll
        for (int u = 0; u < kU; ++u) mm = fmaxf(mm, ms[u]);
    } else {
        for (int s0 = 0; s0 < splits; s0 += kU) {
#pragma unroll
            for (int u = 0; u < kU; ++u)
                ms[u] = s0 + u < splits ? part_ml[((int64_t)(s0 + u) * rows_total + row) * 2] : kNegInf;
#pragma unroll
            for (int u = 0; u < kU; ++u) mm = fmaxf(mm, ms[u]);
        }
    }
    float lt = 0.f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (mm != kNegInf) {
        for (int s0 = 0; s0 < splits; s0 += kU) {
            if (splits > kU) merge_load<kU>(part_o, part_ml, rows_total, D, splits, s0, row, c, out_dtype, ms, ls, v);
            // in split order
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if (ms[u] == kNegInf) continue;
                const float f = __builtin_amdgcn_exp2f(ms[u] - mm);
                lt += ls[u] * f;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += v[u][e] * f;
            }
        }
    }
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int64_t off = row * D + c;
    if (out_dtype == DLLM_F32) {
        float *o = static_cast<float *>(out) + off;
        *reinterpret_cast<float4 *>(o) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
        *reinterpret_cast<float4 *>(o + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    } else {
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + off) =
            make_uint4(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                       pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv));
    }
    if (lse && c == 0) lse[row] = lt > 0.f ? mm * kLn2 + logf(lt) : kNegInf;
}

// ---- float32 VALU path: one wave per query row ----------------------------
// Keys go 64 at a time: lane j scores key j of the tile, the tile's
// probabilities go through LDS, and lane c accumulates output dims c, c+64,
// c+128, c+192.
__device__ __forceinline__ float load_elem(const void *p, int dtype, int64_t i, const float *sc,
                                           int64_t srow, int c) {
    if (dtype == DLLM_F32) return static_cast<const float *>(p)[i];
    if (dtype == DLLM_BF16) return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
    const uint32_t code = static_cast<const uint8_t *>(p)[i];
    const f32x2_t v = __builtin_amdgcn_cvt_pk_f32_fp8(code, false);
    return v[0] * sc[srow + (c >> 7)];
}

__global__ __launch_bounds__(256) void attn_valu_kernel(
    const void *__restrict__ ck, const void *__restrict__ cv, const float *__restrict__ ksc,
    const float *__restrict__ vsc, int kv_dtype, const void *__restrict__ q, int q_dtype, int B,
    int Hq, int Hkv, int L, int D, int b, const int32_t *__restrict__ key_idx, int n_keys,
    float scale, const float *__restrict__ memo_o, const float *__restrict__ memo_lse,
    void *__restrict__ out, int out_dtype, float *__restrict__ lse) {
    __shared__ float sq[4][256];
    __shared__ float sp[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave;     // (bi, hq, i)
    const int64_t rows_total = (int64_t)B * Hq * b;
    const bool live = row < rows_total;
    const int64_t rr = live ? row : 0;
    const int bi = (int)(rr / ((int64_t)Hq * b));
    const int hq = (int)((rr / b) % Hq);
    const int kvh = hq / (Hq / Hkv);
    const int64_t kv_base = ((int64_t)bi * Hkv + kvh) * L;
    const int ng = D >> 7;
    for (int c = lane; c < D; c += 64)
        sq[wave][c] = q_dtype == DLLM_F32 ? static_cast<const float *>(q)[rr * D + c]
                                          : bf16_to_f32(static_cast<const uint16_t *>(q)[rr * D + c]);
    __syncthreads();
    const int32_t *kmap = key_idx ? key_idx + (int64_t)bi * n_keys : nullptr;
    float mrun = kNegInf, lrun = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (memo_lse) {
        // a memoized state (FACache): m = lse, l = 1, O~ = memo_o; -inf is empty
        const float ml = memo_lse[rr];
        if (ml != kNegInf) {
            mrun = ml;
            lrun = 1.f;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (lane + 64 * r < D) acc[r] = memo_o[rr * D + lane + 64 * r];
        }
    }
    for (int j0 = 0; j0 < n_keys; j0 += 64) {
        const int kk = key_at(kmap, n_keys, L, j0 + lane);
        float sc = kNegInf;
        if (kk >= 0) {
            const int64_t krow = kv_base + kk;
            float dot = 0.f;
            for (int c = 0; c < D; ++c)
                dot = fmaf(sq[wave][c], load_elem(ck, kv_dtype, krow * D + c, ksc, krow * ng, c), dot);
            sc = dot * scale;
        }
        float mx = sc;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
        const float mn = fmaxf(mrun, mx);
        if (mn == kNegInf) continue;                         // wave-uniform
        const float corr = expf(mrun - mn);
        const float p = expf(sc - mn);
        float ps = p;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) ps += shfl_xor_f(ps, o);
        lrun = lrun * corr + ps;
        mrun = mn;
        sp[wave][lane] = p;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= corr;
        const int nk = min(64, n_keys - j0);
        for (int j = 0; j < nk; ++j) {
            const float pj = sp[wave][j];
            const int kj = key_at(kmap, n_keys, L, j0 + j);
            if (pj == 0.f || kj < 0) continue;
            const int64_t vrow = kv_base + kj;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = lane + 64 * r;
                if (c < D) acc[r] = fmaf(pj, load_elem(cv, kv_dtype, vrow * D + c, vsc, vrow * ng, c), acc[r]);
            }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
    if (!live) return;
    const float inv = lrun > 0.f ? 1.0f / lrun : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int c = lane + 64 * r;
        if (c >= D) break;
        const float v = acc[r] * inv;
        if (out_dtype == DLLM_F32) static_cast<float *>(out)[rr * D + c] = v;
        else static_cast<uint16_t *>(out)[rr * D + c] = f32_to_bf16(v);
    }
    if (lse && lane == 0) lse[rr] = lrun > 0.f ? mrun + logf(lrun) : kNegInf;
}

template <int D, int KVDT, int RT, bool MAP, bool NT, int NW>
int launch_mfma(const dllm_kv_cache &c, const AttnPlan &p, const void *q, int Hq, int b,
                const int32_t *key_idx, int n_keys, float scale, void *out, int out_dtype,
                float *lse, void *ws, hipStream_t s, const ScatterIn &sc) {
    const int G = Hq / c.n_kv_heads;
    const int64_t rows_total = (int64_t)c.B * Hq * b;
    const int64_t blocks = (int64_t)c.B * c.n_kv_heads * p.row_groups * p.splits;
    if (MAP && p.tiles_per_wave > kMapTableTiles / NW) return DLLM_ESHAPE;   // the key table holds them
    if (blocks > INT_MAX) return DLLM_ERANGE;
    float *part_o = nullptr, *part_ml = nullptr;
    if (p.splits > 1) {
        part_o = static_cast<float *>(ws);
        part_ml = part_o + (int64_t)p.splits * rows_total * D;
    }
    const float scale_log2 = scale * kLog2e;
    attn_mfma_kernel<D, KVDT, RT, MAP, NT, NW><<<dim3((unsigned)blocks), dim3(NW * kWave), 0, s>>>(
        c.k, c.v, c.k_scale, c.v_scale, static_cast<const uint16_t *>(q), Hq, c.n_kv_heads, c.L,
        b, G, key_idx, n_keys, scale_log2, p.row_groups, p.splits, p.tiles_per_wave, rows_total,
        out, out_dtype, lse, part_o, part_ml, sc);
    int rc = launch_status();
    if (rc != DLLM_OK || p.splits == 1) return rc;
    return launch_attn_merge(part_o, part_ml, rows_total, D, p.splits, out, out_dtype, lse, s);
}

}  // namespace

int launch_attn_merge(const float *part_o, const float *part_ml, int64_t rows_total, int D,
                      int splits, void *out, int out_dtype, float *lse, hipStream_t s) {
    const int64_t threads = rows_total * (D / 8);
    attn_merge_kernel<<<dim3((unsigned)cdiv64(threads, 256)), dim3(256), 0, s>>>(
        part_o, part_ml, rows_total, D, splits, out, out_dtype, lse);
    return launch_status();
}

int plan_attention(const dllm_kv_cache &c, int q_dtype, int Hq, int b, int n_keys, bool has_map, AttnPlan *p) {
    const int G = Hq / c.n_kv_heads;
    const int M = G * b;
    const bool mfma = q_dtype == DLLM_BF16 && (c.dtype == DLLM_BF16 || c.dtype == DLLM_E4M3) &&
                      (c.d_head == 64 || c.d_head == 128);
    *p = AttnPlan{};
    p->rows = M;
    if (!mfma) {
        p->path = 0;
        return DLLM_OK;
    }
    // several 32-row groups per KV head: the waves of a workgroup share tiles
    if (M > 32) {
        plan_shared(c, Hq, b, cdiv(M, 32), n_keys, has_map, p);
        return DLLM_OK;
    }
    p->path = 1;
    // 32 rows per workgroup: 64-row waves hold 128 accumulator floats per lane
    // and drop to one wave per SIMD, which measured slower at every shape
    p->row_tiles = 2;
    p->row_groups = cdiv(M, 16 * p->row_tiles);
    const int64_t units = (int64_t)c.B * c.n_kv_heads * p->row_groups;
    const int n_tiles = cdiv(n_keys, 32);
    const int esz = c.dtype == DLLM_E4M3 ? 1 : 2;
    // About 8 waves per CU in all.  Few (sequence, KV head, row group) units
    // first get wider workgroups (8, then 16 waves, while the LDS holds them
    // and every wave keeps 2 key tiles), and only then key splits, which cost
    // a partial write and a merge pass.
    const int64_t want = 2048;
    int nw = 4;
    // 8-wave workgroups when the units are few (16 waves would leave 128
    // VGPRs per lane and spill; measured slower)
    if (units * nw < want && n_tiles >= 16 &&
        attn_smem_bytes(c.d_head, esz, p->row_tiles, 8, has_map) <= kLdsBytes)
        nw = 8;
    p->waves = nw;
    int splits = (int)std::max<int64_t>(1, cdiv64(want, units * nw));
    splits = std::min(splits, std::max(1, n_tiles / (4 * nw)));      // at least 4 tiles per wave
    if (has_map) splits = std::max(splits, cdiv(n_tiles, kMapTableTiles));   // the table holds them
    p->splits = splits;
    p->tiles_per_wave = cdiv(n_tiles, splits * nw);
    p->ws_bytes = splits > 1 ? (size_t)splits * c.B * Hq * b * (c.d_head + 2) * sizeof(float) : 0;
    return DLLM_OK;
}

int plan_facache(const dllm_kv_cache &c, int q_dtype, int Hq, int n_q, int n_keys, bool has_map,
                 AttnPlan *p) {
    const int G = Hq / c.n_kv_heads;
    const int M = G * n_q;
    const bool mfma = q_dtype == DLLM_BF16 && (c.dtype == DLLM_BF16 || c.dtype == DLLM_E4M3) &&
                      (c.d_head == 64 || c.d_head == 128);
    *p = AttnPlan{};
    p->rows = M;
    if (!mfma) {
        p->path = 0;
        return DLLM_OK;
    }
    // the grouped-query layout takes the memo at any row count
    plan_shared(c, Hq, n_q, cdiv(M, 32), n_keys, has_map, p);
    return DLLM_OK;
}

static int launch_attention_sc(const dllm_kv_cache &c, const AttnPlan &p, const void *q, int q_dtype,
                               int Hq, int b, const int32_t *key_idx, int n_keys, float scale,
                               const AttnMemo &memo, void *out, int out_dtype, float *lse, void *ws,
                               hipStream_t s, const ScatterIn &sc) {
    if (p.path == 0) {
        const int64_t rows_total = (int64_t)c.B * Hq * b;
        attn_valu_kernel<<<dim3((unsigned)cdiv64(rows_total, 4)), dim3(256), 0, s>>>(
            c.k, c.v, c.k_scale, c.v_scale, c.dtype, q, q_dtype, c.B, Hq, c.n_kv_heads, c.L,
            c.d_head, b, key_idx, n_keys, scale, memo.o, memo.lse, out, out_dtype, lse);
        return launch_status();
    }
    if (p.path == 2)
        return launch_shared_attention(c, p, q, Hq, b, key_idx, n_keys, scale, memo, out, out_dtype,
                                       lse, ws, s);
    if (memo.lse) return DLLM_EINVAL;           // never planned: the per-wave path takes no memo
    const bool e4 = c.dtype == DLLM_E4M3;
    const bool map = key_idx != nullptr;
    // stream K/V past the caches when only one row group reads each KV head
    const bool nt = p.row_groups == 1;
    auto go = [&](auto dd, auto kv, auto mp) -> int {
        constexpr int DD = decltype(dd)::value, KV = decltype(kv)::value;
        constexpr bool MP = decltype(mp)::value;
        constexpr int ES = KV == DLLM_E4M3 ? 1 : 2;
        auto run = [&](auto ntv, auto nwv) -> int {
            constexpr bool NTV = decltype(ntv)::value;
            constexpr int NW = decltype(nwv)::value;
            if constexpr (attn_smem_bytes(DD, ES, 2, NW, MP) <= kLdsBytes)
                return launch_mfma<DD, KV, 2, MP, NTV, NW>(c, p, q, Hq, b, key_idx, n_keys, scale, out,
                                                           out_dtype, lse, ws, s, sc);
            return DLLM_ESHAPE;                 // never planned
        };
        auto pick = [&](auto ntv) -> int {
            if (p.waves == 4) return run(ntv, std::integral_constant<int, 4>{});
            if (p.waves == 8) return run(ntv, std::integral_constant<int, 8>{});
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
    if (e4) return DLLM_ESHAPE;                 // e4m3 needs d % 128 == 0
    return map ? go(I64{}, KB{}, std::true_type{}) : go(I64{}, KB{}, std::false_type{});
}

int launch_attention(const dllm_kv_cache &c, const AttnPlan &p, const void *q, int q_dtype, int Hq,
                     int b, const int32_t *key_idx, int n_keys, float scale, const AttnMemo &memo,
                     void *out, int out_dtype, float *lse, void *ws, hipStream_t s) {
    return launch_attention_sc(c, p, q, q_dtype, Hq, b, key_idx, n_keys, scale, memo, out, out_dtype, lse,
                               ws, s, ScatterIn{});
}

int launch_scatter_attention(const dllm_kv_cache &c, const AttnPlan &p, const void *k_new,
                             const void *v_new, int src_dtype, const int32_t *pos, int n,
                             int32_t *bad, const void *q, int q_dtype, int Hq, int b,
                             const int32_t *key_idx, int n_keys, float scale, void *out,
                             int out_dtype, float *lse, void *ws, hipStream_t s) {
    // one launch where the per-wave kernel reads the keys in place (bf16
    // cache and rows, no key map); otherwise the scatter, then the attention
    if (n > 0 && p.path == 1 && !key_idx && c.dtype == DLLM_BF16 && src_dtype == DLLM_BF16) {
        ScatterIn sc;
        sc.k_new = static_cast<const uint4 *>(k_new);
        sc.v_new = static_cast<const uint4 *>(v_new);
        sc.pos = pos;
        sc.n = n;
        sc.bad = bad;
        return launch_attention_sc(c, p, q, q_dtype, Hq, b, key_idx, n_keys, scale, AttnMemo{}, out,
                                   out_dtype, lse, ws, s, sc);
    }
    int rc = launch_scatter(c, k_new, v_new, src_dtype, pos, n, bad, s);
    if (rc != DLLM_OK) return rc;
    return launch_attention(c, p, q, q_dtype, Hq, b, key_idx, n_keys, scale, AttnMemo{}, out, out_dtype,
                            lse, ws, s);
}

}  // namespace dllm
