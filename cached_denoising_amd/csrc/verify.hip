// Self-verification of the tokens decoded in parallel in one step, and the
// withdrawal of conflicting spans [Flash-dLLM page, 4.2 and 4.3]: for two
// positions decoded in the same step at most W-1 apart, the conflict score
// is their joint probability over the product of their marginals, and a
// score below tau withdraws every position decoded in the span between
// them.  A withdrawn position is regenerated serially, so its stable flag
// and its cached K/V are dropped and it joins the next step's mask.
//
// One workgroup of 1024 threads per sequence:
//   1. the decoded list is checked (ascending, then -1 padding);
//   2. each entry's conflict bits (bit d-1: the pair at distance d) are
//      computed in float64, the partner of distance d being among the next
//      d entries of an ascending list; entries are taken in chunks with a
//      halo of W-1 earlier entries in LDS, and an entry is withdrawn when a
//      conflicting pair starting at most W-1 entries before it covers it;
//   3. the mask is loaded as bits (kVUnroll loads per thread in flight),
//      each thread owns whole words of it for one scan of the next mask,
//      and one pass over the positions stores the withdrawal flags, the
//      mask, the stable and cached flags and the compacted mask;
//   4. the withdrawn positions are listed in ascending order.
#include "common.hpp"

namespace dllm {
namespace {

constexpr int kVThreads = 1024;
constexpr int kVWaves = kVThreads / kWave;
constexpr int kMaxWin = 8;          // W: pairs at distance 1 .. W-1
constexpr int kMaxLV = 131072;      // bits and prefixes stay within 48 KB of LDS

constexpr int kVUnroll = 8;         // positions per thread in flight in the mask load
__global__ __launch_bounds__(kVThreads) void verify_kernel(
    int L, const int32_t *__restrict__ dec_pos, int n, const float *__restrict__ p_marg,
    const float *__restrict__ p_joint, int W, double tau, uint8_t *__restrict__ rollback,
    uint8_t *__restrict__ mask, uint8_t *__restrict__ stable, uint8_t *__restrict__ cached,
    int32_t *__restrict__ next_pos, int32_t *__restrict__ count, int32_t *__restrict__ n_rollback,
    int32_t *__restrict__ rb_pos) {
    // dynamic LDS: withdrawn positions, then the mask (the next mask once
    // decided), then a prefix per mask word, one bit (word) each
    extern __shared__ uint32_t rbits[];
    __shared__ int s_pos[kVThreads + kMaxWin];         // a chunk of entries after its halo
    __shared__ uint8_t s_cb[kVThreads + kMaxWin];      // their conflict bits
    __shared__ int wave_cnt[2][kVWaves];               // per-wave counts, double-buffered
    __shared__ int s_nv, s_bad;
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int64_t rowoff = (int64_t)b * L;
    const int32_t *dp = dec_pos + (int64_t)b * n;
    const float *pm = p_marg + (int64_t)b * n;
    const int H = W - 1;
    const float *pj = p_joint + (int64_t)b * n * H;
    const int words = (L + 31) >> 5;
    uint32_t *mbits = rbits + words;
    int *wpref = reinterpret_cast<int *>(mbits + words);

    for (int w = tid; w < words; w += kVThreads) rbits[w] = 0;
    if (tid == 0) {
        s_nv = n;
        s_bad = 0;
    }
    __syncthreads();
    // 1. the valid entries end at the first padding entry
    for (int j = tid; j < n; j += kVThreads)
        if (dp[j] < 0 && (j == 0 || dp[j - 1] >= 0)) atomicMin(&s_nv, j);
    __syncthreads();
    const int nv = s_nv;
    for (int j = tid; j < n; j += kVThreads) {
        const int p = dp[j];
        const bool bad = j < nv ? (p >= L || (j + 1 < nv && dp[j + 1] <= p)) : p != -1;
        if (bad) s_bad = 1;
    }
    __syncthreads();
    if (s_bad) {                                        // uniform: the sequence is left unchanged
        if (tid == 0) {
            count[b] = -1;
            if (n_rollback) n_rollback[b] = -1;
        }
        return;
    }

    // 2. conflict bits and withdrawals, chunk by chunk
    for (int c0 = 0; c0 < nv; c0 += kVThreads) {
        for (int t = tid; t < kVThreads + H; t += kVThreads) {
            const int j = c0 - H + t;                   // entry of buffer slot t
            int p = -1;
            uint32_t bits = 0;
            if (j >= 0 && j < nv) {
                p = dp[j];
                const double mj = (double)pm[j];
                for (int d = 1; d <= H; ++d) {
                    for (int k = j + 1; k <= j + d && k < nv; ++k) {
                        const int pk = dp[k];
                        if (pk == p + d) {
                            const double prod = mj * (double)pm[k];
                            const double joint = (double)pj[(int64_t)j * H + (d - 1)];
                            if (prod > 0.0 && joint / prod < tau) bits |= 1u << (d - 1);
                        }
                        if (pk >= p + d) break;
                    }
                }
            }
            s_pos[t] = p;
            s_cb[t] = (uint8_t)bits;
        }
        __syncthreads();
        const int m = c0 + tid;
        if (m < nv) {
            const int pmx = s_pos[tid + H];
            bool rb = false;
            for (int t = tid; t <= tid + H; ++t) {      // entries m - H .. m
                const int pa = s_pos[t];
                const uint32_t bits = s_cb[t];
                if (pa < 0 || !bits) continue;
                for (int d = 1; d <= H; ++d)
                    if (((bits >> (d - 1)) & 1u) && pa + d >= pmx) rb = true;
            }
            if (rb) atomicOr(&rbits[pmx >> 5], 1u << (pmx & 31));
        }
        __syncthreads();                                // the buffers are refilled
    }

    // 3. the mask as bits (a wave's ballot over 64 positions is two words)
    const uint8_t *mr = mask + rowoff;
    for (int i0 = 0; i0 < L; i0 += kVThreads * kVUnroll) {
        uint8_t mv[kVUnroll];
#pragma unroll
        for (int u = 0; u < kVUnroll; ++u) {
            const int i = i0 + u * kVThreads + tid;
            mv[u] = i < L ? mr[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < kVUnroll; ++u) {
            const int c0 = i0 + u * kVThreads;
            if (c0 >= L) break;                         // uniform over the workgroup
            const uint64_t bm = __ballot(mv[u] != 0);
            const int w0 = (c0 + wave * kWave) >> 5;
            if (lane == 0 && w0 < words) mbits[w0] = (uint32_t)bm;
            if (lane == 1 && w0 + 1 < words) mbits[w0 + 1] = (uint32_t)(bm >> 32);
        }
    }
    __syncthreads();
    // the next mask, and its prefix per word: each thread owns a run of words
    const int wpt = (words + kVThreads - 1) / kVThreads;
    const int w_lo = min(words, tid * wpt), w_hi = min(words, w_lo + wpt);
    int n_on = 0;
    for (int w = w_lo; w < w_hi; ++w) {
        const uint32_t on = mbits[w] | rbits[w];
        mbits[w] = on;
        n_on += __popc(on);
    }
    int base;
    int on_off = block_exclusive_scan<kVWaves>(n_on, lane, wave, wave_cnt[0], base);
    for (int w = w_lo; w < w_hi; ++w) {
        wpref[w] = on_off;
        on_off += __popc(mbits[w]);
    }
    __syncthreads();
    // store pass: four consecutive positions per thread, so a wave's
    // withdrawal flags cover 256 contiguous bytes (whole lines); the flags of
    // the few withdrawn positions are written one by one
    const bool al_r = (((uintptr_t)(rollback + rowoff)) & 3u) == 0;
#pragma unroll 2
    for (int i = 4 * tid; i < L; i += 4 * kVThreads) {
        const int w = i >> 5, sh = i & 31;             // the four positions share word w
        const uint32_t r4 = (rbits[w] >> sh) & 0xFu;
        const uint32_t mw = mbits[w];
        store_flags4(rollback + rowoff + i, r4, L - i, al_r);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if ((r4 >> k) & 1u) {
                mask[rowoff + i + k] = 1;
                if (stable) stable[rowoff + i + k] = 0;
                if (cached) cached[rowoff + i + k] = 0;
            }
            if ((mw >> (sh + k)) & 1u) next_pos[rowoff + wpref[w] + __popc(mw & ((1u << (sh + k)) - 1u))] = i + k;
        }
    }
    for (int i = base + tid; i < L; i += kVThreads) next_pos[rowoff + i] = -1;

    // 4. the withdrawn positions in list (ascending) order
    int nr = 0;
    for (int j0 = 0, par = 0; j0 < nv; j0 += kVThreads, par ^= 1) {
        const int j = j0 + tid;
        bool rb = false;
        int p = -1;
        if (j < nv) {
            p = dp[j];
            rb = (rbits[p >> 5] >> (p & 31)) & 1u;
        }
        const uint64_t bal = __ballot(rb);
        if (lane == 0) wave_cnt[par][wave] = __popcll(bal);
        __syncthreads();
        int off = nr, chunk = 0;
        for (int w = 0; w < kVWaves; ++w) {
            const int v = wave_cnt[par][w];
            off += w < wave ? v : 0;
            chunk += v;
        }
        if (rb && rb_pos) rb_pos[(int64_t)b * n + off + __popcll(bal & lanes_below(lane))] = p;
        nr += chunk;
    }
    if (rb_pos)
        for (int j = nr + tid; j < n; j += kVThreads) rb_pos[(int64_t)b * n + j] = -1;
    if (tid == 0) {
        count[b] = base;
        if (n_rollback) n_rollback[b] = nr;
    }
}

}  // namespace

int launch_self_verify(int B, int L, const int32_t *dec_pos, int n, const float *p_marg,
                       const float *p_joint, int W, double tau, uint8_t *rollback, uint8_t *mask,
                       uint8_t *stable, uint8_t *cached, int32_t *next_pos, int32_t *count,
                       int32_t *n_rollback, int32_t *rb_pos, hipStream_t s) {
    if (L > kMaxLV || W > kMaxWin) return DLLM_ERANGE;
    const size_t shmem = 3 * sizeof(uint32_t) * (size_t)((L + 31) / 32);   // withdrawn, mask, prefix
    verify_kernel<<<dim3((unsigned)B), dim3(kVThreads), shmem, s>>>(
        L, dec_pos, n, p_marg, p_joint, W, tau, rollback, mask, stable, cached, next_pos, count,
        n_rollback, rb_pos);
    return launch_status();
}

}  // namespace dllm
