// History ring, stability test, cache confidence and window mask, fused into
// one kernel with one workgroup per sequence.
//   - SWD page, 3.1: a position is stable once its argmax has held for K
//     consecutive steps and the mean max-probability over them exceeds tau;
//     3.3 steps c-d and 4.2 (update_stability): record the step, test only
//     positions not yet stable; 3.2 and 4.2 (get_computation_mask): every
//     position still to compute widens into [u-R, u+R], clamped; with none
//     left the whole sequence is computed.
//   - Flash-dLLM page, 3.1: cache confidence alpha(1 - H/Hmax) +
//     beta exp(-lambda (t - t_write)); a confidence below the threshold
//     sends the position back to be recomputed.
//   - SWD page, 4.4: the window radius may widen over the trajectory (small
//     or none early, larger late): a linear ramp from R_early to R.
//   - Flash-dLLM page, 5.1: a full refresh every few steps.
// The decisions (mean > tau, conf < threshold) are taken in float64, each
// value a chain of single IEEE operations on the same inputs as the plain
// definition: this file is compiled without floating-point contraction (no
// fused multiply-add), and the age factor exp(-lambda dt) is read from a
// table the host computed, so the confidence and every decision on it equal
// the definition's float64 values bit for bit.
//
// Also the budgeted cache of Flash-dLLM 3.3 and 5.2: per sequence, the
// cached positions beyond its quota leave the cache lowest confidence first,
// and every position without cached K/V joins the next step's mask.
#include "common.hpp"

#pragma clang fp contract(off)

namespace dllm {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxL = 131072;      // seed bits stay within 16 KB of LDS
constexpr int kWaves = kThreads / kWave;

__global__ __launch_bounds__(256) void stability_reset_kernel(
    int64_t ring_n, int64_t n, int32_t *__restrict__ ring_argmax, float *__restrict__ ring_maxprob,
    int32_t *__restrict__ ring_step, float *__restrict__ entropy_latest,
    int32_t *__restrict__ t_write, uint8_t *__restrict__ stable) {
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t st = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = i0; i < ring_n; i += st) {
        ring_argmax[i] = 0;
        ring_maxprob[i] = 0.f;
        ring_step[i] = -1;
    }
    for (int64_t i = i0; i < n; i += st) {
        entropy_latest[i] = 0.f;
        t_write[i] = 0;
        stable[i] = 0;
    }
}

// The confidence and seed bit of one position, from its entropy, the step
// its K/V were written and its stable flag.
__device__ __forceinline__ bool seed_of(double alpha, double beta, const double *__restrict__ decay,
                                        int n_decay, double hmax, double conf_thresh, int step, float en,
                                        int tw, bool st, float *conf_out) {
    // with the gate off (alpha = beta = 0) the score is +0 whatever the
    // entropy and age; a zero beta drops the age term, which would add +0
    // (the table is then not read)
    double cf = 0.0;
    if (alpha != 0.0 || beta != 0.0) {
        const double h = (double)en;
        double age = 0.0;
        if (beta != 0.0) {
            const int dt = step - tw;
            age = beta * decay[dt < 0 ? 0 : min(dt, n_decay - 1)];
        }
        cf = alpha * (1.0 - h / hmax) + age;
    }
    if (conf_out) *conf_out = (float)cf;
    return !st || cf < conf_thresh;
}

// ALL: every position recomputed in list order (pos == NULL, n == L <= 2
// kThreads), so thread t holds the new state of positions t and t + kThreads
// and takes their confidence and seed bits in the same pass, without reading
// the state back.
template <bool ALL>
__global__ __launch_bounds__(kThreads) void stability_kernel(
    int B, int L, int step_arg, int32_t *__restrict__ step_dev, int advance, const int32_t *__restrict__ pos, int n,
    const int32_t *__restrict__ argmax, const float *__restrict__ maxprob,
    const float *__restrict__ entropy, int32_t *__restrict__ ring_argmax,
    float *__restrict__ ring_maxprob, int32_t *__restrict__ ring_step,
    float *__restrict__ entropy_latest, int32_t *__restrict__ t_write,
    uint8_t *__restrict__ stable, int K, int D, int R, int R_early, int T_steps, int refresh_every,
    double tau, double alpha, double beta, const double *__restrict__ decay, int n_decay,
    double conf_thresh, double hmax, uint8_t *__restrict__ mask,
    float *__restrict__ conf, int32_t *__restrict__ next_pos, int32_t *__restrict__ count,
    uint8_t *__restrict__ all_stable) {
    extern __shared__ uint32_t seed_bits[];            // one bit per position
    __shared__ int any_seed;
    __shared__ int wave_cnt[kWaves];
    const int b = blockIdx.x;
    const int step = step_dev ? step_dev[b] : step_arg;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int64_t rowoff = (int64_t)b * L;
    const int64_t plane = (int64_t)B * L;              // one ring slot
    const int slot = step % D;
    // the window radius of this step (a ramp from R_early at step 0 to R at
    // step T_steps - 1) and whether this step is a scheduled full refresh
    const int Rs = T_steps > 1 ? R_early + (R - R_early) * min(step, T_steps - 1) / (T_steps - 1) : R;
    const bool refresh = refresh_every > 0 && step > 0 && step % refresh_every == 0;

    if (tid == 0) any_seed = 0;

    // 1-2: record this step, then test the recomputed positions.  Every load
    // of a position is independent of the others, so they are all in flight
    // together; K is small.
    bool fused_seed[2] = {false, false};
    for (int j = tid; j < n; j += kThreads) {
        const int p = pos ? pos[(int64_t)b * n + j] : j;
        if (p < 0 || p >= L) continue;
        const int64_t src = (int64_t)b * n + j;
        const int tok = argmax[src];
        const float mp = maxprob[src];
        const float en = entropy[src];
        const uint8_t was_stable = stable[rowoff + p];
        const bool test = !was_stable && step + 1 >= K;
        bool same = true;
        double sum = 0.0;
        if (test) {
            for (int k = K - 1; k >= 1; --k) {         // oldest record first
                const int64_t rk = (int64_t)((step - k) % D) * plane + rowoff + p;
                const int rs = ring_step[rk];
                const int ra = ring_argmax[rk];
                const float rp = ring_maxprob[rk];
                same = same && rs == step - k && ra == tok;
                sum += (double)rp;
            }
            sum += (double)mp;                         // this step's record last
        }
        const int64_t ri = slot * plane + rowoff + p;
        ring_argmax[ri] = tok;
        ring_maxprob[ri] = mp;
        ring_step[ri] = step;
        entropy_latest[rowoff + p] = en;
        t_write[rowoff + p] = step;
        const bool now_stable = was_stable || (test && same && sum / (double)K > tau);
        if (!was_stable && now_stable) stable[rowoff + p] = 1;
        if (ALL) {
            float cf;
            fused_seed[j / kThreads] = seed_of(alpha, beta, decay, n_decay, hmax, conf_thresh, step, en, step,
                                               now_stable, &cf);
            if (conf) conf[rowoff + p] = cf;
        }
    }
    __syncthreads();                                   // also orders any_seed's reset before its sets

    // 3-4a: confidence and the seed bit of every position (one per thread)
    for (int i0 = 0; i0 < L; i0 += kThreads) {
        const int i = i0 + tid;
        bool seed = false;
        if (ALL) {
            seed = i < L && fused_seed[i0 / kThreads];
        } else if (i < L) {
            float cf;
            seed = seed_of(alpha, beta, decay, n_decay, hmax, conf_thresh, step, entropy_latest[rowoff + i],
                           t_write[rowoff + i], stable[rowoff + i] != 0, &cf);
            if (conf) conf[rowoff + i] = cf;
        }
        const uint64_t bal = __ballot(seed);
        if (lane == 0) {
            const int w = (i0 >> 5) + wave * 2;         // two 32-bit words per wave
            seed_bits[w] = (uint32_t)bal;
            seed_bits[w + 1] = (uint32_t)(bal >> 32);
            if (bal) any_seed = 1;
        }
    }
    __syncthreads();
    const bool none = any_seed == 0;
    const bool all_on = none || refresh;

    // 4b-5: window test per position, then ascending compaction, 1024 at a time
    int base = 0;
    for (int i0 = 0; i0 < L; i0 += kThreads) {
        const int i = i0 + tid;
        bool on = false;
        if (i < L) {
            if (all_on) {
                on = true;
            } else {
                const int lo = max(0, i - Rs), hi = min(L - 1, i + Rs);
                const int wl = lo >> 5, wh = hi >> 5;
                for (int q = wl; q <= wh && !on; ++q) {
                    uint32_t m = seed_bits[q];
                    if (q == wl) m &= 0xffffffffu << (lo & 31);
                    if (q == wh && (hi & 31) != 31) m &= (1u << ((hi & 31) + 1)) - 1u;
                    on = m != 0;
                }
            }
            mask[rowoff + i] = on ? 1 : 0;
        }
        const uint64_t bal = __ballot(on);
        if (lane == 0) wave_cnt[wave] = __popcll(bal);
        __syncthreads();
        int off = base;
        for (int w = 0; w < wave; ++w) off += wave_cnt[w];
        int chunk_total = 0;
        for (int w = 0; w < kWaves; ++w) chunk_total += wave_cnt[w];
        if (on) {
            const uint64_t below = lane ? (bal & ((~0ull) >> (64 - lane))) : 0ull;
            next_pos[rowoff + off + __popcll(below)] = i;
        }
        base += chunk_total;
        __syncthreads();                               // wave_cnt is reused
    }
    for (int i = base + tid; i < L; i += kThreads) next_pos[rowoff + i] = -1;
    if (tid == 0) {
        count[b] = base;
        all_stable[b] = none ? 1 : 0;
        // every thread of this workgroup read step_dev[b] before the barriers above
        if (advance) step_dev[b] = step + 1;
    }
}

// ---- eviction under a per-sequence quota ------------------------------------
// One workgroup per sequence.  The cached flags (with this step's recomputed
// positions added) become an LDS bitset; when they outnumber the quota, a
// four-pass radix select over order-preserving 32-bit keys of the
// confidences finds the quota-th largest key T and how many of the
// positions at T stay (the lowest positions among them, by an ascending
// ballot scan).  Integer decisions only, so the result does not depend on the
// thread count.
__device__ __forceinline__ uint32_t conf_key(float c) {
    uint32_t u = __float_as_uint(c);
    if (u == 0x80000000u) u = 0;                       // -0 orders as +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The selection histogram is kept in 16 copies (a lane adds to copy lane % 16)
// 257 words apart, so that the lanes of a wave counting one digit -- the
// top key byte of confidences within a binade is shared -- land on 16
// different banks instead of serialising on one word.
constexpr int kHistCopies = 16;
constexpr int kHistStride = 257;

// The digit at which the `need`-th largest key lies, from the 256-bin
// histogram: one wave, four bins per lane from the top, a lane scan of the
// counts.  Writes the digit and the count of keys above it, and leaves the
// histogram cleared for the next pass.
__device__ __forceinline__ void select_digit(int *hist, int need, int lane, int *s_sel) {
    int h[4];
    int tot = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int d = 255 - 4 * lane - k;
        int c = 0;
#pragma unroll
        for (int cp = 0; cp < kHistCopies; ++cp) c += hist[cp * kHistStride + d];
#pragma unroll
        for (int cp = 0; cp < kHistCopies; ++cp) hist[cp * kHistStride + d] = 0;
        h[k] = c;
        tot += c;
    }
    int incl = tot;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    const uint64_t hit = __ballot(incl >= need);
    const int first = hit ? __ffsll((unsigned long long)hit) - 1 : kWave - 1;
    if (lane == first) {
        int run = incl - tot;
        int d = 255 - 4 * lane - 3, above = run + h[0] + h[1] + h[2];
        bool found = false;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (!found && run + h[k] >= need) {
                d = 255 - 4 * lane - k;
                above = run;
                found = true;
            }
            run += h[k];
        }
        s_sel[0] = d;
        s_sel[1] = above;
    }
}

// Sequences up to this length keep their keys in LDS through the selection
// (4 bytes each: 128 KB at the limit, with the bitsets and the histogram
// copies within the CU's 160 KB); longer ones read them from memory per pass.
constexpr int kEvictKeysLds = 32768;
constexpr int kEvictUnroll = 8;     // positions per thread in flight in the load pass
// Short sequences run in 512-thread workgroups: the phase barriers and the
// block scans span eight waves instead of sixteen (64 x 512: 11.1 -> 10.5 us)
constexpr int kEvictSmallL = 2048;
constexpr int kEvictSmallThreads = 512;
constexpr int kPassUnroll = 4;      // positions per thread per step of the LDS passes

// The lowest r set bits of x (r >= 0).
__device__ __forceinline__ uint32_t lowest_set_bits(uint32_t x, int r) {
    uint32_t y = x;
    for (int j = 0; j < r && y; ++j) y &= y - 1;
    return x ^ y;
}

template <bool KEYS_LDS, int NT>
__global__ __launch_bounds__(NT) void evict_kernel(
    int L, const float *__restrict__ conf, const int32_t *__restrict__ quota,
    const int32_t *__restrict__ pos, int n, uint8_t *__restrict__ cached, uint8_t *__restrict__ mask,
    int32_t *__restrict__ next_pos, int32_t *__restrict__ count, int32_t *__restrict__ evicted) {
    // dynamic LDS: cached bits (kept bits once decided), mask bits (the next
    // mask once decided), then the keys (0 for an uncached position)
    extern __shared__ uint32_t cbits[];
    // the selection histogram; afterwards the at-threshold bits, then the
    // per-word prefix of the next mask
    constexpr int NW = NT / kWave;
    __shared__ int hist[kHistCopies * kHistStride];
    __shared__ int tmp[3][NW];                         // one per scan
    __shared__ int s_sel[2];                           // the digit found, the count above it
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int q = quota[b];
    const int64_t rowoff = (int64_t)b * L;
    const int words = (L + 31) >> 5;
    uint32_t *mbits = cbits + words;
    uint32_t *keys = mbits + words;
    uint32_t *abits = reinterpret_cast<uint32_t *>(hist);
    const float *cf = conf + rowoff;
    const uint8_t *cr = cached + rowoff;
    const uint8_t *mr = mask + rowoff;
    const bool all_fresh = !pos && n == L;             // every position recomputed

    for (int k = tid; k < kHistCopies * kHistStride; k += NT) hist[k] = 0;
    // load pass: cached and mask flags as bits (a wave's ballot over 64
    // positions is two words) and the keys; kEvictUnroll loads per thread
    // are issued before their results are used
    for (int i0 = 0; i0 < L; i0 += NT * kEvictUnroll) {
        uint8_t cv[kEvictUnroll], mv[kEvictUnroll];
        float fv[kEvictUnroll];
#pragma unroll
        for (int u = 0; u < kEvictUnroll; ++u) {
            const int i = i0 + u * NT + tid;
            cv[u] = i < L ? (all_fresh ? 1 : cr[i]) : 0;
            mv[u] = i < L ? mr[i] : 0;
            if (KEYS_LDS) fv[u] = i < L ? cf[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kEvictUnroll; ++u) {
            const int c0 = i0 + u * NT;
            const int i = c0 + tid;
            const uint64_t bc = __ballot(cv[u] != 0);
            const uint64_t bm = __ballot(mv[u] != 0);
            const int w0 = (c0 + wave * kWave) >> 5;
            if (lane == 0 && w0 < words) { cbits[w0] = (uint32_t)bc; mbits[w0] = (uint32_t)bm; }
            if (lane == 1 && w0 + 1 < words) {
                cbits[w0 + 1] = (uint32_t)(bc >> 32);
                mbits[w0 + 1] = (uint32_t)(bm >> 32);
            }
            if (KEYS_LDS && i < L) keys[i] = conf_key(fv[u]);
        }
    }
    __syncthreads();
    // this step's recomputed positions hold fresh K/V.  The lanes of a wave
    // whose positions share a bitset word (runs of a sorted list) OR their
    // bits together first, so that one atomic per word and wave is issued.
    if (pos) {
        for (int j0 = 0; j0 < n; j0 += NT) {
            const int j = j0 + tid;
            const int p = j < n ? pos[(int64_t)b * n + j] : -1;
            const bool ok = p >= 0 && p < L;
            const int w = ok ? p >> 5 : -1;
            uint32_t v = ok ? 1u << (p & 31) : 0u;
            const int wprev = __shfl_up(w, 1, kWave);
            const bool head = lane == 0 || !ok || w != wprev;
            const uint64_t heads = __ballot(head);
            const int seg = __popcll(heads & ((2ull << lane) - 1ull));   // heads at or below the lane
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const uint32_t ov = __shfl_down(v, d, kWave);
                const int os = __shfl_down(seg, d, kWave);
                if (lane + d < kWave && os == seg) v |= ov;
            }
            if (head && ok) atomicOr(&cbits[w], v);
        }
        __syncthreads();
    }
    auto is_cached = [&](int i) { return (cbits[i >> 5] >> (i & 31)) & 1u; };
    // the key of a cached position; 0 (below every key of a float that is
    // not NaN) for an uncached one
    auto key_of = [&](int i) { return KEYS_LDS ? keys[i] : (is_cached(i) ? conf_key(cf[i]) : 0u); };
    int nc = 0;
    for (int i0 = 0; i0 < L; i0 += NT * kPassUnroll) {
        bool c[kPassUnroll];
#pragma unroll
        for (int u = 0; u < kPassUnroll; ++u) {
            const int i = i0 + u * NT + tid;
            c[u] = i < L && is_cached(i);
            if (KEYS_LDS && i < L && !c[u]) keys[i] = 0;
        }
#pragma unroll
        for (int u = 0; u < kPassUnroll; ++u) {
            if (i0 + u * NT >= L) break;                // uniform over the workgroup
            const uint64_t bal = __ballot(c[u]);
            if (lane == 0) nc += __popcll(bal);
        }
    }
    int nc_total;
    block_exclusive_scan<NW>(nc, lane, wave, tmp[0], nc_total);   // also: keys and hist settled
    nc = nc_total;
    const bool select = q >= 0 && nc > q;

    // radix select of the q-th largest key among the cached positions: the
    // threshold key T, and how many positions at T stay (`need`)
    uint32_t prefix = 0;
    int need = q;
    if (select) {
        uint32_t pmask = 0;
        int *my_hist = hist + (lane & (kHistCopies - 1)) * kHistStride;
        for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll 4
            for (int i = tid; i < L; i += NT) {
                const uint32_t key = key_of(i);
                if (key && (key & pmask) == prefix) atomicAdd(&my_hist[(key >> shift) & 255], 1);
            }
            __syncthreads();
            if (wave == 0) select_digit(hist, need, lane, s_sel);
            __syncthreads();
            prefix |= (uint32_t)s_sel[0] << shift;
            pmask |= 255u << shift;
            need -= s_sel[1];
        }
        // the positions above T (in place of the cached bits: a wave reads and
        // writes only the two words of its own 64 positions) and at T
        for (int i0 = 0; i0 < L; i0 += NT * kPassUnroll) {
            uint32_t kk[kPassUnroll];
#pragma unroll
            for (int u = 0; u < kPassUnroll; ++u) {
                const int i = i0 + u * NT + tid;
                kk[u] = i < L ? key_of(i) : 0u;
            }
#pragma unroll
            for (int u = 0; u < kPassUnroll; ++u) {
                if (i0 + u * NT >= L) break;            // uniform over the workgroup
                const uint64_t ba = __ballot(kk[u] > prefix);
                const uint64_t bt = __ballot(kk[u] != 0 && kk[u] == prefix);
                const int w0 = (i0 + u * NT + wave * kWave) >> 5;
                if (lane == 0 && w0 < words) { cbits[w0] = (uint32_t)ba; abits[w0] = (uint32_t)bt; }
                if (lane == 1 && w0 + 1 < words) {
                    cbits[w0 + 1] = (uint32_t)(ba >> 32);
                    abits[w0 + 1] = (uint32_t)(bt >> 32);
                }
            }
        }
        __syncthreads();
    }

    // each thread owns a run of whole words, in position order
    const int wpt = (words + NT - 1) / NT;
    const int w_lo = min(words, tid * wpt), w_hi = min(words, w_lo + wpt);
    if (select) {
        // the first `need` positions at T (position order) stay
        int n_at = 0;
        for (int w = w_lo; w < w_hi; ++w) n_at += __popc(abits[w]);
        int unused;
        int at_off = block_exclusive_scan<NW>(n_at, lane, wave, tmp[1], unused);
        for (int w = w_lo; w < w_hi; ++w) {
            const uint32_t aw = abits[w];
            const int r = max(0, min(need - at_off, __popc(aw)));
            cbits[w] |= lowest_set_bits(aw, r);
            at_off += __popc(aw);
        }
    }
    // every uncached position joins the mask
    int n_on = 0;
    for (int w = w_lo; w < w_hi; ++w) {
        const int valid = min(32, L - 32 * w);
        const uint32_t vmask = valid == 32 ? ~0u : ((1u << valid) - 1u);
        const uint32_t on = (mbits[w] | ~cbits[w]) & vmask;
        mbits[w] = on;
        n_on += __popc(on);
    }
    int n_total;
    int on_off = block_exclusive_scan<NW>(n_on, lane, wave, tmp[2], n_total);
    uint32_t *wpref = abits;                            // the at bits are used up
    for (int w = w_lo; w < w_hi; ++w) {
        wpref[w] = (uint32_t)on_off;
        on_off += __popc(mbits[w]);
    }
    __syncthreads();

    // store pass: flags and the compacted mask, four consecutive positions
    // per thread, so a wave's flag stores cover 256 contiguous bytes (whole
    // lines) instead of 64
    const bool al_c = (((uintptr_t)(cached + rowoff)) & 3u) == 0;
    const bool al_m = (((uintptr_t)(mask + rowoff)) & 3u) == 0;
#pragma unroll 2
    for (int i = 4 * tid; i < L; i += 4 * NT) {
        const int w = i >> 5, sh = i & 31;             // the four positions share word w
        const uint32_t mw = mbits[w];
        const uint32_t m4 = (mw >> sh) & 0xFu;
        store_flags4(cached + rowoff + i, (cbits[w] >> sh) & 0xFu, L - i, al_c);
        store_flags4(mask + rowoff + i, m4, L - i, al_m);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if ((m4 >> k) & 1u) next_pos[rowoff + wpref[w] + __popc(mw & ((1u << (sh + k)) - 1u))] = i + k;
    }
    for (int i = n_total + tid; i < L; i += NT) next_pos[rowoff + i] = -1;
    if (tid == 0) {
        count[b] = n_total;
        if (evicted) evicted[b] = select ? nc - q : 0;
    }
}

}  // namespace

int launch_evict(int B, int L, const float *conf, const int32_t *quota, const int32_t *pos, int n,
                 uint8_t *cached, uint8_t *mask, int32_t *next_pos, int32_t *count, int32_t *evicted,
                 hipStream_t s) {
    if (L > kMaxL) return DLLM_ERANGE;
    // two bitsets (cached, mask), then the keys when they fit
    const size_t bits = 2 * sizeof(uint32_t) * (size_t)((L + 31) / 32);
    if (L <= kEvictSmallL)
        evict_kernel<true, kEvictSmallThreads><<<dim3((unsigned)B), dim3(kEvictSmallThreads),
                                                 bits + sizeof(uint32_t) * (size_t)L, s>>>(
            L, conf, quota, pos, n, cached, mask, next_pos, count, evicted);
    else if (L <= kEvictKeysLds)
        evict_kernel<true, kThreads><<<dim3((unsigned)B), dim3(kThreads), bits + sizeof(uint32_t) * (size_t)L, s>>>(
            L, conf, quota, pos, n, cached, mask, next_pos, count, evicted);
    else
        evict_kernel<false, kThreads><<<dim3((unsigned)B), dim3(kThreads), bits, s>>>(
            L, conf, quota, pos, n, cached, mask, next_pos, count, evicted);
    return launch_status();
}

int launch_stability_reset(int B, int L, int D, int32_t *ring_argmax, float *ring_maxprob,
                           int32_t *ring_step, float *entropy_latest, int32_t *t_write,
                           uint8_t *stable, hipStream_t s) {
    const int64_t n = (int64_t)B * L, ring_n = n * D;
    const unsigned blocks = (unsigned)std::min<int64_t>(cdiv64(ring_n, 256), 4096);
    stability_reset_kernel<<<blocks, 256, 0, s>>>(ring_n, n, ring_argmax, ring_maxprob, ring_step,
                                                  entropy_latest, t_write, stable);
    return launch_status();
}

int launch_stability(int B, int L, int step, int32_t *step_dev, const int32_t *pos, int n,
                     const int32_t *argmax,
                     const float *maxprob, const float *entropy, int32_t *ring_argmax,
                     float *ring_maxprob, int32_t *ring_step, float *entropy_latest,
                     int32_t *t_write, uint8_t *stable, const dllm_stab_params &prm, double hmax,
                     uint8_t *mask, float *conf, int32_t *next_pos, int32_t *count,
                     uint8_t *all_stable, hipStream_t s) {
    if (L > kMaxL) return DLLM_ERANGE;
    const int words = cdiv(L, kThreads) * (kThreads / 32);   // whole 1024-position chunks
    const size_t shmem = sizeof(uint32_t) * (size_t)words;
    auto go = [&](auto all) {
        stability_kernel<decltype(all)::value><<<dim3((unsigned)B), dim3(kThreads), shmem, s>>>(
            B, L, step, step_dev, prm.advance_step, pos, n, argmax, maxprob, entropy, ring_argmax, ring_maxprob,
            ring_step, entropy_latest, t_write, stable, prm.K, prm.D, prm.R, prm.R_early, prm.T_steps,
            prm.refresh_every, prm.tau, prm.alpha, prm.beta,
            prm.decay, prm.n_decay, prm.conf_thresh, hmax, mask, conf, next_pos, count, all_stable);
    };
    if (!pos && n == L && L <= 2 * kThreads) go(std::true_type{});
    else go(std::false_type{});
    return launch_status();
}

}  // namespace dllm
