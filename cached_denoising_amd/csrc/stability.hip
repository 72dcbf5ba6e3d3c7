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
// The decisions (mean > tau, conf < threshold) are taken in float64.
//
// Also the budgeted cache of Flash-dLLM 3.3 and 5.2: per sequence, the
// cached positions beyond its quota leave the cache lowest confidence first,
// and every position without cached K/V joins the next step's mask.
#include "common.hpp"

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

__global__ __launch_bounds__(kThreads) void stability_kernel(
    int B, int L, int step_arg, int32_t *__restrict__ step_dev, int advance, const int32_t *__restrict__ pos, int n,
    const int32_t *__restrict__ argmax, const float *__restrict__ maxprob,
    const float *__restrict__ entropy, int32_t *__restrict__ ring_argmax,
    float *__restrict__ ring_maxprob, int32_t *__restrict__ ring_step,
    float *__restrict__ entropy_latest, int32_t *__restrict__ t_write,
    uint8_t *__restrict__ stable, int K, int D, int R, int R_early, int T_steps, int refresh_every,
    double tau, double alpha, double beta,
    double lambda, double conf_thresh, double hmax, uint8_t *__restrict__ mask,
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
        if (test && same && sum / (double)K > tau) stable[rowoff + p] = 1;
    }
    __syncthreads();

    // 3-4a: confidence and the seed bit of every position (one per thread)
    for (int i0 = 0; i0 < L; i0 += kThreads) {
        const int i = i0 + tid;
        bool seed = false;
        if (i < L) {
            const double h = (double)entropy_latest[rowoff + i];
            const double dt = (double)(step - t_write[rowoff + i]);
            const bool st = stable[rowoff + i] != 0;
            const double cf = alpha * (1.0 - h / hmax) + beta * exp(-lambda * dt);
            if (conf) conf[rowoff + i] = (float)cf;
            seed = !st || cf < conf_thresh;
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

__global__ __launch_bounds__(kThreads) void evict_kernel(
    int L, const float *__restrict__ conf, const int32_t *__restrict__ quota,
    const int32_t *__restrict__ pos, int n, uint8_t *__restrict__ cached, uint8_t *__restrict__ mask,
    int32_t *__restrict__ next_pos, int32_t *__restrict__ count, int32_t *__restrict__ evicted) {
    extern __shared__ uint32_t cbits[];                // cached, then kept: one bit per position each
    __shared__ int hist[256];
    __shared__ int wave_cnt[kWaves];
    __shared__ int s_sel[2];                           // the digit found, the count above it
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int64_t rowoff = (int64_t)b * L;
    const int words = (L + 31) >> 5;
    uint32_t *kbits = cbits + words;
    const float *cf = conf + rowoff;

    // the cached flags as bits: a wave's ballot over 64 positions is two words
    for (int i0 = 0; i0 < L; i0 += kThreads) {
        const int i = i0 + tid;
        const uint64_t bal = __ballot(i < L && cached[rowoff + i] != 0);
        const int w0 = (i0 + wave * kWave) >> 5;
        if (lane == 0 && w0 < words) { cbits[w0] = (uint32_t)bal; kbits[w0] = 0; }
        if (lane == 1 && w0 + 1 < words) { cbits[w0 + 1] = (uint32_t)(bal >> 32); kbits[w0 + 1] = 0; }
    }
    __syncthreads();
    // this step's recomputed positions hold fresh K/V
    for (int j = tid; j < n; j += kThreads) {
        const int p = pos ? pos[(int64_t)b * n + j] : j;
        if (p >= 0 && p < L) atomicOr(&cbits[p >> 5], 1u << (p & 31));
    }
    __syncthreads();
    auto is_cached = [&](int i) { return (cbits[i >> 5] >> (i & 31)) & 1u; };
    int nc = 0;
    for (int w = tid; w < words; w += kThreads) nc += __popc(cbits[w]);
    for (int o = 32; o >= 1; o >>= 1) nc += __shfl_xor(nc, o, kWave);
    if (lane == 0) wave_cnt[wave] = nc;
    __syncthreads();
    nc = 0;
    for (int w = 0; w < kWaves; ++w) nc += wave_cnt[w];
    __syncthreads();                                    // wave_cnt is reused
    const int q = quota[b];
    int ev = 0;

    if (q >= 0 && nc > q) {
        // radix select of the q-th largest key among the cached positions
        uint32_t prefix = 0, pmask = 0;
        int need = q;                                   // still to keep at or below the prefix
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int k = tid; k < 256; k += kThreads) hist[k] = 0;
            __syncthreads();
            for (int i = tid; i < L; i += kThreads) {
                if (!is_cached(i)) continue;
                const uint32_t key = conf_key(cf[i]);
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
            }
            __syncthreads();
            if (tid == 0) {
                int above = 0, d = 255;
                for (; d > 0; --d) {
                    if (above + hist[d] >= need) break;
                    above += hist[d];
                }
                s_sel[0] = d;
                s_sel[1] = above;
            }
            __syncthreads();
            prefix |= (uint32_t)s_sel[0] << shift;
            pmask |= 255u << shift;
            need -= s_sel[1];
            __syncthreads();                            // s_sel and hist are reused
        }
        // prefix = T; keep keys above T, and the first `need` positions at T
        int base = 0;
        for (int i0 = 0; i0 < L; i0 += kThreads) {
            const int i = i0 + tid;
            uint32_t key = 0;
            bool c = false;
            if (i < L) {
                c = is_cached(i) != 0;
                key = c ? conf_key(cf[i]) : 0u;
            }
            const bool at = c && key == prefix;
            const uint64_t bal = __ballot(at);
            if (lane == 0) wave_cnt[wave] = __popcll(bal);
            __syncthreads();
            int off = base;
            for (int w = 0; w < wave; ++w) off += wave_cnt[w];
            int chunk = 0;
            for (int w = 0; w < kWaves; ++w) chunk += wave_cnt[w];
            const uint64_t below = lane ? (bal & ((~0ull) >> (64 - lane))) : 0ull;
            const bool keep = c && (key > prefix || (at && off + __popcll(below) < need));
            if (keep) atomicOr(&kbits[i >> 5], 1u << (i & 31));
            if (c && !keep) ++ev;
            base += chunk;
            __syncthreads();                            // wave_cnt is reused
        }
    } else {
        for (int w = tid; w < words; w += kThreads) kbits[w] = cbits[w];
    }
    __syncthreads();

    // the uncached positions join the mask; ascending compaction
    int base = 0;
    for (int i0 = 0; i0 < L; i0 += kThreads) {
        const int i = i0 + tid;
        bool on = false;
        if (i < L) {
            const bool kept = (kbits[i >> 5] >> (i & 31)) & 1u;
            cached[rowoff + i] = kept ? 1 : 0;
            on = mask[rowoff + i] != 0 || !kept;
            mask[rowoff + i] = on ? 1 : 0;
        }
        const uint64_t bal = __ballot(on);
        if (lane == 0) wave_cnt[wave] = __popcll(bal);
        __syncthreads();
        int off = base;
        for (int w = 0; w < wave; ++w) off += wave_cnt[w];
        int chunk = 0;
        for (int w = 0; w < kWaves; ++w) chunk += wave_cnt[w];
        if (on) {
            const uint64_t below = lane ? (bal & ((~0ull) >> (64 - lane))) : 0ull;
            next_pos[rowoff + off + __popcll(below)] = i;
        }
        base += chunk;
        __syncthreads();
    }
    for (int i = base + tid; i < L; i += kThreads) next_pos[rowoff + i] = -1;
    // the evicted count: a sum over the threads in a fixed order
    for (int o = 32; o >= 1; o >>= 1) ev += __shfl_xor(ev, o, kWave);
    if (lane == 0) wave_cnt[wave] = ev;
    __syncthreads();
    if (tid == 0) {
        int tot = 0;
        for (int w = 0; w < kWaves; ++w) tot += wave_cnt[w];
        count[b] = base;
        if (evicted) evicted[b] = tot;
    }
}

}  // namespace

int launch_evict(int B, int L, const float *conf, const int32_t *quota, const int32_t *pos, int n,
                 uint8_t *cached, uint8_t *mask, int32_t *next_pos, int32_t *count, int32_t *evicted,
                 hipStream_t s) {
    if (L > kMaxL) return DLLM_ERANGE;
    const size_t shmem = 2 * sizeof(uint32_t) * (size_t)((L + 31) / 32);
    evict_kernel<<<dim3((unsigned)B), dim3(kThreads), shmem, s>>>(L, conf, quota, pos, n, cached, mask,
                                                                  next_pos, count, evicted);
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
    stability_kernel<<<dim3((unsigned)B), dim3(kThreads), shmem, s>>>(
        B, L, step, step_dev, prm.advance_step, pos, n, argmax, maxprob, entropy, ring_argmax, ring_maxprob, ring_step,
        entropy_latest, t_write, stable, prm.K, prm.D, prm.R, prm.R_early, prm.T_steps,
        prm.refresh_every, prm.tau, prm.alpha, prm.beta,
        prm.lambda, prm.conf_thresh, hmax, mask, conf, next_pos, count, all_stable);
    return launch_status();
}

}  // namespace dllm
