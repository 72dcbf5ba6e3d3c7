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
// The decisions (mean > tau, conf < threshold) are taken in float64.
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
    uint8_t *__restrict__ stable, int K, int D, int R, double tau, double alpha, double beta,
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

    // 4b-5: window test per position, then ascending compaction, 1024 at a time
    int base = 0;
    for (int i0 = 0; i0 < L; i0 += kThreads) {
        const int i = i0 + tid;
        bool on = false;
        if (i < L) {
            if (none) {
                on = true;
            } else {
                const int lo = max(0, i - R), hi = min(L - 1, i + R);
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

}  // namespace

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
        entropy_latest, t_write, stable, prm.K, prm.D, prm.R, prm.tau, prm.alpha, prm.beta,
        prm.lambda, prm.conf_thresh, hmax, mask, conf, next_pos, count, all_stable);
    return launch_status();
}

}  // namespace dllm
