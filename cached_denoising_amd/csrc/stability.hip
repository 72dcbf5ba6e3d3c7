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
constexpr int kMaxL = 131072;      // seed bits + counts stay within 32 KB of LDS
constexpr int kMaxWords = kMaxL / 32;

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
    int B, int L, int step, const int32_t *__restrict__ pos, int n,
    const int32_t *__restrict__ argmax, const float *__restrict__ maxprob,
    const float *__restrict__ entropy, int32_t *__restrict__ ring_argmax,
    float *__restrict__ ring_maxprob, int32_t *__restrict__ ring_step,
    float *__restrict__ entropy_latest, int32_t *__restrict__ t_write,
    uint8_t *__restrict__ stable, int K, int D, int R, double tau, double alpha, double beta,
    double lambda, double conf_thresh, double hmax, uint8_t *__restrict__ mask,
    float *__restrict__ conf, int32_t *__restrict__ next_pos, int32_t *__restrict__ count,
    uint8_t *__restrict__ all_stable) {
    extern __shared__ uint32_t seed_bits[];            // [words] seeds, then [words + 1] scan
    __shared__ int any_seed;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t rowoff = (int64_t)b * L;
    const int64_t plane = (int64_t)B * L;              // one ring slot
    const int slot = step % D;
    const int words = (L + 31) >> 5;
    uint32_t *scan = seed_bits + words;

    if (tid == 0) any_seed = 0;

    // 1-2: record this step and test the recomputed positions
    for (int j = tid; j < n; j += kThreads) {
        const int p = pos ? pos[(int64_t)b * n + j] : j;
        if (p < 0 || p >= L) continue;
        const int64_t src = (int64_t)b * n + j;
        const int64_t ri = slot * plane + rowoff + p;
        const int tok = argmax[src];
        ring_argmax[ri] = tok;
        ring_maxprob[ri] = maxprob[src];
        ring_step[ri] = step;
        entropy_latest[rowoff + p] = entropy[src];
        t_write[rowoff + p] = step;
        if (stable[rowoff + p] || step + 1 < K) continue;
        bool same = true;
        double sum = 0.0;
        for (int k = K - 1; k >= 0; --k) {             // oldest record first
            const int64_t rk = (int64_t)((step - k) % D) * plane + rowoff + p;
            if (ring_step[rk] != step - k || ring_argmax[rk] != tok) { same = false; break; }
            sum += (double)ring_maxprob[rk];
        }
        if (same && sum / (double)K > tau) stable[rowoff + p] = 1;
    }
    __syncthreads();

    // 3-4a: confidence and the seed bit of every position, 32 per word
    for (int w = tid; w < words; w += kThreads) {
        uint32_t bits = 0;
        const int i0 = w * 32;
        const int i1 = min(L, i0 + 32);
        for (int i = i0; i < i1; ++i) {
            const double h = (double)entropy_latest[rowoff + i];
            const double dt = (double)(step - t_write[rowoff + i]);
            const double cf = alpha * (1.0 - h / hmax) + beta * exp(-lambda * dt);
            if (conf) conf[rowoff + i] = (float)cf;
            if (!stable[rowoff + i] || cf < conf_thresh) bits |= 1u << (i - i0);
        }
        seed_bits[w] = bits;
        if (bits) any_seed = 1;
    }
    __syncthreads();
    const bool none = any_seed == 0;

    // 4b: window expansion, and the number of mask positions per word
    for (int w = tid; w < words; w += kThreads) {
        const int i0 = w * 32;
        uint32_t mbits = 0;
        if (none) {
            mbits = 0xffffffffu;
        } else {
            for (int e = 0; e < 32; ++e) {
                const int i = i0 + e;
                const int lo = max(0, i - R), hi = min(L - 1, i + R);
                if (lo > hi) continue;
                const int wl = lo >> 5, wh = hi >> 5;
                bool hit = false;
                for (int q = wl; q <= wh && !hit; ++q) {
                    uint32_t m = seed_bits[q];
                    if (q == wl) m &= 0xffffffffu << (lo & 31);
                    if (q == wh && (hi & 31) != 31) m &= (1u << ((hi & 31) + 1)) - 1u;
                    hit = m != 0;
                }
                if (hit) mbits |= 1u << e;
            }
        }
        const int i1 = min(L, i0 + 32);
        if (i1 - i0 < 32) mbits &= (1u << (i1 - i0)) - 1u;
        scan[w + 1] = mbits;                           // kept until the counts are scanned
    }
    __syncthreads();

    // 5: compaction.  Thread t owns words [t*per, (t+1)*per); an exclusive
    // scan of the per-thread counts gives each its first output slot.
    const int per = (words + kThreads - 1) / kThreads;
    const int w0 = tid * per, w1 = min(words, w0 + per);
    int local = 0;
    for (int w = w0; w < w1; ++w) local += __popc(scan[w + 1]);
    __shared__ int tsum[kThreads];
    tsum[tid] = local;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {     // Hillis-Steele inclusive scan
        const int v = tid >= off ? tsum[tid - off] : 0;
        __syncthreads();
        tsum[tid] += v;
        __syncthreads();
    }
    int out = tsum[tid] - local;
    for (int w = w0; w < w1; ++w) {
        const uint32_t mbits = scan[w + 1];
        const int i0 = w * 32;
        const int i1 = min(L, i0 + 32);
        for (int i = i0; i < i1; ++i) {
            const bool on = (mbits >> (i - i0)) & 1u;
            mask[rowoff + i] = on ? 1 : 0;
            if (on) next_pos[rowoff + out++] = i;
        }
    }
    const int total = tsum[kThreads - 1];
    for (int i = total + tid; i < L; i += kThreads) next_pos[rowoff + i] = -1;
    if (tid == 0) {
        count[b] = total;
        all_stable[b] = none ? 1 : 0;
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

int launch_stability(int B, int L, int step, const int32_t *pos, int n, const int32_t *argmax,
                     const float *maxprob, const float *entropy, int32_t *ring_argmax,
                     float *ring_maxprob, int32_t *ring_step, float *entropy_latest,
                     int32_t *t_write, uint8_t *stable, const dllm_stab_params &prm, double hmax,
                     uint8_t *mask, float *conf, int32_t *next_pos, int32_t *count,
                     uint8_t *all_stable, hipStream_t s) {
    if (L > kMaxL) return DLLM_ERANGE;
    const int words = (L + 31) / 32;
    const size_t shmem = sizeof(uint32_t) * (size_t)(2 * words + 1);
    stability_kernel<<<dim3((unsigned)B), dim3(kThreads), shmem, s>>>(
        B, L, step, pos, n, argmax, maxprob, entropy, ring_argmax, ring_maxprob, ring_step,
        entropy_latest, t_write, stable, prm.K, prm.D, prm.R, prm.tau, prm.alpha, prm.beta,
        prm.lambda, prm.conf_thresh, hmax, mask, conf, next_pos, count, all_stable);
    return launch_status();
}

}  // namespace dllm
