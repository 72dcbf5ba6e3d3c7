// Vocab statistics: for every row of logits, the argmax token (lowest index
// wins ties), the largest softmax probability and the entropy, in one pass
// over the row.  [SWD page, 3.1 and 4.2: per-position max probability and
// its token; Flash-dLLM page, 3.1: entropy of the step's distribution.]
//
// One workgroup of 256 threads (512 when there are too few rows to fill the
// chip) streams one row, or one contiguous split of a row when there are very
// few rows, with non-temporal 16-byte loads.  The loop is software-pipelined:
// each thread keeps the next step's loads (three or two 16-byte vectors) in
// flight while it folds the current ones, so a wave never waits on memory
// with nothing issued.  The few
// elements before the first 16-byte boundary and after the last are peeled
// off.  Each thread keeps an online state over base-2 exponents
// a_j = (x_j - m) log2(e):
//     m = max,  s = sum 2^a_j,  t = sum 2^a_j a_j,  idx = argmax
// so that  maxprob = 1/s  and  entropy = ln s - ln2 * t / s.  In the main
// loop m is a reference up to 8 below the max (terms up to e^8), and the
// state is taken to the max once at the end; the entropy does not depend on
// the reference, 1/s does.  States merge in a fixed order (wave butterfly,
// then the waves in order, then splits), so the result is bitwise
// reproducible.  The probabilities never touch memory.
#include "common.hpp"

#include <climits>

namespace dllm {
namespace {

// 16-byte loads per thread per step (two steps in flight): three in the
// 256-thread form (at gpt2's 8192 rows 127.7 -> 125.6 us between event pairs
// and the decode step 1.5 % faster, though 131.8 -> 135.3 us back to back;
// four needed 143 VGPRs and ran slower), two in the 512-thread form (the
// 512-row LLaDA block: three measured 25.0 -> 26.1 us)
template <int kThreads> struct VocabUnroll { static constexpr int value = kThreads == 256 ? 3 : 2; };
constexpr float kNegInf = -__builtin_inff();
// In the main loop the exponents are taken against a reference max that moves
// only when a step's max exceeds it by more than this (natural units): terms
// then stay below e^8, and the rescale is rare instead of taken by some lane
// of the wave on almost every step
constexpr float kLazyRef = 8.0f;

struct Acc {
    float m, s, t;
    int idx;
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// streaming 16-byte load: the logits are read once, so keep them out of the caches' way
__device__ __forceinline__ uint4 load_stream(const uint4 *p) {
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ Acc acc_empty() { return Acc{kNegInf, 0.f, 0.f, INT_MAX}; }

// merge b into a; a tie in the max keeps the lower index
__device__ __forceinline__ void acc_merge(Acc &a, const Acc &b) {
    const float m = fmaxf(a.m, b.m);
    int idx;
    if (a.m > b.m) idx = a.idx;
    else if (b.m > a.m) idx = b.idx;
    else idx = min(a.idx, b.idx);
    float s = 0.f, t = 0.f;
    if (a.s > 0.f) {
        const float d = (a.m - m) * kLog2e;
        const float f = exp2f(d);
        s += a.s * f;
        t += f * (a.t + a.s * d);
    }
    if (b.s > 0.f) {
        const float d = (b.m - m) * kLog2e;
        const float f = exp2f(d);
        s += b.s * f;
        t += f * (b.t + b.s * d);
    }
    a = Acc{m, s, t, idx};
}

// Add the terms 2^a and 2^a a of NE logits, a = (x - m) log2(e), to s and t
// (m finite).  A -inf logit gives 0 * -inf = NaN in t; such terms add
// nothing, so the logits are then summed again without them.
template <int NE>
__device__ __forceinline__ void fold_sums(const float (&x)[NE], float m, float &s, float &t) {
    const float mL = m * kLog2e;
    float s0 = 0.f, s1 = 0.f, t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int e = 0; e < NE; e += 2) {
        const float a0 = fmaf(x[e], kLog2e, -mL);
        const float p0 = __builtin_amdgcn_exp2f(a0);
        s0 += p0;
        t0 = fmaf(p0, a0, t0);
        if (e + 1 < NE) {
            const float a1 = fmaf(x[e + 1], kLog2e, -mL);
            const float p1 = __builtin_amdgcn_exp2f(a1);
            s1 += p1;
            t1 = fmaf(p1, a1, t1);
        }
    }
    float cs = s0 + s1, ct = t0 + t1;
    if (ct != ct) {
        // a -inf logit gave 0 * -inf; such terms add nothing, drop them
        cs = 0.f;
        ct = 0.f;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            if (x[e] != kNegInf) {
                const float a = fmaf(x[e], kLog2e, -mL);
                const float p = __builtin_amdgcn_exp2f(a);
                cs += p;
                ct = fmaf(p, a, ct);
            }
        }
    }
    s += cs;
    t += ct;
}

// Fold NE consecutive-in-thread-order elements into the state.  gidx(e)
// gives element e's column; columns increase with e.
template <int NE, typename IdxFn>
__device__ __forceinline__ void consume(Acc &st, const float (&x)[NE], IdxFn gidx) {
    // IEEE maximum: a NaN logit would propagate, but logits are finite or
    // -inf, where it equals fmaxf; on gfx950 it is a v_maximum3_f32 chain
    // without fmaxf's canonicalising moves
    float cm = x[0];
#pragma unroll
    for (int e = 1; e < NE; ++e) cm = __builtin_elementwise_maximum(cm, x[e]);
    if (cm >= st.m && cm != kNegInf) {
        int first = NE - 1;
#pragma unroll
        for (int e = NE - 1; e >= 0; --e)
            if (x[e] == cm) first = e;
        const int gi = gidx(first);
        if (cm > st.m) {
            if (st.s > 0.f) {                    // rescale to the new max
                const float d = (st.m - cm) * kLog2e;
                const float f = __builtin_amdgcn_exp2f(d);
                st.t = f * (st.t + st.s * d);
                st.s *= f;
            }
            st.m = cm;
            st.idx = gi;
        } else if (gi < st.idx) {
            st.idx = gi;
        }
    }
    if (st.m == kNegInf) return;                 // nothing finite seen yet
    fold_sums<NE>(x, st.m, st.s, st.t);
}

template <int DT> struct Elem;
template <> struct Elem<DLLM_F32> {
    typedef float T;
    static constexpr int kVec = 4;
    __device__ static void unpack(const uint4 &w, float *x) {
        x[0] = __uint_as_float(w.x);
        x[1] = __uint_as_float(w.y);
        x[2] = __uint_as_float(w.z);
        x[3] = __uint_as_float(w.w);
    }
    __device__ static float scalar(const T *p) { return *p; }
};
template <> struct Elem<DLLM_BF16> {
    typedef uint16_t T;
    static constexpr int kVec = 8;
    __device__ static void unpack(const uint4 &w, float *x) {
        x[0] = bf16lo(w.x); x[1] = bf16hi(w.x);
        x[2] = bf16lo(w.y); x[3] = bf16hi(w.y);
        x[4] = bf16lo(w.z); x[5] = bf16hi(w.z);
        x[6] = bf16lo(w.w); x[7] = bf16hi(w.w);
    }
    __device__ static float scalar(const T *p) { return bf16_to_f32(*p); }
};

__device__ __forceinline__ void write_stats(const Acc &a, int64_t row, int32_t *argmax,
                                            float *maxprob, float *entropy) {
    argmax[row] = a.idx == INT_MAX ? 0 : a.idx;
    maxprob[row] = 1.0f / a.s;
    entropy[row] = logf(a.s) - kLn2 * a.t / a.s;
}

template <int DT, int kThreads>
__global__ __launch_bounds__(kThreads) void vocab_stats_kernel(
    const typename Elem<DT>::T *__restrict__ logits, int64_t V, int64_t stride, int64_t chunk,
    int splits, int32_t *__restrict__ argmax, float *__restrict__ maxprob,
    float *__restrict__ entropy, float4 *__restrict__ partial) {
    typedef Elem<DT> E;
    constexpr int kVec = E::kVec;
    constexpr int kUnroll = VocabUnroll<kThreads>::value;
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x / splits;
    const int split = blockIdx.x - (int)(row * splits);
    const int64_t j0 = (int64_t)split * chunk;
    const int64_t j1 = min(V, j0 + chunk);
    const typename E::T *rp = logits + row * stride;

    Acc st = acc_empty();
    if (j0 < j1) {
        // aligned body [a0, a1) of whole 16-byte vectors
        const uintptr_t addr = (uintptr_t)(rp + j0);
        const int64_t mis = (int64_t)(((16u - (unsigned)(addr & 15u)) & 15u) / sizeof(typename E::T));
        const int64_t a0 = min(j1, j0 + mis);
        const int64_t nvec = (j1 - a0) / kVec;
        const int64_t a1 = a0 + nvec * kVec;
        // peeled elements: [j0, a0) and [a1, j1), fewer than 2*kVec; the
        // load goes first so that it is not waited for on its own
        const int64_t nhead = a0 - j0, ntail = j1 - a1;
        const bool peel = tid < nhead + ntail;
        const int64_t jp = tid < nhead ? j0 + tid : a1 + (tid - nhead);
        float xp[1] = {0.f};
        if (peel) xp[0] = E::scalar(rp + jp);

        const uint4 *vp = reinterpret_cast<const uint4 *>(rp + a0);
        constexpr unsigned kStep = kUnroll * kThreads;       // vectors per step
        const int steps = (int)(nvec / kStep);               // full steps, uniform
        // loads at 32-bit byte offsets from the row's wave-uniform base (a row
        // spans less than 4 GiB): no 64-bit address per lane and load
        const unsigned char *vb = reinterpret_cast<const unsigned char *>(vp);
        auto issue = [&](uint4 (&w)[kUnroll], unsigned o) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                w[u] = load_stream(reinterpret_cast<const uint4 *>(vb + (o + u * kThreads) * 16u));
        };
        // The main loop keeps a lazy state: sums lm_s, lm_t against the
        // reference lm, and the step with the first maximum so far (its max
        // bm and offset bo by selects, its raw vectors in this thread's LDS
        // slot, stored under the lanes' record mask).  The position of the
        // maximum within that step is found once after the loop, and the sums
        // are then taken to bm: the state the per-step form keeps, without
        // its position scan and rescale, which some lane of the wave needed on
        // almost every step.
        constexpr int NE = kUnroll * kVec;
        float lm = kNegInf, lm_s = 0.f, lm_t = 0.f, bm = kNegInf;
        unsigned bo = 0;
        __shared__ uint4 s_bw[kUnroll][kThreads];     // the recorded step's raw vectors, per thread
        auto fold = [&](const uint4 (&w)[kUnroll], unsigned o) {
            float x[NE];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) E::unpack(w[u], x + u * kVec);
            // IEEE maximum (v_maximum3_f32, no canonicalising moves): logits
            // are finite or -inf, where it equals fmaxf
            float cm = x[0];
#pragma unroll
            for (int e = 1; e < NE; ++e) cm = __builtin_elementwise_maximum(cm, x[e]);
            // a later step with an equal max keeps the earlier one (lower positions)
            const bool rec = cm > bm;
            bm = rec ? cm : bm;
            bo = rec ? o : bo;
            if (rec) {
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) s_bw[u][tid] = w[u];
            }
            if (cm > lm + kLazyRef) {                    // also the first finite step (lm = -inf)
                if (lm_s > 0.f) {
                    const float d = (lm - cm) * kLog2e;
                    const float f = __builtin_amdgcn_exp2f(d);
                    lm_t = f * (lm_t + lm_s * d);
                    lm_s *= f;
                }
                lm = cm;
            }
            if (lm != kNegInf) fold_sums<NE>(x, lm, lm_s, lm_t);
        };
        // two register buffers: step i+1 is in flight while step i is folded
        uint4 wa[kUnroll], wb[kUnroll];
        unsigned off = tid;
        if (steps > 0) issue(wa, off);
        int i = 0;
        for (; i + 2 <= steps; i += 2) {
            issue(wb, off + kStep);
            fold(wa, off);
            if (i + 2 < steps) issue(wa, off + 2 * kStep);
            fold(wb, off + kStep);
            off += 2 * kStep;
        }
        if (i < steps) {
            fold(wa, off);
            off += kStep;
        }
        if (bm != kNegInf) {
            // the first position of the maximum in the recorded step, and the
            // sums relative to the maximum (the max term alone gives lm_s >= 1)
            float x[NE];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) E::unpack(s_bw[u][tid], x + u * kVec);
            int first = NE - 1;
#pragma unroll
            for (int e = NE - 1; e >= 0; --e)
                if (x[e] == bm) first = e;
            const int gi = (int)(a0 + (int64_t)(bo + (first / kVec) * kThreads) * kVec + (first % kVec));
            const float d = (lm - bm) * kLog2e;
            const float f = __builtin_amdgcn_exp2f(d);
            st = Acc{bm, lm_s * f, f * (lm_t + lm_s * d), gi};
        }
        if (peel) consume<1>(st, xp, [&](int) { return (int)jp; });
        // the rest: fewer than kStep vectors
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const unsigned v = off + u * kThreads;
            if (v < nvec) {
                const uint4 w = load_stream(vp + v);
                float x[kVec];
                E::unpack(w, x);
                consume<kVec>(st, x, [&](int e) { return (int)(a0 + (int64_t)v * kVec + e); });
            }
        }
    }

    // the wave: its max, every lane's sums taken to it (one exponential per
    // lane), then butterfly sums and the lowest index among the lanes at the
    // max (every lane ends with the same values); then the waves in order
    {
        float wm = st.m;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) wm = fmaxf(wm, shfl_xor_f(wm, o));
        float ws = 0.f, wt = 0.f;
        if (st.s > 0.f) {
            const float d = (st.m - wm) * kLog2e;
            const float f = exp2f(d);
            ws = st.s * f;
            wt = f * (st.t + st.s * d);
        }
        int wi = st.m == wm ? st.idx : INT_MAX;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            ws += shfl_xor_f(ws, o);
            wt += shfl_xor_f(wt, o);
            wi = min(wi, shfl_xor_i(wi, o));
        }
        st = Acc{wm, ws, wt, wi};
    }
    __shared__ Acc waves[kThreads / kWave];
    if ((tid & (kWave - 1)) == 0) waves[tid / kWave] = st;
    __syncthreads();
    if (tid == 0) {
        Acc r = waves[0];
#pragma unroll
        for (int w = 1; w < kThreads / kWave; ++w) acc_merge(r, waves[w]);
        if (splits == 1)
            write_stats(r, row, argmax, maxprob, entropy);
        else
            partial[blockIdx.x] = make_float4(r.m, r.s, r.t, __int_as_float(r.idx));
    }
}

__global__ __launch_bounds__(256) void vocab_merge_kernel(const float4 *__restrict__ partial,
                                                          int64_t N, int splits,
                                                          int32_t *__restrict__ argmax,
                                                          float *__restrict__ maxprob,
                                                          float *__restrict__ entropy) {
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= N) return;
    const float4 *p = partial + row * splits;
    Acc r = acc_empty();
    for (int i = 0; i < splits; ++i) {
        const float4 q = p[i];
        acc_merge(r, Acc{q.x, q.y, q.z, __float_as_int(q.w)});
    }
    write_stats(r, row, argmax, maxprob, entropy);
}

}  // namespace

VocabPlan plan_vocab(int64_t N, int64_t V) {
    VocabPlan p;
    // 256-thread workgroups take one row each once the rows fill a round of
    // the chip (6 resident per CU); with fewer rows, 512-thread workgroups
    // keep more loads in flight per row (measured 25 vs 30 us on 512 rows of
    // 126464); below one row per CU the rows are split, with a merge pass.
    const int64_t cus = 256;
    p.threads = N >= 6 * cus ? 256 : 512;
    const int64_t target_blocks = cus;
    const int64_t min_chunk = 16384;        // elements per split, at least
    int64_t splits = N > 0 ? cdiv64(target_blocks, N) : 1;
    splits = std::max<int64_t>(1, std::min<int64_t>(splits, cdiv64(V, min_chunk)));
    int64_t chunk = cdiv64(V, splits);
    chunk = cdiv64(chunk, 8) * 8;
    splits = cdiv64(V, chunk);
    p.splits = (int)splits;
    p.chunk = chunk;
    p.ws_bytes = splits > 1 ? (size_t)(N * splits) * sizeof(float4) : 0;
    return p;
}

int launch_vocab(const void *logits, int dtype, int64_t N, int64_t V, int64_t stride,
                 int32_t *argmax, float *maxprob, float *entropy, const VocabPlan &p, void *ws,
                 hipStream_t s) {
    if (N == 0) return DLLM_OK;
    const int64_t blocks = N * p.splits;
    if (blocks > INT_MAX) return DLLM_ERANGE;
    float4 *partial = static_cast<float4 *>(ws);
#define DLLM_VOCAB(DT, TT, T)                                                                     \
    vocab_stats_kernel<DT, T><<<dim3((unsigned)blocks), dim3(T), 0, s>>>(                         \
        static_cast<const TT *>(logits), V, stride, p.chunk, p.splits, argmax, maxprob, entropy, \
        partial)
    if (dtype == DLLM_BF16) {
        if (p.threads == 256) DLLM_VOCAB(DLLM_BF16, uint16_t, 256);
        else DLLM_VOCAB(DLLM_BF16, uint16_t, 512);
    } else {
        if (p.threads == 256) DLLM_VOCAB(DLLM_F32, float, 256);
        else DLLM_VOCAB(DLLM_F32, float, 512);
    }
#undef DLLM_VOCAB
    int rc = launch_status();
    if (rc != DLLM_OK || p.splits == 1) return rc;
    vocab_merge_kernel<<<dim3((unsigned)cdiv64(N, 256)), dim3(256), 0, s>>>(partial, N, p.splits,
                                                                            argmax, maxprob,
                                                                            entropy);
    return launch_status();
}

}  // namespace dllm
