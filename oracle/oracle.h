/*
 * oracle.h -- plain, slow, obviously-correct CPU reference for one step of
 * cached masked-diffusion decoding.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link
 * or call this code: only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library; the two meet only at the seeded input generators.
 *
 * Everything is computed in IEEE binary64 (double), scalar, in the order the
 * pages state, with no FMA contraction and no fast-math.  Inputs are the
 * exact bytes the GPU reads: float32 as float, bfloat16 as raw uint16 bits,
 * OCP e4m3fn codes as uint8 with one float32 scale per 128-element group.
 *
 * Page titles used in citations:
 *   [SWD]     "Stable Window Decoding (SWD)" blog page on temporal stability
 *             in diffusion-LM decoding (wmrh.cn/news/51151)
 *   [LaCache] "LaCache: Exact Caching and Precision-Adaptive Inference for
 *             Diffusion Large Language Models" (gist.science explainer)
 *   [Sinks]   "Attention sinks and the rolling K/V cache" blog page on GPT-2
 *             (wmrh.cn/news/159578)
 *   [Flash]   "Diffusion-LM inference acceleration: I/O-aware KV cache and
 *             self-verifying parallel decoding" (Flash-dLLM, bjdmk.com.cn)
 *
 * Where the pages leave a step open, the plainest reading is taken and is
 * stated next to the function that takes it.
 */
#ifndef DLLM_ORACLE_H
#define DLLM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage codes, numerically equal to the library's but defined here anew */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3 = 2, ORC_F64 = 9 };

/* number of OpenMP threads used by the parallel loops; returns the count */
int oracle_set_threads(int n);
int oracle_get_threads(void);

/* ---- number formats --------------------------------------------------- */
/* bfloat16 bits -> exact value */
double oracle_bf16_value(uint16_t bits);
/* OCP e4m3fn code -> exact value (0x7f / 0xff are NaN) */
double oracle_e4m3_value(uint8_t code);
/* float32 -> OCP e4m3fn code, round to nearest, ties to even mantissa,
 * finite overflow saturates to +-448 [LaCache, Methodology 2: per-group FP8;
 * the pages give only the group shapes, so format and rounding are a reading] */
uint8_t oracle_e4m3_encode(float x);
/* quantize one group of n values: scale = amax/448 (float32 divide),
 * code_i = encode(x_i / scale) (float32 divide); amax == 0 -> scale 0, codes 0 */
void oracle_e4m3_quantize_group(const float *x, int n, uint8_t *codes, float *scale);

/* ---- A1: scatter fresh K/V rows into the persistent cache ---------------
 * [LaCache, Methodology 1 (RoPECache) and 3 (workflow)]; [SWD, 4.1/4.3
 * write-back of masked positions]; [Sinks, 3.2 fixed-size cache].
 * cache_k/cache_v: [B, Hkv, L, d] in cache_dtype; k_scale/v_scale:
 * [B, Hkv, L, d/128] float (e4m3 only).  k_new/v_new: [B, n, Hkv, d] in
 * src_dtype (== cache dtype for f32/bf16; f32 or bf16 for e4m3).
 * pos: [B, n] int32, unique per sequence, each in [0, L) or -1 (padding,
 * skipped).  Returns 0, or -1 on a bad argument (nothing written). */
int oracle_scatter_kv(int cache_dtype, int B, int L, int Hkv, int d,
                      void *cache_k, void *cache_v, float *k_scale, float *v_scale,
                      int src_dtype, const void *k_new, const void *v_new,
                      const int32_t *pos, int n);

/* ---- A2: sink + rolling key map [Sinks, 2.3 and 3.2] --------------------
 * keys = {0..S-1} followed by the newest R keys before `end`, i.e.
 * [max(S, end-R), end).  Writes at most S+R indices, returns the count. */
int oracle_sink_rolling_keys(int S, int R, int end, int32_t *key_idx);

/* ---- A3: block attention over the cache ---------------------------------
 * softmax(q . K^T * scale) V per query, bidirectional, over the selected
 * keys [Sinks, 2.1]; [LaCache, problem statement: bidirectional attention].
 * q: [B, Hq, b, d] in q_dtype (f32 or bf16); cache as in A1; key_idx:
 * [B, n_keys] or NULL (= 0..L-1, n_keys = L), an entry of -1 is padding
 * (no key; a row with only padding gets out = 0, lse = -inf); query head h reads KV head
 * h / (Hq/Hkv).  scale <= 0 -> 1/sqrt(d).  out: [B, Hq, b, d] double;
 * lse: [B, Hq, b] double (natural-log log-sum-exp of the scaled scores) or
 * NULL.  Optional head subset: when heads != NULL, only the n_heads listed
 * (b_idx, h) pairs are computed, packed in order into out/lse. */
int oracle_block_attention(int cache_dtype, int B, int L, int Hkv, int d,
                           const void *cache_k, const void *cache_v,
                           const float *k_scale, const float *v_scale,
                           int q_dtype, const void *q, int Hq, int b,
                           const int32_t *key_idx, int n_keys, double scale,
                           double *out, double *lse,
                           const int32_t *heads, int n_heads);

/* ---- N1: FACache merge [LaCache, Methodology 1 (FACache) and 3] --------
 * For queries whose memoized online-softmax state over the unchanged keys
 * is given, continue that state over the listed (changed) keys and
 * normalise.  The memo of a row is stored normalised: memo_o = O~/l and
 * memo_lse = m + ln l (natural log), i.e. the state (m, l, O~) with its
 * reference point moved to m' = memo_lse, l' = 1, O~' = memo_o; a row with
 * memo_lse = -inf has an empty memo (l' = 0, memo_o ignored).
 * Per query row, with s_j = scale * q . k_j over the listed keys:
 *   m_new = max(m', max_j s_j)
 *   l_new = l' e^(m' - m_new) + sum_j e^(s_j - m_new)
 *   O_new = O~' e^(m' - m_new) + sum_j e^(s_j - m_new) v_j
 *   out = O_new / l_new, lse = m_new + ln l_new (0 and -inf when l_new = 0).
 * q: [B, Hq, n_q, d]; memo_o: [B, Hq, n_q, d] float; memo_lse: [B, Hq, n_q]
 * float; key_idx, cache, scale, heads, out, lse as in A3 (b = n_q). */
int oracle_facache_merge(int cache_dtype, int B, int L, int Hkv, int d,
                         const void *cache_k, const void *cache_v,
                         const float *k_scale, const float *v_scale,
                         int q_dtype, const void *q, int Hq, int n_q,
                         const float *memo_o, const float *memo_lse,
                         const int32_t *key_idx, int n_keys, double scale,
                         double *out, double *lse,
                         const int32_t *heads, int n_heads);

/* ---- N2: per-group FP8 for the FFN [LaCache, Methodology 2] -------------
 * Activations are quantised in 1 x 128 groups, weights in 128 x 128 blocks,
 * each group with one power-of-two scale 2^e stored as the E8M0 code e + 127
 * (the pages give the group shapes only; the scale format is a reading):
 * e is the smallest integer >= -127 with amax <= 448 * 2^e, and
 * code = RNE_e4m3(x / 2^e).  An all-zero group gets e = -127. */
int oracle_e8m0_exponent(double amax);
double oracle_e8m0_value(uint8_t code);
void oracle_fp8_quantize_pow2(const double *x, int n, uint8_t *codes, uint8_t *e8m0);
/* x: [M, ld] rows of dtype (f32, bf16, or ORC_F64 doubles), K % 128 == 0;
 * codes [M, K]; scales [K/128, M] (group-major, one code per group). */
int oracle_fp8_quant_rows(int dtype, const void *x, int64_t M, int K, int64_t ld,
                          uint8_t *codes, uint8_t *scales);
/* w: [N, K] (f32 or bf16); codes [N, K]; scales [N/128, K/128]. */
int oracle_fp8_quant_weight(int dtype, const void *w, int N, int K, uint8_t *codes,
                            uint8_t *scales);
/* c [n_rows or M, N] = dequant(A) dequant(B)^T in fp64. */
int oracle_fp8_gemm(const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb,
                    int64_t M, int N, int K, const int64_t *rows, int64_t n_rows, double *c);
/* r = x + res (float32 add, stored in dtype: res_out may be NULL), then
 * y = gamma * r / sqrt(mean(r^2) + eps) in fp64; res may be NULL (= 0). */
int oracle_addnorm(int dtype, const void *x, const void *res, const void *gamma, double eps,
                   int64_t M, int K, void *res_out, double *y);
double oracle_silu(double g);
/* y_i = silu(g_i) * u_i, the SwiGLU product of the gate and up halves */
void oracle_swiglu(const double *g, const double *u, int64_t n, double *y);

/* ---- A4: vocab statistics per row ---------------------------------------
 * p = softmax(x); argmax = lowest index of the largest logit; maxprob =
 * max_j p_j; entropy = -sum p_j ln p_j (terms with p_j = 0 add nothing).
 * [SWD, 3.1 and 4.2: max probability token]; [Flash, 3.1: entropy].
 * logits: rows of length V at stride row_stride elements, f32 or bf16.
 * rows != NULL selects n_rows row indices (outputs packed in that order). */
int oracle_vocab_stats(int dtype, const void *logits, int64_t N, int64_t V,
                       int64_t row_stride, int32_t *argmax, double *maxprob,
                       double *entropy, const int64_t *rows, int64_t n_rows);

/* ---- A5-A7: history, stability, confidence, window mask -----------------
 * One decode step s for B sequences of length L.
 * pos [B, n] lists the positions recomputed this step (NULL: all L, n = L;
 * -1 entries are padding);
 * argmax/maxprob/entropy are this step's statistics for those rows,
 * laid out [B, n].  State (in/out): ring_argmax/ring_maxprob/ring_step
 * [D, B, L] (slot s mod D holds step s; ring_step = -1 marks empty),
 * entropy_latest/t_write [B, L], stable [B, L] (0/1, sticky).
 * Params: K steps, tau (strict >), D ring depth >= K, R radius >= 0,
 * alpha, beta, lambda, conf_thresh (<= 0 disables the gate), vocab V
 * (Hmax = ln V), R_early / T_steps (the dynamic radius, T_steps <= 1: off),
 * refresh_every (0: off).  Outputs: mask [B, L] (0/1), conf [B, L] double,
 * next_pos [B, L] (ascending masked positions, rest -1), count [B],
 * all_stable [B].
 * [SWD, 3.1 stability test; 3.2 window; 3.3 steps c-d; 4.2 scheduler];
 * [Flash, 3.1 cache confidence]. */
/* ---- N3: radius and refresh schedules, eviction under a budget ----------
 * dynamic radius [SWD, 4.4]: R_early at step 0 rising linearly to R at step
 * T-1 (integer division), R after; T <= 1 keeps R.  Refresh [Flash, 5.1]:
 * every F-th step (s > 0, s % F == 0) recomputes the whole sequence; the
 * interval for T steps is round(T/10) within [3, 10].  Quotas [Flash, 5.2]
 * and confidence-ordered eviction [Flash, 3.3]: see oracle.c. */
int oracle_dynamic_radius(int R_early, int R, int T, int step);
int oracle_is_refresh_step(int F, int step);
int oracle_refresh_interval(int T);
int oracle_cache_quotas(int B, const int32_t *len, int64_t budget, double min_frac,
                        int32_t *quota);
int oracle_evict_by_confidence(int B, int L, const float *conf, const int32_t *quota,
                               const int32_t *pos, int n, uint8_t *cached, uint8_t *mask,
                               int32_t *next_pos, int32_t *count, int32_t *evicted);

/* N4 [Flash, 4.1-4.3]: the parallel width ramps from w_early at step 0 to
 * w_late at step T-1; the self-verification of a step's parallel decodes and
 * the withdrawal of conflicting spans: see oracle.c. */
int oracle_parallel_width(int w_early, int w_late, int T, int step);
int oracle_self_verify(int B, int L, const int32_t *dec_pos, int n, const float *p_marg,
                       const float *p_joint, int W, double tau, uint8_t *rollback,
                       uint8_t *mask, uint8_t *stable, uint8_t *cached, int32_t *next_pos,
                       int32_t *count, int32_t *n_rollback, int32_t *rb_pos);

/* Validity of a scatter's position list: per sequence b, bad[b] = entries
 * outside [0, L) other than -1, dup[b] = entries equal to an earlier entry
 * of the same sequence.  See oracle.c. */
int oracle_check_positions(int B, int L, const int32_t *pos, int n, int32_t *bad, int32_t *dup);

/* A5-A7 [SWD, 3.1-3.3 and 4.2; Flash, 3.1]: record, stability test,
 * confidence alpha(1 - H/ln V) + beta exp(-lambda dt), window mask and
 * compaction for one step.  The age dt = s - t_write is clamped to
 * [0, n_decay - 1] (n_decay >= 1): the library reads the age factor from a
 * table of n_decay entries, and with n_decay above every age the clamp never
 * applies.  See oracle.c. */
int oracle_stability_step(int B, int L, int step, const int32_t *pos, int n,
                          const int32_t *argmax, const float *maxprob,
                          const float *entropy,
                          int32_t *ring_argmax, float *ring_maxprob, int32_t *ring_step,
                          float *entropy_latest, int32_t *t_write, uint8_t *stable,
                          int K, double tau, int D, int R,
                          double alpha, double beta, double lambda, int n_decay,
                          double conf_thresh, int64_t V,
                          int R_early, int T_steps, int refresh_every,
                          uint8_t *mask, double *conf, int32_t *next_pos,
                          int32_t *count, uint8_t *all_stable);

#ifdef __cplusplus
}
#endif
#endif
