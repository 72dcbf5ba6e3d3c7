/*
 * dllm.h -- C ABI of the per-step hot path of cached masked-diffusion
 * language-model decoding on AMD Instinct MI355X (gfx950).
 *
 * One decoding step of a diffusion LM recomputes only the positions of the
 * active block.  This library covers what happens around that recompute:
 *
 *   dllm_cache_init        describe and clear a persistent per-layer K/V cache
 *   dllm_scatter_kv        write the block's fresh K/V rows into the cache
 *   dllm_scatter_attention the scatter and the block attention in one call
 *   dllm_sink_rolling_map  build a sink + rolling-window key index map
 *   dllm_block_attention   block queries vs. the cached keys, bidirectional
 *   dllm_facache_maps      unchanged / changed key lists of a block's steps
 *   dllm_facache_merge     queries outside the block: memoized softmax state
 *                          continued over the changed keys only
 *   dllm_fp8_*             per-group FP8 FFN: quantisers, add & norm + quant,
 *                          block-scaled GEMM, GEMM + SwiGLU + quant
 *   dllm_vocab_stats       argmax token, max-probability, entropy per row
 *   dllm_*_workspace, dllm_workspace_size
 *                          scratch bytes a call needs for its shapes
 *   dllm_stability_reset   clear the per-position decode state
 *   dllm_stability_mask    history ring, stability test, confidence score and
 *                          window expansion -> next step's compute mask
 *   dllm_evict_by_confidence / dllm_cache_quotas / dllm_refresh_interval
 *                          budgeted cache and refresh schedule
 *   dllm_self_verify / dllm_parallel_width
 *                          conflict check of a step's parallel decodes
 *
 * Page titles cited below (section numbers are the pages' own):
 *   [SWD]     Stable Window Decoding blog page on temporal stability in
 *             diffusion-LM decoding (wmrh.cn/news/51151)
 *   [LaCache] "LaCache: Exact Caching and Precision-Adaptive Inference for
 *             Diffusion Large Language Models" (gist.science explainer;
 *             sections of its technical summary)
 *   [Sinks]   attention-sinks and rolling K/V cache blog page for GPT-2
 *             (wmrh.cn/news/159578)
 *   [Flash]   Flash-dLLM page: I/O-aware KV cache and self-verifying
 *             parallel decoding (bjdmk.com.cn/news/5926815)
 *
 * Conventions shared by every call
 *   - Every array argument is a DEVICE pointer to memory the caller owns
 *     (the library allocates no device memory and keeps no state between
 *     calls, apart from the fixed per-GPU array that
 *     dllm_scatter_attention_noalloc works in).  Scalars and parameter
 *     structs are host values.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls enqueue work on it and return without synchronising.
 *   - Shapes are row-major (C order), innermost dimension last.
 *   - Host-side validation returns a negative dllm_status and enqueues
 *     nothing; a HIP launch error returns DLLM_EHIP.
 *   - An index of -1 in a position list or key map is padding and is
 *     skipped; any other index outside [0, L) is skipped too and counted in
 *     the optional `bad_count` where a call has one.  A position given
 *     twice for one sequence in a single scatter is a caller error: the
 *     cache row at that position is then unspecified (its 16-byte chunks
 *     may come from either fresh row, and an e4m3 row's codes may pair with
 *     the other row's scale).  dllm_check_positions finds such lists.
 *   - Results are bitwise reproducible run to run: reductions merge in a
 *     fixed order and use no floating-point atomics.
 */
#ifndef DLLM_H
#define DLLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DLLM_OK = 0,
    DLLM_EINVAL = -1,      /* null pointer or out-of-range scalar argument   */
    DLLM_EDTYPE = -2,      /* unsupported dtype or dtype combination         */
    DLLM_ESHAPE = -3,      /* inconsistent or unsupported shape              */
    DLLM_EALIGN = -4,      /* pointer or row size not 16-byte aligned        */
    DLLM_ERANGE = -5,      /* size beyond a supported maximum                */
    DLLM_EHIP = -6,        /* a HIP runtime call or kernel launch failed     */
    DLLM_EWORKSPACE = -7   /* workspace missing or smaller than required     */
} dllm_status;

typedef enum {
    DLLM_F32 = 0,          /* IEEE binary32                                  */
    DLLM_BF16 = 1,         /* bfloat16                                       */
    DLLM_E4M3 = 2          /* OCP e4m3fn, one float32 scale per 128 elements */
} dllm_dtype;

/* Descriptor of one layer's persistent K/V cache, filled by dllm_cache_init.
 * Plain data; the caller owns the memory it points to.
 *   k, v       [B, n_kv_heads, L, d_head] elements of `dtype`
 *   k_scale,   [B, n_kv_heads, L, d_head/128] float32, E4M3 only (else NULL):
 *   v_scale    element c of a row decodes to code * scale[c / 128]        */
typedef struct {
    int32_t B, L, n_kv_heads, d_head;
    int32_t dtype;
    int32_t reserved;
    void *k, *v;
    float *k_scale, *v_scale;
} dllm_kv_cache;

/* Parameters of the stability / confidence / window step.
 *   K            steps a position's argmax must persist [SWD, 3.1]
 *   D            depth of the step-history ring, D >= K
 *   R            window radius around each position to recompute [SWD, 3.2]
 *   tau          stability threshold: mean max-prob over the K steps must
 *                exceed it (strictly) [SWD, 3.1]
 *   alpha, beta, decay, n_decay
 *                cache confidence alpha*(1 - H/ln V) + beta*exp(-lambda*dt)
 *                [Flash, 3.1].  The exponential comes from a table:
 *                decay is a DEVICE array of n_decay float64 values,
 *                decay[k] = exp(-lambda*k) as dllm_confidence_decay writes
 *                it on the host, read at k = min(dt, n_decay - 1) (dt < 0
 *                reads k = 0); so every value of the score is plain IEEE
 *                float64 arithmetic (no fused multiply-add) on host-computed
 *                inputs.  n_decay >= the trajectory length makes the
 *                lookup exact.  With beta = 0 the table is not read and may
 *                be NULL.
 *   conf_thresh  positions whose confidence is below it are recomputed
 *                [Flash, 3.1]; <= 0 turns the gate off
 *   vocab        V of the vocab pass (max entropy ln V)
 *   advance_step nonzero: with per-sequence step numbers in device memory,
 *                each sequence's number is incremented once the call has
 *                used it (the decode loop's step counter, kept on the GPU)
 *   R_early, T_steps
 *                the window radius widens over the trajectory [SWD, 4.4]:
 *                at step s it is R_early + (R - R_early) * min(s, T_steps-1)
 *                / (T_steps - 1) (integer division); T_steps <= 1 keeps R
 *   refresh_every
 *                every refresh_every-th step (s > 0) recomputes the whole
 *                sequence [Flash, 5.1]; 0 never (dllm_refresh_interval gives
 *                the pages' interval for a trajectory length) */
typedef struct {
    int32_t K, D, R, advance_step;
    double tau, alpha, beta, conf_thresh;
    const double *decay;
    int64_t vocab;
    int32_t R_early, T_steps, refresh_every, n_decay;
} dllm_stab_params;

/* Human-readable name of a status code (static string). */
const char *dllm_status_str(int status);

/* Library version, as major*10000 + minor*100 + patch. */
int dllm_version(void);

/* ---------------------------------------------------------------------------
 * dllm_cache_init -- validate and fill `cache`, and zero the K/V (and scale)
 * storage on `stream`.  The persistent per-layer cache of the states of the
 * unchanged tokens [LaCache, Methodology 1: RoPECache], fixed in size for
 * its lifetime [Sinks, 3.1].
 *   dtype     DLLM_F32, DLLM_BF16 or DLLM_E4M3 (E4M3 needs d % 128 == 0 and
 *             non-NULL scale arrays)
 *   k, v      device, 16-byte aligned, B*n_kv_heads*L*d elements each
 * Limits: B, L, n_kv_heads >= 1; d in 16..256 with d*size(dtype) % 16 == 0;
 * L*d*size(dtype) < 2^32 bytes (the rows of one sequence and KV head),
 * else DLLM_ERANGE.  Every call that takes a cache checks the same.
 * Returns DLLM_OK or a negative dllm_status.
 * ------------------------------------------------------------------------- */
int dllm_cache_init(dllm_kv_cache *cache, int B, int L, int n_kv_heads, int d_head,
                    int dtype, void *k, void *v, float *k_scale, float *v_scale,
                    void *stream);

/* ---------------------------------------------------------------------------
 * dllm_scatter_kv -- write the recomputed block's fresh K/V rows into the
 * cache: cache[b, h, pos[b, j], :] = new[b, j, h, :].  Every other row is
 * left bit-for-bit unchanged, so the cache then holds exactly what a full
 * recompute would assemble [LaCache, Methodology 1 and 3; SWD, 4.1 and 4.3
 * write-back of masked positions; Sinks, 3.2 and 5.1 index writes].
 *   k_new, v_new  [B, n, n_kv_heads, d] in src_dtype.  For F32/BF16 caches
 *                 src_dtype must equal the cache dtype (plain copy).  For
 *                 E4M3 caches src_dtype is F32 or BF16 and each 128-element
 *                 group is quantised: scale = amax/448 (float32 divide),
 *                 code = round-to-nearest-even(x/scale) on the e4m3 grid,
 *                 saturating at +-448; an all-zero group gets scale 0
 *                 [LaCache, Methodology 2: per-group 1x128 FP8].
 *   pos           [B, n] int32 device; -1 = padding.  Positions must be
 *                 distinct within a sequence (see the conventions above).
 *   bad_count     optional device int32; out-of-range positions (other than
 *                 -1) are skipped and atomically added here.  May be NULL.
 * n == 0 is a no-op.
 * ------------------------------------------------------------------------- */
int dllm_scatter_kv(const dllm_kv_cache *cache, const void *k_new, const void *v_new,
                    int src_dtype, const int32_t *pos, int n, int32_t *bad_count,
                    void *stream);

/* ---------------------------------------------------------------------------
 * dllm_check_positions -- the debug check of a scatter's position list
 * [Sinks, 5.1 warns that cache rows written to the wrong place corrupt every
 * later step]: per sequence b, bad[b] = the entries of pos[b, :] outside
 * [0, L) other than the padding value -1, and dup[b] = the entries that
 * repeat a position an earlier entry of the same sequence holds (n_valid -
 * n_distinct).  A list is a valid dllm_scatter_kv argument iff both are 0.
 *   pos      [B, n] int32 device
 *   bad, dup [B] int32 device outputs
 * Limits: 1 <= L <= 131072 (one bit per position in on-chip memory),
 * B <= 65535, n >= 0.
 * ------------------------------------------------------------------------- */
int dllm_check_positions(int B, int L, const int32_t *pos, int n, int32_t *bad, int32_t *dup,
                         void *stream);

/* ---------------------------------------------------------------------------
 * dllm_sink_rolling_map -- key index map of S attention sinks plus a rolling
 * window of the R newest keys [Sinks, 2.3 and 3.2]: for sequence b with
 * block end e = end[b] (one past its last position),
 *   key_idx[b, :] = {0, ..., min(S, e)-1} then [max(S, e-R), e), ascending,
 * padded with -1 up to n_keys.  The sinks keep their original positions and
 * the map never holds more than S + R keys.
 *   end      [B] int32 device, values in [0, L]; values outside are clamped
 *   key_idx  [B, n_keys] int32 device; n_keys >= S + R
 * ------------------------------------------------------------------------- */
int dllm_sink_rolling_map(int B, int L, int S, int R, const int32_t *end,
                          int32_t *key_idx, int n_keys, void *stream);

/* ---------------------------------------------------------------------------
 * dllm_block_attention -- for every query of the active block,
 *   out = softmax(q . K^T * scale) . V
 * over the selected cached keys, with no causal mask (the block attends
 * bidirectionally to the whole context) [LaCache, problem statement and
 * Methodology 1 (FACache's online-softmax statistics m, l, O~); Sinks, 2.1].
 * Query head h reads KV head h / (Hq / n_kv_heads).
 *   q        [B, Hq, b, d] in q_dtype.  BF16 queries run on bf16 MFMA with
 *            float32 accumulation (BF16 or E4M3 caches, d in {64, 128});
 *            F32 queries with an F32 cache run a float32 VALU path.
 *   key_idx  [B, n_keys] int32 device, or NULL for all L keys (n_keys = L);
 *            -1 entries are padding.  A row with no key gets out = 0 and
 *            lse = -inf.
 *   scale    > 0, or 0 for 1/sqrt(d)
 *   out      [B, Hq, b, d] in out_dtype (F32 or BF16)
 *   lse      optional [B, Hq, b] float32: natural-log log-sum-exp of the
 *            scaled scores (the softmax normaliser).  May be NULL.
 *   workspace / ws_bytes: device scratch of at least
 *            dllm_block_attention_workspace(...) bytes (may be 0 bytes).
 * ------------------------------------------------------------------------- */
int dllm_block_attention(const dllm_kv_cache *cache, const void *q, int q_dtype, int Hq,
                         int b, const int32_t *key_idx, int n_keys, float scale,
                         void *out, int out_dtype, float *lse,
                         void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes dllm_block_attention needs for these shapes, with or
 * without a key map (0 if none: the keys are not split over workgroups). */
size_t dllm_block_attention_workspace(const dllm_kv_cache *cache, int q_dtype, int Hq,
                                      int b, int n_keys);

/* ---------------------------------------------------------------------------
 * dllm_scatter_attention -- dllm_scatter_kv then dllm_block_attention, as one
 * call: the block's fresh K/V rows go into the cache and the block's queries
 * attend over the cache with them [LaCache, Methodology 3: the step
 * recomputes the block, writes its K/V, and attends over the whole cached
 * context].  Arguments as for the two calls (k_new, v_new, src_dtype, pos,
 * n, bad_count as for dllm_scatter_kv; the rest as for dllm_block_attention,
 * with the same workspace).  The cache and out afterwards hold exactly what
 * the two calls in sequence leave.  With a bf16 cache and bf16 rows and no
 * key map, when the block's queries fit one 32-row group per KV head, the
 * attention kernel writes the rows itself (each workgroup the positions in
 * its own key range) before it loads any key tile; otherwise the two kernels
 * run in sequence on the stream.  Positions must be distinct within a
 * sequence, as for dllm_scatter_kv.  Errors: those of the two calls, all
 * checked before anything is enqueued.
 * ------------------------------------------------------------------------- */
int dllm_scatter_attention(const dllm_kv_cache *cache, const void *k_new, const void *v_new,
                           int src_dtype, const int32_t *pos, int n, int32_t *bad_count,
                           const void *q, int q_dtype, int Hq, int b, const int32_t *key_idx,
                           int n_keys, float scale, void *out, int out_dtype, float *lse,
                           void *workspace, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * dllm_scatter_attention_noalloc -- dllm_scatter_attention for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same arguments without the
 * workspace, the same kernels and bit-identical results.  The key-split
 * partials go to a scratch array inside the library, one per GPU, of
 * DLLM_NOALLOC_SCRATCH_BYTES; a call whose partials need more returns
 * DLLM_ERANGE before anything is enqueued (dllm_block_attention_workspace
 * gives the size).  The call allocates nothing.  The first call on a device
 * looks that device's array up (a host-side query, no allocation).  Every
 * call on one GPU shares its array: calls that overlap on one GPU (two
 * streams, or two threads) race on it; calls on one stream are ordered and
 * safe.  The array keeps the last call's partials, which no later call reads
 * before writing.
 * ------------------------------------------------------------------------- */
#define DLLM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int dllm_scatter_attention_noalloc(const dllm_kv_cache *cache, const void *k_new, const void *v_new,
                                   int src_dtype, const int32_t *pos, int n, int32_t *bad_count,
                                   const void *q, int q_dtype, int Hq, int b, const int32_t *key_idx,
                                   int n_keys, float scale, void *out, int out_dtype, float *lse,
                                   void *stream);

/* ---------------------------------------------------------------------------
 * dllm_facache_maps -- the key lists of FACache for one block's denoising
 * steps [LaCache, problem statement and Methodology 1: within the steps of
 * one block only the active block's tokens change, the prompt and the masked
 * suffix keep theirs]: for sequence b with block [o, o + blk), o = start[b],
 *   unchanged_idx[b, :] = {0..o-1} then {o+blk..L-1}   (L - blk entries)
 *   block_idx[b, :]     = {o..o+blk-1}                 (blk entries)
 * both ascending.
 *   start          [B] int32 device; values are clamped to [0, L - blk]
 *   unchanged_idx  [B, L - blk] int32 device (output)
 *   block_idx      [B, blk] int32 device (output)
 * Needs 1 <= blk < L.
 * ------------------------------------------------------------------------- */
int dllm_facache_maps(int B, int L, int blk, const int32_t *start, int32_t *unchanged_idx,
                      int32_t *block_idx, void *stream);

/* ---------------------------------------------------------------------------
 * dllm_facache_merge -- FACache for the queries outside the active block
 * [LaCache, Methodology 1 (FACache) and 3 (inference workflow)]: the online-
 * softmax state (m, l, O~) of each such query over the unchanged keys is
 * memoized at the block's first step, and every later step starts each
 * query's state from the memo and walks only the changed keys, so the
 * (unchanged query, unchanged key) tiles are never recomputed.
 * The memo is stored normalised, as the output of dllm_block_attention with
 * out_dtype = DLLM_F32 and an lse array (the same state with its reference
 * moved to m' = lse, l' = 1, O~' = O); that call, with the unchanged queries
 * over key_idx = unchanged_idx, is the memo fill.  Per row:
 *   m_new = max(memo_lse, max_j s_j),  s_j = scale * q . k_j
 *   out   = (memo_o e^(memo_lse - m_new) + sum_j e^(s_j - m_new) v_j)
 *           / (e^(memo_lse - m_new) + sum_j e^(s_j - m_new))
 *   lse   = m_new + ln(denominator)
 *   q         [B, Hq, n_q, d] in q_dtype: the queries outside the block
 *   key_idx   [B, n_keys] int32 device: the changed keys (block_idx of
 *             dllm_facache_maps), -1 entries are padding; NULL = all L keys
 *   memo_o    [B, Hq, n_q, d] float32 device, 16-byte aligned
 *   memo_lse  [B, Hq, n_q] float32 device, natural log; -inf marks an empty
 *             memo (its memo_o row is ignored); other values must be finite
 *   out       [B, Hq, n_q, d] in out_dtype (F32 or BF16); lse optional
 *             [B, Hq, n_q] float32.  out and lse must not overlap the memo.
 *   cache, q_dtype, scale, workspace: as for dllm_block_attention, with the
 *             workspace size from dllm_facache_merge_workspace.
 * The memo and the queries are only read.
 * ------------------------------------------------------------------------- */
int dllm_facache_merge(const dllm_kv_cache *cache, const void *q, int q_dtype, int Hq, int n_q,
                       const int32_t *key_idx, int n_keys, float scale,
                       const float *memo_o, const float *memo_lse,
                       void *out, int out_dtype, float *lse,
                       void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes dllm_facache_merge needs for these shapes, with or without
 * a key map (0 if the keys are not split over workgroups). */
size_t dllm_facache_merge_workspace(const dllm_kv_cache *cache, int q_dtype, int Hq,
                                    int n_q, int n_keys);

/* ---------------------------------------------------------------------------
 * Per-group FP8 for the FFN [LaCache, Methodology 2: Gate-Up and FF-Out in
 * FP8 with 1 x 128 activation groups and 128 x 128 weight groups, the
 * quantisation fused into the add & norm and into SwiGLU].
 * Every group carries one power-of-two scale 2^e stored as the E8M0 byte
 * e + 127 (the pages fix the group shapes only): e is the smallest integer
 * >= -127 with amax <= 448 * 2^e, and each code is the OCP e4m3fn value
 * RNE(x / 2^e), so no code saturates.  An all-zero group gets e = -127.
 * Layouts (row-major):
 *   activation codes [M, K] u8, activation scales [K/128, M] u8 (the scales
 *     of one 128-column group are contiguous over the rows);
 *   weight codes [N, K] u8 (the product is A . W^T), weight scales
 *     [N/128, K/128] u8.
 * K must be a multiple of 128 throughout; code arrays 16-byte aligned.
 * ------------------------------------------------------------------------- */

/* dllm_fp8_quant_rows -- quantise the 1 x 128 groups of an [M, K] matrix
 * (rows at stride ld elements, F32 or BF16; ld * size % 16 == 0). */
int dllm_fp8_quant_rows(const void *x, int dtype, int64_t M, int K, int64_t ld,
                        uint8_t *codes, uint8_t *scales, void *stream);

/* dllm_fp8_addnorm_quant -- the add & norm before the FFN, fused with the
 * quantisation of its output: per row, r = x + residual (float32 add,
 * rounded to dtype and written to residual_out when non-NULL), then
 * y = gamma * r / sqrt(mean(r^2) + eps) (RMS normalisation, float32), then
 * the 1 x 128 groups of y as codes and scales.  residual may be NULL (= 0).
 *   x, residual, residual_out [M, K]; gamma [K]; all of dtype (F32 / BF16)
 * Limits: K <= 16384, eps >= 0. */
int dllm_fp8_addnorm_quant(const void *x, const void *residual, const void *gamma, int dtype,
                           float eps, int64_t M, int K, void *residual_out,
                           uint8_t *codes, uint8_t *scales, void *stream);

/* dllm_fp8_quant_weight -- quantise the 128 x 128 blocks of a weight
 * matrix W [N, K] (F32 or BF16; N % 128 == 0). */
int dllm_fp8_quant_weight(const void *w, int dtype, int N, int K, uint8_t *codes,
                          uint8_t *scales, void *stream);

/* dllm_fp8_gemm -- C = dequant(A) . dequant(W)^T on the block-scaled FP8
 * matrix cores with float32 accumulation, C [M, N] bf16 (the FF-Out
 * product).  N % 256 == 0, 128 <= K <= 12288, any M >= 0. */
int dllm_fp8_gemm(const uint8_t *a, const uint8_t *a_scale, const uint8_t *w,
                  const uint8_t *w_scale, int M, int N, int K, void *c, void *stream);

/* dllm_fp8_gemm_swiglu -- the Gate-Up product fused with SwiGLU and the
 * quantisation of its output: W's rows come in pairs of 128-row blocks,
 * block 2j holding gate features 128j .. 128j+127 and block 2j+1 the up
 * features of the same indices; per row and feature f,
 *   h_f = silu(gate_f) * up_f,  silu(g) = g / (1 + e^-g)  (float32)
 * and h [M, N/2] is written as codes with scales [N/256, M] (the 1 x 128
 * groups of h), the input of the FF-Out product.  Limits as dllm_fp8_gemm. */
int dllm_fp8_gemm_swiglu(const uint8_t *a, const uint8_t *a_scale, const uint8_t *w,
                         const uint8_t *w_scale, int M, int N, int K, uint8_t *out_codes,
                         uint8_t *out_scales, void *stream);

/* ---------------------------------------------------------------------------
 * dllm_vocab_stats -- one pass over each row of logits:
 *   argmax[r]  lowest index of the largest logit
 *   maxprob[r] largest softmax probability, 1 / sum_j exp(x_j - max)
 *   entropy[r] -sum_j p_j ln p_j (natural log)
 * [SWD, 3.1 and 4.2: per-position max probability and its token;
 *  Flash, 3.1: the entropy of the step's distribution].  The probabilities
 * are never written out.
 *   logits     [N, row_stride] of dtype F32 or BF16; columns >= V are ignored
 *   V          1 <= V <= row_stride, V < 2^31
 *   Logits are finite or -inf with at least one finite value per row (other
 *   rows give unspecified results).
 *   workspace / ws_bytes: at least dllm_vocab_stats_workspace(N, V) bytes.
 * ------------------------------------------------------------------------- */
int dllm_vocab_stats(const void *logits, int dtype, int64_t N, int64_t V, int64_t row_stride,
                     int32_t *argmax, float *maxprob, float *entropy,
                     void *workspace, size_t ws_bytes, void *stream);

size_t dllm_vocab_stats_workspace(int64_t N, int64_t V);

/* ---------------------------------------------------------------------------
 * dllm_workspace_size -- the three workspace queries above behind one call,
 * for a caller that sizes every workspace through a single entry point.
 *   which       a dllm_workspace_kind
 *   shape_args  host pointer to a dllm_workspace_args.  The block-attention
 *               and FACache kinds read cache, q_dtype, Hq, n_q (the block's
 *               b for block attention) and n_keys; the vocab kind reads N and
 *               V.  Other fields are ignored.
 * Returns what the matching query returns for those shapes, and 0 for an
 * unknown kind or a NULL shape_args (as the queries do for shapes they
 * reject: the call itself then reports the error).
 * ------------------------------------------------------------------------- */
typedef enum {
    DLLM_WS_BLOCK_ATTENTION = 0,  /* dllm_block_attention, dllm_scatter_attention */
    DLLM_WS_FACACHE_MERGE = 1,    /* dllm_facache_merge                          */
    DLLM_WS_VOCAB_STATS = 2       /* dllm_vocab_stats                            */
} dllm_workspace_kind;

typedef struct {
    const dllm_kv_cache *cache;
    int q_dtype;
    int Hq;
    int n_q;
    int n_keys;
    int64_t N;
    int64_t V;
} dllm_workspace_args;

size_t dllm_workspace_size(int which, const dllm_workspace_args *shape_args);

/* ---------------------------------------------------------------------------
 * dllm_stability_reset -- empty the history ring (ring_step = -1) and clear
 * entropy_latest, t_write and stable for B sequences of length L with ring
 * depth D: the scheduler reset of [SWD, 4.2].
 * ------------------------------------------------------------------------- */
int dllm_stability_reset(int B, int L, int D, int32_t *ring_argmax, float *ring_maxprob,
                         int32_t *ring_step, float *entropy_latest, int32_t *t_write,
                         uint8_t *stable, void *stream);

/* ---------------------------------------------------------------------------
 * dllm_stability_mask -- after the forward of step s (s >= 0), for each
 * sequence:
 *  1. record (argmax, maxprob, s) of every recomputed position in ring slot
 *     s mod D, set entropy_latest and t_write = s [SWD, 3.3 step c];
 *  2. a recomputed position that is not yet stable becomes stable when its
 *     ring holds the steps s, s-1, ..., s-K+1, all with one argmax, and the
 *     mean of their max-probs (float64, oldest first) exceeds tau; stable
 *     is never cleared [SWD, 3.1 and 4.2];
 *  3. conf = alpha(1 - H/ln V) + beta decay[min(s - t_write, n_decay - 1)]
 *     in float64 for every position, H = entropy_latest, decay[k] =
 *     exp(-lambda k) [Flash, 3.1]; the division, subtraction, products and
 *     sum are single IEEE operations, none fused, and conf is their value
 *     rounded once to float32;
 *  4. seed = not stable, or conf < conf_thresh; mask[j] = 1 when a seed lies
 *     within R of j (clamped to the sequence); with no seed at all the mask
 *     is all ones and all_stable = 1 [SWD, 3.2 and 4.2];
 *  5. next_pos lists the mask's positions ascending, padded with -1, and
 *     count holds their number: the positions to recompute at step s+1.
 *   pos        [B, n] recomputed positions of step s, or NULL for all L
 *              (then n must be L, or 0 for none); -1 entries are padding
 *   argmax, maxprob, entropy  [B, n] statistics of those rows (as written
 *              by dllm_vocab_stats)
 *   ring_*     [D, B, L] state; entropy_latest, t_write, stable [B, L] state
 *   mask [B, L] u8, conf [B, L] f32, next_pos [B, L] i32, count [B] i32,
 *   all_stable [B] u8: outputs (conf may be NULL)
 *   step_dev   optional [B] device int32: when non-NULL, sequence b's step
 *              number is read from step_dev[b] when the kernel runs (`step`
 *              is then ignored) and, with params->advance_step, written back
 *              plus one, so a captured graph of a decode step replays as
 *              successive steps; values must be >= 0.  May be NULL.
 * Limits: L <= 131072, 1 <= K <= D, R >= 0, vocab >= 2; with beta != 0 a
 * non-NULL 8-byte aligned decay table and n_decay >= 1.
 * ------------------------------------------------------------------------- */
int dllm_stability_mask(int B, int L, int step, int32_t *step_dev, const int32_t *pos, int n,
                        const int32_t *argmax, const float *maxprob, const float *entropy,
                        int32_t *ring_argmax, float *ring_maxprob, int32_t *ring_step,
                        float *entropy_latest, int32_t *t_write, uint8_t *stable,
                        const dllm_stab_params *params,
                        uint8_t *mask, float *conf, int32_t *next_pos, int32_t *count,
                        uint8_t *all_stable, void *stream);

/* ---------------------------------------------------------------------------
 * dllm_confidence_decay -- the age factor of the cache confidence [Flash,
 * 3.1: beta exp(-lambda (t - t_write))] as a table: table[k] =
 * exp(-lambda * k) for k = 0 .. n-1, float64, computed on the host with the
 * C library's exp.  HOST array of n values; the caller copies it to the
 * device once and passes it as dllm_stab_params.decay.  Returns DLLM_EINVAL
 * for a NULL table, n < 1 or a lambda that is negative or not finite.
 * ------------------------------------------------------------------------- */
int dllm_confidence_decay(double lambda, int n, double *table);

/* ---------------------------------------------------------------------------
 * dllm_refresh_interval -- the full-refresh interval for a trajectory of T
 * denoising steps [Flash, 5.1: every 5-10 steps for T in 50..100, every 3-5
 * below 50]: round(T / 10) kept within [3, 10].  Host only.
 * ------------------------------------------------------------------------- */
int dllm_refresh_interval(int T);

/* ---------------------------------------------------------------------------
 * dllm_cache_quotas -- per-request shares of a cache budget in positions
 * [Flash, 5.2: each request keeps at least a fraction (0.2 on the page) of
 * its length; the rest goes by arrival].  quota[b] = ceil(min_frac * len[b])
 * (at most len[b]), then what the budget has left is handed out in index
 * order, each request up to len[b].  Host arrays.  DLLM_ERANGE when the
 * budget cannot cover the guaranteed shares.
 * ------------------------------------------------------------------------- */
int dllm_cache_quotas(int B, const int32_t *len, int64_t budget, double min_frac, int32_t *quota);

/* ---------------------------------------------------------------------------
 * dllm_evict_by_confidence -- keep a sequence's cached K/V within its quota
 * [Flash, 3.3: the lowest-confidence positions leave first, a position's K
 * and V together; per-request quotas, 5.2].  Per sequence b:
 *  1. the positions recomputed this step (pos, or NULL for all L) hold fresh
 *     K/V and are marked cached;
 *  2. when more than quota[b] positions are cached (quota < 0: no limit), the
 *     quota[b] with the highest conf stay (ties: the lower position), the
 *     rest are evicted (cached = 0);
 *  3. every uncached position must be recomputed before it is attended to:
 *     mask |= !cached, and next_pos / count are compacted again.
 * Run after dllm_stability_mask, with its conf, mask, next_pos and count.
 *   conf      [B, L] float32 device (not NaN)
 *   quota     [B] int32 device
 *   pos, n    [B, n] int32 device, -1 padding (entries outside [0, L) are
 *             skipped); NULL with n = L: every position, NULL with n = 0: none
 *   cached    [B, L] u8 device state (0/1), in/out; all 0 before step 0
 *   mask, next_pos, count   as written by dllm_stability_mask (updated)
 *   evicted   optional [B] int32: positions evicted by this call
 * Limits: L <= 131072, B <= 65535.
 * ------------------------------------------------------------------------- */
int dllm_evict_by_confidence(int B, int L, const float *conf, const int32_t *quota,
                             const int32_t *pos, int n, uint8_t *cached, uint8_t *mask,
                             int32_t *next_pos, int32_t *count, int32_t *evicted, void *stream);

/* ---------------------------------------------------------------------------
 * dllm_parallel_width -- how many positions a step decodes in parallel
 * [Flash, 4.1: many early in the trajectory (8-16 on the page), few late
 * (2-4)]: w_early at step 0 falling linearly to w_late at step T-1 (integer
 * division), w_late afterwards; T <= 1 gives w_late.  Host only.
 * ------------------------------------------------------------------------- */
int dllm_parallel_width(int w_early, int w_late, int T, int step);

/* ---------------------------------------------------------------------------
 * dllm_self_verify -- check the tokens a step decoded in parallel and
 * withdraw conflicting spans [Flash, 4.2 and 4.3].  Per sequence b, for two
 * decoded positions a < c with c - a < W, the conflict score is
 * P(tok_a, tok_c) / (P(tok_a) P(tok_c)), in float64; a score below tau (0.5
 * on the page) is a conflict, a zero product never is.  Every position
 * decoded this step in [a, c] is withdrawn: rollback = 1, mask = 1, stable =
 * 0 and cached = 0 there (it is regenerated serially and its K/V
 * recomputed); next_pos / count are compacted from the mask again.
 *   dec_pos   [B, n] int32 device: the positions decoded this step,
 *             ascending, then -1 padding (as a compacted mask lists them)
 *   p_marg    [B, n] float32 device: the probability of each decoded token
 *   p_joint   [B, n, W-1] float32 device: entry (j, d-1) is the joint
 *             probability of the tokens at dec_pos[j] and dec_pos[j] + d,
 *             read only when that position was decoded too (the pages leave
 *             its computation to the model's verification pass)
 *   W         window of positions, 2..8 (3-5 on the page); tau >= 0
 *   rollback  [B, L] u8 device out; mask [B, L] u8 in/out; stable, cached
 *             [B, L] u8 in/out or NULL; next_pos [B, L], count [B] out
 *   n_rollback [B] int32 out or NULL; rb_pos [B, n] int32 out or NULL: the
 *             withdrawn positions ascending, -1 after
 * A sequence whose list is not ascending (or has a position outside [0, L),
 * or padding before a position) is left unchanged with count = -1 (and
 * n_rollback = -1).  Limits: L <= 131072, B <= 65535.
 * ------------------------------------------------------------------------- */
int dllm_self_verify(int B, int L, const int32_t *dec_pos, int n, const float *p_marg,
                     const float *p_joint, int W, double tau, uint8_t *rollback, uint8_t *mask,
                     uint8_t *stable, uint8_t *cached, int32_t *next_pos, int32_t *count,
                     int32_t *n_rollback, int32_t *rb_pos, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DLLM_H */
