/*
 * oracle.c -- plain fp64 CPU reference for one step of cached
 * masked-diffusion decoding.  TEST INFRASTRUCTURE ONLY (see oracle.h).
 *
 * Build: gcc -std=c11 -O2 -fopenmp -ffp-contract=off -fno-fast-math
 *        -shared -fPIC oracle.c -lm
 * Parallel loops run over independent rows or heads only, so results do not
 * depend on the thread count.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* number formats                                                            */
/* ------------------------------------------------------------------------ */

double oracle_bf16_value(uint16_t bits)
{
    /* a bfloat16 is the upper half of a float32 */
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* OCP e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal (value m * 2^-9); exponent 15 with mantissa
 * 7 is NaN; there are no infinities.  Largest finite value 1.75 * 2^8 = 448. */
double oracle_e4m3_value(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                 /* m/8 * 2^(1-7) */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Round |x| to the e4m3 grid by direct construction: find the spacing of
 * the grid in x's binade, divide (exact: power of two), round half to even
 * with rint (the default rounding mode), multiply back, then read the code
 * off the rounded value. */
static uint8_t e4m3_encode_double(double x);

uint8_t oracle_e4m3_encode(float xf)
{
    return e4m3_encode_double((double)xf);
}

static uint8_t e4m3_encode_double(double x)
{
    uint8_t sign = 0;
    double a, spacing, r, v;
    int e, E, M;

    if (isnan(x)) return 0x7F;
    if (signbit(x)) { sign = 0x80; a = -x; } else { a = x; }
    if (a > 448.0) return (uint8_t)(sign | 0x7E);   /* saturate: 0x7E = 448 */
    if (a == 0.0) return sign;

    frexp(a, &e);              /* a = f * 2^e with f in [0.5, 1): binade 2^(e-1) */
    e -= 1;                    /* a in [2^e, 2^(e+1)) */
    if (e < -6)
        spacing = ldexp(1.0, -9);            /* subnormal spacing */
    else
        spacing = ldexp(1.0, e - 3);          /* 3 mantissa bits */
    r = rint(a / spacing);                    /* ties to even */
    v = r * spacing;
    if (v == 0.0) return sign;
    if (v < ldexp(1.0, -6)) {                 /* subnormal result */
        E = 0;
        M = (int)(v / ldexp(1.0, -9));
    } else {
        frexp(v, &e);
        e -= 1;
        E = e + 7;
        M = (int)((v / ldexp(1.0, e) - 1.0) * 8.0);
    }
    return (uint8_t)(sign | (E << 3) | M);
}

void oracle_e4m3_quantize_group(const float *x, int n, uint8_t *codes, float *scale)
{
    float amax = 0.0f, s;
    int i;
    for (i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        *scale = 0.0f;
        for (i = 0; i < n; ++i) codes[i] = 0;
        return;
    }
    s = amax / 448.0f;                        /* float32 divide */
    *scale = s;
    for (i = 0; i < n; ++i) {
        float q = x[i] / s;                   /* float32 divide */
        codes[i] = oracle_e4m3_encode(q);
    }
}

/* element -> double for the two float source formats */
static double load_src(int dtype, const void *p, int64_t i)
{
    if (dtype == ORC_F32) return (double)((const float *)p)[i];
    return oracle_bf16_value(((const uint16_t *)p)[i]);
}

/* ------------------------------------------------------------------------ */
/* A1: scatter                                                               */
/* ------------------------------------------------------------------------ */

int oracle_scatter_kv(int cache_dtype, int B, int L, int Hkv, int d,
                      void *cache_k, void *cache_v, float *k_scale, float *v_scale,
                      int src_dtype, const void *k_new, const void *v_new,
                      const int32_t *pos, int n)
{
    int b, j, h, c, g;
    if (B < 0 || L <= 0 || Hkv <= 0 || d <= 0 || n < 0) return -1;
    if (cache_dtype == ORC_E4M3) {
        if (d % 128 != 0 || !k_scale || !v_scale) return -1;
        if (src_dtype != ORC_F32 && src_dtype != ORC_BF16) return -1;
    } else if (cache_dtype == ORC_F32 || cache_dtype == ORC_BF16) {
        if (src_dtype != cache_dtype) return -1;
    } else {
        return -1;
    }
    for (b = 0; b < B; ++b)
        for (j = 0; j < n; ++j) {
            int p = pos[(int64_t)b * n + j];
            if (p < -1 || p >= L) return -1;     /* -1 is padding */
        }

    for (b = 0; b < B; ++b) {
        for (j = 0; j < n; ++j) {
            int p = pos[(int64_t)b * n + j];
            if (p == -1) continue;
            for (h = 0; h < Hkv; ++h) {
                int64_t src_row = (((int64_t)b * n + j) * Hkv + h) * d;
                int64_t dst_row = (((int64_t)b * Hkv + h) * L + p) * d;
                if (cache_dtype == ORC_F32) {
                    memcpy((float *)cache_k + dst_row, (const float *)k_new + src_row, (size_t)d * 4);
                    memcpy((float *)cache_v + dst_row, (const float *)v_new + src_row, (size_t)d * 4);
                } else if (cache_dtype == ORC_BF16) {
                    memcpy((uint16_t *)cache_k + dst_row, (const uint16_t *)k_new + src_row, (size_t)d * 2);
                    memcpy((uint16_t *)cache_v + dst_row, (const uint16_t *)v_new + src_row, (size_t)d * 2);
                } else {
                    /* per-group FP8: one float32 scale per 128 consecutive
                     * elements of a row [LaCache, Methodology 2: 1x128 groups] */
                    float xk[128], xv[128];
                    int ng = d / 128;
                    for (g = 0; g < ng; ++g) {
                        int64_t sidx = (((int64_t)b * Hkv + h) * L + p) * ng + g;
                        for (c = 0; c < 128; ++c) {
                            xk[c] = (float)load_src(src_dtype, k_new, src_row + g * 128 + c);
                            xv[c] = (float)load_src(src_dtype, v_new, src_row + g * 128 + c);
                        }
                        oracle_e4m3_quantize_group(xk, 128, (uint8_t *)cache_k + dst_row + g * 128, &k_scale[sidx]);
                        oracle_e4m3_quantize_group(xv, 128, (uint8_t *)cache_v + dst_row + g * 128, &v_scale[sidx]);
                    }
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* A2: sink + rolling key index map                                          */
/* ------------------------------------------------------------------------ */

int oracle_sink_rolling_keys(int S, int R, int end, int32_t *key_idx)
{
    /* sinks keep their original positions; the rolling part keeps the R
     * newest keys, oldest first [Sinks, 2.3 and 3.2] */
    int k = 0, i, start;
    if (S < 0 || R < 0 || end < 0) return -1;
    for (i = 0; i < S && i < end; ++i) key_idx[k++] = i;
    start = end - R;
    if (start < S) start = S;
    for (i = start; i < end; ++i) key_idx[k++] = i;
    return k;
}

/* ------------------------------------------------------------------------ */
/* A3: block attention                                                       */
/* ------------------------------------------------------------------------ */

/* value of element c of cached row (bh, key) */
static double cache_value(int dtype, const void *cache, const float *scale,
                          int64_t row, int d, int c)
{
    int64_t i = row * d + c;
    if (dtype == ORC_F32) return (double)((const float *)cache)[i];
    if (dtype == ORC_BF16) return oracle_bf16_value(((const uint16_t *)cache)[i]);
    /* e4m3: code times its group's float32 scale, exact in double */
    return oracle_e4m3_value(((const uint8_t *)cache)[i]) *
           (double)scale[row * (d / 128) + c / 128];
}

int oracle_block_attention(int cache_dtype, int B, int L, int Hkv, int d,
                           const void *cache_k, const void *cache_v,
                           const float *k_scale, const float *v_scale,
                           int q_dtype, const void *q, int Hq, int b,
                           const int32_t *key_idx, int n_keys, double scale,
                           double *out, double *lse,
                           const int32_t *heads, int n_heads)
{
    int64_t task, n_tasks;
    int group, err = 0;
    if (B <= 0 || L <= 0 || Hkv <= 0 || d <= 0 || Hq <= 0 || b <= 0) return -1;
    if (Hq % Hkv != 0) return -1;
    if (cache_dtype == ORC_E4M3 && (d % 128 != 0 || !k_scale || !v_scale)) return -1;
    if (!key_idx) n_keys = L;
    if (n_keys <= 0) return -1;
    if (key_idx) {
        int64_t i;
        for (i = 0; i < (int64_t)B * n_keys; ++i)
            if (key_idx[i] < -1 || key_idx[i] >= L) return -1;   /* -1 is padding */
    }
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    group = Hq / Hkv;
    n_tasks = heads ? (int64_t)n_heads : (int64_t)B * Hq;

#pragma omp parallel for schedule(dynamic, 1)
    for (task = 0; task < n_tasks; ++task) {
        int bi, h, kvh, i, j, c;
        double *s = (double *)malloc(sizeof(double) * (size_t)n_keys);
        if (!s) { err = 1; continue; }
        if (heads) { bi = heads[2 * task]; h = heads[2 * task + 1]; }
        else { bi = (int)(task / Hq); h = (int)(task % Hq); }
        kvh = h / group;
        for (i = 0; i < b; ++i) {
            int64_t qrow = (((int64_t)bi * Hq + h) * b + i) * d;
            int64_t orow = (task * b + i) * d;
            double m = -INFINITY, z = 0.0;
            /* scores s_j = scale * q . k_j; a padding key has no score */
            for (j = 0; j < n_keys; ++j) {
                int key = key_idx ? key_idx[(int64_t)bi * n_keys + j] : j;
                int64_t krow = ((int64_t)bi * Hkv + kvh) * L + key;
                double dot = 0.0;
                if (key < 0) { s[j] = -INFINITY; continue; }
                for (c = 0; c < d; ++c)
                    dot += load_src(q_dtype, q, qrow + c) *
                           cache_value(cache_dtype, cache_k, k_scale, krow, d, c);
                s[j] = scale * dot;
                if (s[j] > m) m = s[j];
            }
            for (c = 0; c < d; ++c) out[orow + c] = 0.0;
            if (m == -INFINITY) {                /* only padding: no keys at all */
                if (lse) lse[task * b + i] = -INFINITY;
                continue;
            }
            /* softmax weights and the weighted sum of values */
            for (j = 0; j < n_keys; ++j) {
                s[j] = exp(s[j] - m);
                z += s[j];
            }
            for (j = 0; j < n_keys; ++j) {
                int key = key_idx ? key_idx[(int64_t)bi * n_keys + j] : j;
                int64_t vrow = ((int64_t)bi * Hkv + kvh) * L + key;
                double p = s[j] / z;
                if (key < 0) continue;
                for (c = 0; c < d; ++c)
                    out[orow + c] += p * cache_value(cache_dtype, cache_v, v_scale, vrow, d, c);
            }
            if (lse) lse[task * b + i] = m + log(z);
        }
        free(s);
    }
    return err ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* N1: FACache merge                                                         */
/* ------------------------------------------------------------------------ */

/* The memoized state of a query over the unchanged keys initialises the
 * online softmax; the changed keys are then folded in as one more tile
 * [LaCache, Methodology 1: FACache keeps m, l and O~ of query tiles outside
 * the active block and, when only the KV tile is new, starts from them]. */
int oracle_facache_merge(int cache_dtype, int B, int L, int Hkv, int d,
                         const void *cache_k, const void *cache_v,
                         const float *k_scale, const float *v_scale,
                         int q_dtype, const void *q, int Hq, int n_q,
                         const float *memo_o, const float *memo_lse,
                         const int32_t *key_idx, int n_keys, double scale,
                         double *out, double *lse,
                         const int32_t *heads, int n_heads)
{
    int64_t task, n_tasks;
    int group, err = 0;
    if (B <= 0 || L <= 0 || Hkv <= 0 || d <= 0 || Hq <= 0 || n_q <= 0) return -1;
    if (Hq % Hkv != 0 || !memo_o || !memo_lse) return -1;
    if (cache_dtype == ORC_E4M3 && (d % 128 != 0 || !k_scale || !v_scale)) return -1;
    if (!key_idx) n_keys = L;
    if (n_keys < 0) return -1;
    if (key_idx) {
        int64_t i;
        for (i = 0; i < (int64_t)B * n_keys; ++i)
            if (key_idx[i] < -1 || key_idx[i] >= L) return -1;
    }
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    group = Hq / Hkv;
    n_tasks = heads ? (int64_t)n_heads : (int64_t)B * Hq;

#pragma omp parallel for schedule(dynamic, 1)
    for (task = 0; task < n_tasks; ++task) {
        int bi, h, kvh, i, j, c;
        double *s = (double *)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !acc) { free(s); free(acc); err = 1; continue; }
        if (heads) { bi = heads[2 * task]; h = heads[2 * task + 1]; }
        else { bi = (int)(task / Hq); h = (int)(task % Hq); }
        kvh = h / group;
        for (i = 0; i < n_q; ++i) {
            int64_t row = ((int64_t)bi * Hq + h) * n_q + i;
            int64_t qrow = row * d;
            int64_t orow = (task * n_q + i) * d;
            /* the memoized state: m' = lse, l' = 1, O~' = O (or empty) */
            double m0 = (double)memo_lse[row];
            double l0 = m0 == -INFINITY ? 0.0 : 1.0;
            double m_new = m0, l_new, f0;
            /* scores of the changed keys */
            for (j = 0; j < n_keys; ++j) {
                int key = key_idx ? key_idx[(int64_t)bi * n_keys + j] : j;
                int64_t krow = ((int64_t)bi * Hkv + kvh) * L + key;
                double dot = 0.0;
                if (key < 0) { s[j] = -INFINITY; continue; }
                for (c = 0; c < d; ++c)
                    dot += load_src(q_dtype, q, qrow + c) *
                           cache_value(cache_dtype, cache_k, k_scale, krow, d, c);
                s[j] = scale * dot;
                if (s[j] > m_new) m_new = s[j];
            }
            if (m_new == -INFINITY) {            /* empty memo and no key */
                for (c = 0; c < d; ++c) out[orow + c] = 0.0;
                if (lse) lse[task * n_q + i] = -INFINITY;
                continue;
            }
            /* rescale the memo to the new reference, then add the keys */
            f0 = l0 > 0.0 ? exp(m0 - m_new) : 0.0;
            l_new = l0 * f0;
            for (c = 0; c < d; ++c) acc[c] = l0 > 0.0 ? (double)memo_o[qrow + c] * f0 : 0.0;
            for (j = 0; j < n_keys; ++j) {
                int key = key_idx ? key_idx[(int64_t)bi * n_keys + j] : j;
                int64_t vrow = ((int64_t)bi * Hkv + kvh) * L + key;
                double p;
                if (key < 0) continue;
                p = exp(s[j] - m_new);
                l_new += p;
                for (c = 0; c < d; ++c)
                    acc[c] += p * cache_value(cache_dtype, cache_v, v_scale, vrow, d, c);
            }
            for (c = 0; c < d; ++c) out[orow + c] = acc[c] / l_new;
            if (lse) lse[task * n_q + i] = m_new + log(l_new);
        }
        free(s);
        free(acc);
    }
    return err ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* N2: per-group FP8 for the FFN                                             */
/* ------------------------------------------------------------------------ */

/* The group's scale is a power of two 2^e, stored as its E8M0 code e + 127:
 * the smallest e >= -127 with amax <= 448 * 2^e, so no code saturates.
 * With amax = f * 2^E, f in [0.5, 1) and 448 = 0.875 * 2^9, that is
 * e = E - 9 when f <= 0.875, else E - 8. */
int oracle_e8m0_exponent(double amax)
{
    int E, e;
    double f;
    if (!(amax > 0.0)) return -127;
    f = frexp(amax, &E);
    e = f <= 0.875 ? E - 9 : E - 8;
    return e < -127 ? -127 : e;
}

double oracle_e8m0_value(uint8_t code)
{
    return ldexp(1.0, (int)code - 127);
}

void oracle_fp8_quantize_pow2(const double *x, int n, uint8_t *codes, uint8_t *e8m0)
{
    double amax = 0.0;
    int i, e;
    for (i = 0; i < n; ++i)
        if (fabs(x[i]) > amax) amax = fabs(x[i]);
    e = oracle_e8m0_exponent(amax);
    *e8m0 = (uint8_t)(e + 127);
    for (i = 0; i < n; ++i)
        codes[i] = e4m3_encode_double(ldexp(x[i], -e));   /* exact: a power of two */
}

/* activations: every 1 x 128 group of a row [LaCache, Methodology 2] */
int oracle_fp8_quant_rows(int dtype, const void *x, int64_t M, int K, int64_t ld,
                          uint8_t *codes, uint8_t *scales)
{
    int64_t m;
    if (M < 0 || K <= 0 || K % 128 != 0 || ld < K) return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16 && dtype != ORC_F64) return -1;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        double g[128];
        int gi, c;
        for (gi = 0; gi < K / 128; ++gi) {
            for (c = 0; c < 128; ++c) {
                int64_t i = m * ld + gi * 128 + c;
                g[c] = dtype == ORC_F64 ? ((const double *)x)[i] : load_src(dtype, x, i);
            }
            oracle_fp8_quantize_pow2(g, 128, codes + m * K + gi * 128, scales + (int64_t)gi * M + m);
        }
    }
    return 0;
}

/* weights: every 128 x 128 block [LaCache, Methodology 2] */
int oracle_fp8_quant_weight(int dtype, const void *w, int N, int K, uint8_t *codes, uint8_t *scales)
{
    int64_t blk;
    const int nb = N / 128, kb = K / 128;
    if (N <= 0 || K <= 0 || N % 128 != 0 || K % 128 != 0) return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16) return -1;
#pragma omp parallel for schedule(static)
    for (blk = 0; blk < (int64_t)nb * kb; ++blk) {
        const int bn = (int)(blk / kb), bk = (int)(blk % kb);
        double amax = 0.0, v;
        int r, c, e;
        for (r = 0; r < 128; ++r)
            for (c = 0; c < 128; ++c) {
                v = fabs(load_src(dtype, w, (int64_t)(bn * 128 + r) * K + bk * 128 + c));
                if (v > amax) amax = v;
            }
        e = oracle_e8m0_exponent(amax);
        scales[blk] = (uint8_t)(e + 127);
        for (r = 0; r < 128; ++r)
            for (c = 0; c < 128; ++c) {
                int64_t i = (int64_t)(bn * 128 + r) * K + bk * 128 + c;
                codes[i] = e4m3_encode_double(ldexp(load_src(dtype, w, i), -e));
            }
    }
    return 0;
}

/* C = dequant(A) dequant(B)^T in fp64: element (m, k) of A is
 * e4m3(a[m, k]) * 2^(sa[k/128, m] - 127), element (n, k) of B is
 * e4m3(b[n, k]) * 2^(sb[n/128, k/128] - 127).  rows selects output rows. */
int oracle_fp8_gemm(const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb,
                    int64_t M, int N, int K, const int64_t *rows, int64_t n_rows, double *c)
{
    int64_t t, n_out = rows ? n_rows : M;
    double *bd;
    int64_t i;
    if (M <= 0 || N <= 0 || K <= 0 || N % 128 != 0 || K % 128 != 0) return -1;
    bd = (double *)malloc(sizeof(double) * (size_t)N * K);
    if (!bd) return -1;
    for (i = 0; i < (int64_t)N * K; ++i) {
        const int n = (int)(i / K), k = (int)(i % K);
        bd[i] = oracle_e4m3_value(b[i]) * oracle_e8m0_value(sb[(n / 128) * (K / 128) + k / 128]);
    }
#pragma omp parallel for schedule(dynamic, 4)
    for (t = 0; t < n_out; ++t) {
        const int64_t m = rows ? rows[t] : t;
        double *ad = (double *)malloc(sizeof(double) * (size_t)K);
        int n, k;
        if (!ad) continue;
        for (k = 0; k < K; ++k)
            ad[k] = oracle_e4m3_value(a[m * K + k]) * oracle_e8m0_value(sa[(int64_t)(k / 128) * M + m]);
        for (n = 0; n < N; ++n) {
            double acc = 0.0;
            const double *br = bd + (int64_t)n * K;
            for (k = 0; k < K; ++k) acc += ad[k] * br[k];
            c[t * N + n] = acc;
        }
        free(ad);
    }
    free(bd);
    return 0;
}

/* Add & norm before the FFN: r = x + res in float32, stored in the source
 * dtype (the residual stream), then y = gamma * r / sqrt(mean(r^2) + eps)
 * in fp64 (RMS normalisation). */
int oracle_addnorm(int dtype, const void *x, const void *res, const void *gamma, double eps,
                   int64_t M, int K, void *res_out, double *y)
{
    int64_t m;
    if (M < 0 || K <= 0 || (dtype != ORC_F32 && dtype != ORC_BF16)) return -1;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        double ss = 0.0, inv;
        int k;
        for (k = 0; k < K; ++k) {
            const int64_t i = m * K + k;
            float r = (float)load_src(dtype, x, i) + (float)(res ? load_src(dtype, res, i) : 0.0);
            double rv;
            if (dtype == ORC_BF16) {
                uint32_t u;
                uint16_t h;
                memcpy(&u, &r, sizeof u);
                /* round to nearest even into bfloat16 (inputs are finite) */
                u += 0x7fffu + ((u >> 16) & 1u);
                h = (uint16_t)(u >> 16);
                if (res_out) ((uint16_t *)res_out)[i] = h;
                rv = oracle_bf16_value(h);
            } else {
                if (res_out) ((float *)res_out)[i] = r;
                rv = (double)r;
            }
            y[i] = rv;
            ss += rv * rv;
        }
        inv = 1.0 / sqrt(ss / K + eps);
        for (k = 0; k < K; ++k)
            y[m * K + k] = y[m * K + k] * inv * load_src(dtype, gamma, k);
    }
    return 0;
}

/* SwiGLU: silu(g) * u with silu(g) = g / (1 + e^-g) */
double oracle_silu(double g)
{
    return g / (1.0 + exp(-g));
}

void oracle_swiglu(const double *g, const double *u, int64_t n, double *y)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) y[i] = oracle_silu(g[i]) * u[i];
}

/* ------------------------------------------------------------------------ */
/* A4: vocab statistics                                                      */
/* ------------------------------------------------------------------------ */

int oracle_vocab_stats(int dtype, const void *logits, int64_t N, int64_t V,
                       int64_t row_stride, int32_t *argmax, double *maxprob,
                       double *entropy, const int64_t *rows, int64_t n_rows)
{
    int64_t t, n_out;
    if (N < 0 || V <= 0 || row_stride < V) return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16) return -1;
    n_out = rows ? n_rows : N;
    if (rows) {
        for (t = 0; t < n_rows; ++t)
            if (rows[t] < 0 || rows[t] >= N) return -1;
    }

#pragma omp parallel for schedule(dynamic, 4)
    for (t = 0; t < n_out; ++t) {
        int64_t r = rows ? rows[t] : t;
        int64_t base = r * row_stride, j, best = 0;
        double m = -INFINITY, z = 0.0, h = 0.0;
        /* the largest logit, lowest index first */
        for (j = 0; j < V; ++j) {
            double x = load_src(dtype, logits, base + j);
            if (x > m) { m = x; best = j; }
        }
        /* normaliser of the softmax */
        for (j = 0; j < V; ++j)
            z += exp(load_src(dtype, logits, base + j) - m);
        /* entropy -sum p ln p; a zero probability adds nothing */
        for (j = 0; j < V; ++j) {
            double p = exp(load_src(dtype, logits, base + j) - m) / z;
            if (p > 0.0) h -= p * log(p);
        }
        argmax[t] = (int32_t)best;
        maxprob[t] = exp(load_src(dtype, logits, base + best) - m) / z;
        entropy[t] = h;
    }
    return 0;
}

/* Validity of a scatter's position list ([Sinks, 5.1]: rows written to the
 * wrong cache slot corrupt every later step): per sequence, the entries
 * outside [0, L) other than the padding -1, and the entries equal to an
 * earlier entry of the same sequence. */
int oracle_check_positions(int B, int L, const int32_t *pos, int n, int32_t *bad, int32_t *dup)
{
    int b, j, i;
    if (B <= 0 || L <= 0 || n < 0) return -1;
    for (b = 0; b < B; ++b) {
        const int32_t *row = pos + (int64_t)b * n;
        int nb = 0, nd = 0;
        for (j = 0; j < n; ++j) {
            int p = row[j];
            if (p == -1) continue;
            if (p < 0 || p >= L) { ++nb; continue; }
            for (i = 0; i < j; ++i)
                if (row[i] == p) { ++nd; break; }
        }
        bad[b] = nb;
        dup[b] = nd;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* A5-A7: history ring, stability test, confidence, window mask             */
/* ------------------------------------------------------------------------ */

/* ------------------------------------------------------------------------ */
/* N3: radius and refresh schedules, eviction under a budget                 */
/* ------------------------------------------------------------------------ */

/* [SWD, 4.4]: small (or no) window early, wider late.  The reading: a
 * linear ramp from R_early at step 0 to R at step T-1, in whole positions
 * (integer division), R afterwards; T <= 1 keeps R throughout. */
int oracle_dynamic_radius(int R_early, int R, int T, int step)
{
    int s;
    if (T <= 1) return R;
    s = step < T - 1 ? step : T - 1;
    return R_early + (R - R_early) * s / (T - 1);
}

/* [Flash, 5.1]: a full refresh every F steps; F = 0 never.  Step 0
 * recomputes everything anyway. */
int oracle_is_refresh_step(int F, int step)
{
    return F > 0 && step > 0 && step % F == 0;
}

/* [Flash, 5.1]: T in 50..100 -> every 5..10 steps, T < 50 -> every 3..5.
 * The reading: F = round(T / 10), kept within [3, 10]. */
int oracle_refresh_interval(int T)
{
    int f = (int)floor((double)T / 10.0 + 0.5);
    return f < 3 ? 3 : (f > 10 ? 10 : f);
}

/* [Flash, 5.2]: each request is guaranteed ceil(min_frac * len) cached
 * positions (min_frac = 0.2 on the page); what the budget has left goes to
 * the requests in arrival order (index order), each up to its length.
 * Returns -1 when the budget cannot cover the guarantees. */
int oracle_cache_quotas(int B, const int32_t *len, int64_t budget, double min_frac, int32_t *quota)
{
    int b;
    int64_t need = 0, left;
    if (B <= 0 || budget < 0 || !(min_frac >= 0.0)) return -1;
    for (b = 0; b < B; ++b) {
        double m = ceil(min_frac * (double)len[b]);
        if (len[b] < 0) return -1;
        quota[b] = (int32_t)(m > (double)len[b] ? (double)len[b] : m);
        need += quota[b];
    }
    if (need > budget) return -1;
    left = budget - need;
    for (b = 0; b < B; ++b) {
        int64_t extra = (int64_t)len[b] - quota[b];
        if (extra > left) extra = left;
        quota[b] += (int32_t)extra;
        left -= extra;
    }
    return 0;
}

/* ordering of eviction candidates: higher confidence first, then lower
 * position */
typedef struct { float conf; int pos; } orc_cand;
static int cand_order(const void *x, const void *y)
{
    const orc_cand *a = (const orc_cand *)x, *b = (const orc_cand *)y;
    if (a->conf > b->conf) return -1;
    if (a->conf < b->conf) return 1;
    return a->pos - b->pos;
}

/* [Flash, 3.3]: when a sequence's cached positions exceed its quota, the
 * lowest-confidence positions leave the cache first, a position's K and V
 * together.  Positions recomputed this step (pos, NULL for all L) hold fresh
 * K/V and count as cached; of the cached positions the quota[b] with the
 * highest confidence (ties: lower position) stay, quota < 0 meaning no
 * limit.  A position without cached K/V must be recomputed before it can be
 * attended to, so every uncached position joins the next step's mask, and
 * next_pos / count are compacted again.  evicted[b] counts the positions
 * this call evicted. */
int oracle_evict_by_confidence(int B, int L, const float *conf, const int32_t *quota,
                               const int32_t *pos, int n, uint8_t *cached, uint8_t *mask,
                               int32_t *next_pos, int32_t *count, int32_t *evicted)
{
    int b;
    if (B <= 0 || L <= 0) return -1;
    if (!pos) n = L;
    if (n < 0 || n > L) return -1;
    for (b = 0; b < B; ++b) {
        int64_t row = (int64_t)b * L;
        int i, j, nc = 0, c, ev = 0;
        orc_cand *cand = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)L);
        if (!cand) return -1;
        for (j = 0; j < n; ++j) {
            int p = pos ? pos[(int64_t)b * n + j] : j;
            if (p >= 0 && p < L) cached[row + p] = 1;
        }
        for (i = 0; i < L; ++i)
            if (cached[row + i]) { cand[nc].conf = conf[row + i]; cand[nc].pos = i; ++nc; }
        if (quota[b] >= 0 && nc > quota[b]) {
            qsort(cand, (size_t)nc, sizeof(orc_cand), cand_order);
            for (j = quota[b]; j < nc; ++j) { cached[row + cand[j].pos] = 0; ++ev; }
        }
        evicted[b] = ev;
        for (i = 0; i < L; ++i)
            if (!cached[row + i]) mask[row + i] = 1;
        c = 0;
        for (i = 0; i < L; ++i)
            if (mask[row + i]) next_pos[row + c++] = i;
        count[b] = c;
        for (i = c; i < L; ++i) next_pos[row + i] = -1;
        free(cand);
    }
    return 0;
}

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
                          int32_t *count, uint8_t *all_stable)
{
    int b, R_eff;
    double hmax;
    if (B <= 0 || L <= 0 || step < 0 || K < 1 || D < K || R < 0 || V < 2) return -1;
    if (n_decay < 1) return -1;
    if (R_early < 0 || refresh_every < 0) return -1;
    if (!pos) n = L;
    if (n < 0 || n > L) return -1;
    if (pos) {
        int64_t i;
        for (i = 0; i < (int64_t)B * n; ++i)
            if (pos[i] < -1 || pos[i] >= L) return -1;     /* -1 is padding */
    }
    hmax = log((double)V);                    /* entropy of the uniform row */
    R_eff = oracle_dynamic_radius(R_early, R, T_steps, step);

    for (b = 0; b < B; ++b) {
        int j, i, k, c;
        int64_t row = (int64_t)b * L;
        int slot = step % D;
        uint8_t *seed = (uint8_t *)calloc((size_t)L, 1);
        int any_seed = 0;
        if (!seed) return -1;

        /* (c) record this step's prediction for every recomputed position
         * [SWD, 3.3 step c]; the position's K/V were written at this step */
        for (j = 0; j < n; ++j) {
            int p = pos ? pos[(int64_t)b * n + j] : j;
            int64_t ri = (int64_t)slot * B * L + row + p;
            if (p < 0) continue;
            ring_argmax[ri] = argmax[(int64_t)b * n + j];
            ring_maxprob[ri] = maxprob[(int64_t)b * n + j];
            ring_step[ri] = step;
            entropy_latest[row + p] = entropy[(int64_t)b * n + j];
            t_write[row + p] = step;
        }

        /* (d) a position not yet stable becomes stable when its last K
         * records are the steps s, s-1, ..., s-K+1, all with the same token,
         * and the mean of their max-probabilities exceeds tau
         * [SWD, 3.1 criterion; 4.2 update_stability]; stable is sticky */
        for (j = 0; j < n; ++j) {
            int p = pos ? pos[(int64_t)b * n + j] : j;
            int ok = 1, tok;
            double sum = 0.0, mean;
            if (p < 0 || stable[row + p]) continue;
            if (step + 1 < K) continue;              /* fewer than K steps so far */
            tok = ring_argmax[(int64_t)slot * B * L + row + p];
            for (k = K - 1; k >= 0; --k) {           /* oldest record first */
                int sk = (step - k) % D;
                int64_t ri = (int64_t)sk * B * L + row + p;
                if (ring_step[ri] != step - k || ring_argmax[ri] != tok) { ok = 0; break; }
                sum += (double)ring_maxprob[ri];
            }
            if (!ok) continue;
            mean = sum / (double)K;
            if (mean > tau) stable[row + p] = 1;
        }

        /* cache confidence alpha(1 - H/Hmax) + beta exp(-lambda (s - t_write))
         * for every position; below the threshold its cache is refreshed
         * [Flash, 3.1].  The age is clamped to [0, n_decay - 1]. */
        for (i = 0; i < L; ++i) {
            double h = (double)entropy_latest[row + i];
            int age = step - t_write[row + i];
            double dt, cf;
            if (age < 0) age = 0;
            if (age > n_decay - 1) age = n_decay - 1;
            dt = (double)age;
            cf = alpha * (1.0 - h / hmax) + beta * exp(-lambda * dt);
            int low = cf < conf_thresh;
            conf[row + i] = cf;
            seed[i] = (uint8_t)(!stable[row + i] || low);
            if (seed[i]) any_seed = 1;
        }

        /* window: each seed position u covers [max(0, u-R), min(L-1, u+R)];
         * nothing to recompute -> full mask and the all-stable flag
         * [SWD, 3.2; 4.2 get_computation_mask] */
        for (i = 0; i < L; ++i) mask[row + i] = 0;
        if (!any_seed || oracle_is_refresh_step(refresh_every, step)) {
            /* nothing left to recompute, or a scheduled full refresh
             * [Flash, 5.1]: the whole sequence */
            for (i = 0; i < L; ++i) mask[row + i] = 1;
        } else {
            for (i = 0; i < L; ++i) {
                int lo, hi, u;
                if (!seed[i]) continue;
                lo = i - R_eff < 0 ? 0 : i - R_eff;
                hi = i + R_eff > L - 1 ? L - 1 : i + R_eff;
                for (u = lo; u <= hi; ++u) mask[row + u] = 1;
            }
        }
        all_stable[b] = (uint8_t)(!any_seed);

        /* positions to recompute next step, ascending */
        c = 0;
        for (i = 0; i < L; ++i)
            if (mask[row + i]) next_pos[row + c++] = i;
        count[b] = c;
        for (i = c; i < L; ++i) next_pos[row + i] = -1;
        free(seed);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* N4: self-verification of tokens decoded in parallel                       */
/* ------------------------------------------------------------------------ */

/* [Flash, 4.1]: many positions per step early in the trajectory (8-16 on the
 * page), few late (2-4).  The reading: a linear ramp in whole positions from
 * w_early at step 0 to w_late at step T-1 (integer division, rounding toward
 * w_early), w_late afterwards; T <= 1 keeps w_late. */
int oracle_parallel_width(int w_early, int w_late, int T, int step)
{
    int s;
    if (T <= 1) return w_late;
    s = step < T - 1 ? step : T - 1;
    return w_early - (w_early - w_late) * s / (T - 1);
}

/* [Flash, 4.2-4.3]: for two positions decoded in the same step, at most W-1
 * apart (a window of W consecutive positions), the conflict score is the
 * pair's joint probability over the product of the two marginals; a score
 * below tau is a conflict (a zero product never is).  Every position decoded
 * this step that lies between the two (both included) is withdrawn: it is
 * regenerated serially, so its stable flag and its cached K/V are dropped and
 * it joins the next step's mask.
 *   dec_pos [B, n]: positions decoded this step, ascending, then -1 padding
 *   p_marg  [B, n]: the probability of each decoded token
 *   p_joint [B, n, W-1]: entry (j, d-1) is P(token at dec_pos[j], token at
 *                        dec_pos[j]+d), read when that position is decoded too
 * Outputs: rollback [B, L] (1 = withdrawn), n_rollback [B], rb_pos [B, n]
 * (withdrawn positions ascending, -1 after); mask |= rollback, stable and
 * cached (either may be NULL) cleared at withdrawn positions; next_pos and
 * count recompacted from the mask. */
int oracle_self_verify(int B, int L, const int32_t *dec_pos, int n, const float *p_marg,
                       const float *p_joint, int W, double tau, uint8_t *rollback,
                       uint8_t *mask, uint8_t *stable, uint8_t *cached, int32_t *next_pos,
                       int32_t *count, int32_t *n_rollback, int32_t *rb_pos)
{
    int b;
    if (B <= 0 || L <= 0 || n < 0 || W < 2 || !(tau >= 0.0)) return -1;
    for (b = 0; b < B; ++b) {
        int64_t row = (int64_t)b * L;
        const int32_t *dp = dec_pos + (int64_t)b * n;
        const float *pm = p_marg + (int64_t)b * n;
        int j, k, d, i, c, nr, nv = 0;
        /* the decoded positions ascending, then -1 padding (the order in
         * which a step's compacted mask lists them) */
        while (nv < n && dp[nv] >= 0) ++nv;
        for (j = 0; j < n; ++j) {
            if (j < nv && (dp[j] >= L || (j + 1 < nv && dp[j + 1] <= dp[j]))) return -1;
            if (j >= nv && dp[j] != -1) return -1;
        }
        for (i = 0; i < L; ++i) rollback[row + i] = 0;
        for (j = 0; j < n; ++j) {
            if (dp[j] < 0) continue;
            for (d = 1; d < W; ++d) {
                int partner = -1;
                for (k = 0; k < n; ++k)
                    if (dp[k] == dp[j] + d) { partner = k; break; }
                if (partner < 0) continue;
                {
                    double prod = (double)pm[j] * (double)pm[partner];
                    double joint = (double)p_joint[((int64_t)b * n + j) * (W - 1) + (d - 1)];
                    if (prod > 0.0 && joint / prod < tau) {
                        /* withdraw every decoded position in [dp[j], dp[j] + d] */
                        for (k = 0; k < n; ++k)
                            if (dp[k] >= dp[j] && dp[k] <= dp[j] + d) rollback[row + dp[k]] = 1;
                    }
                }
            }
        }
        nr = 0;
        for (i = 0; i < L; ++i) {
            if (!rollback[row + i]) continue;
            mask[row + i] = 1;
            if (stable) stable[row + i] = 0;
            if (cached) cached[row + i] = 0;
            if (rb_pos && nr < n) rb_pos[(int64_t)b * n + nr] = i;
            ++nr;
        }
        if (rb_pos)
            for (k = nr; k < n; ++k) rb_pos[(int64_t)b * n + k] = -1;
        if (n_rollback) n_rollback[b] = nr;
        c = 0;
        for (i = 0; i < L; ++i)
            if (mask[row + i]) next_pos[row + c++] = i;
        count[b] = c;
        for (i = c; i < L; ++i) next_pos[row + i] = -1;
    }
    return 0;
}
