/*
 * oracle.c -- plain, slow CPU reference of the BitNet v2 H-BitLinear forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark load it.  It shares no code, header or constant with the HIP
 * path.
 *
 * Sources (the pages print no formula; every formula image is missing, so the
 * steps below are the plain reading of the surrounding text):
 *   [QbitAI]  量子位 article on BitNet v2, section 引入H-BitLinear模块
 *   [XZY]     新智元 article "微软再放LLM量化大招！原生4bit量化...", sections
 *             BitNet v2：原生4位激活 and H-BitLinear模块
 *   [AINEWS]  "微软LLM量化再突破：BitNet v2实现原生4bit..." section
 *             揭秘核心魔法：H-BitLinear与Hadamard变换
 *   [DIGEST]  "BitNet v2: Native 4-bit Activations with Hadamard Transformation
 *             for 1-bit LLMs" (arXiv digest page), abstract and 方法详解
 *   Variants beside H-BitLinear (same quantisers and matmul):
 *     BitLinear without the rotation, for the layers whose inputs are already
 *       close to Gaussian (attention/FFN input projections) [XZY §H-BitLinear模块];
 *     weights rotated offline as well (weight + activation rotation, the
 *       ablation of [XZY §实验效果], table 5).
 *   Backward pass [QbitAI §引入H-BitLinear模块] (training paragraph): the
 *     quantisers are bypassed (straight-through estimator) and the gradient
 *     goes through the transposed Hadamard transform, which is the transform.
 *   Low-bit attention states [XZY §实验效果], [QbitAI]: post-RoPE Q/K/V heads
 *     quantised per head by absmax to unsigned integers (3-bit KV cache), and
 *     one decode step of attention over that cache.
 *
 * Parity unpinned by the pages: the INT4 multiplier sqrt(7) (see Q4 below);
 * every function is otherwise pinned by the tests in test_oracle_pins.py.
 *
 * Precision: every floating-point step is done in double; values are rounded
 * only where the method itself produces a stored low-precision quantity
 * (the per-tensor weight scale, the integer codes) -- see each function.
 * Rounding is round-half-to-even (nearbyint under the default FE_TONEAREST).
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC
 * OpenMP is used only across tokens (rows), never inside one token.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Constants of the specification (the pages give none; readings listed in the
 * design notes).  RMSNorm epsilon is added to the mean square; the quantiser
 * floor is applied to the per-tensor / per-token statistic. */
static const double EPS_NORM = 1e-6;
static const double EPS_Q = 1e-5;
static const double Q8 = 127.0;      /* INT8 absmax: max |x| maps to code 127 */
/* INT4 absmean multiplier: sqrt(7) (reading; not printed on the pages, so
 * this constant is parity unpinned by the pages: the tests pin every
 * consequence of it -- hand-worked codes, Gaussian code-edge frequencies --
 * but no page fixes the value itself). */
#define Q4 (sqrt(7.0))

int oracle_version(void) { return 1; }

static double rne(double v) { return nearbyint(v); }

static double clampd(double v, double lo, double hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

/* ---------------------------------------------------------------------------
 * Weights: per-tensor absmean ternarisation to {-1, 0, 1}.
 * [QbitAI §引入H-BitLinear模块], [XZY §H-BitLinear模块], [AINEWS].
 *   S      = sum of |w| over the whole tensor in double: each row summed
 *            left to right, then the row sums added in row order (a plain
 *            ordered sum; its rounding error is far below fp32's);
 *   alpha  = (float)(S / (N*K))       -- the stored per-tensor scale (fp32);
 *   a      = max(alpha, EPS_Q);
 *   w_t    = clamp(round(w / a), -1, 1)  (w / a in double).
 * Returns 0, or -1 on bad arguments.
 * ------------------------------------------------------------------------- */
/* Sum of |v| over one row, left to right. */
static double row_abs_sum_f(const float *v, int64_t K)
{
    double row = 0.0;
    for (int64_t k = 0; k < K; ++k) row += fabs((double)v[k]);
    return row;
}

static double row_abs_sum_d(const double *v, int64_t K)
{
    double row = 0.0;
    for (int64_t k = 0; k < K; ++k) row += fabs(v[k]);
    return row;
}

int oracle_quantize_weights(const float *w, int64_t N, int64_t K, int8_t *wt, float *alpha_out)
{
    if (!w || !wt || !alpha_out || N <= 0 || K <= 0) return -1;
    double S = 0.0;
    for (int64_t n = 0; n < N; ++n) S += row_abs_sum_f(w + n * K, K);
    float alpha = (float)(S / ((double)N * (double)K));
    double a = (double)alpha;
    if (a < EPS_Q) a = (double)(float)EPS_Q;
    for (int64_t i = 0; i < N * K; ++i)
        wt[i] = (int8_t)clampd(rne((double)w[i] / a), -1.0, 1.0);
    *alpha_out = alpha;
    return 0;
}

/* The effective weight scale used for both ternarising and dequantising. */
double oracle_weight_scale(float alpha)
{
    double a = (double)alpha;
    if (a < EPS_Q) a = (double)(float)EPS_Q;
    return a;
}

/* ---------------------------------------------------------------------------
 * RMSNorm (the "LN" inside H-BitLinear; the stack is LLaMA-like with RMS
 * normalisation and no bias) [XZY §BitNet v2：原生4位激活], [QbitAI].
 *   r = sqrt(mean_k x_k^2 + EPS_NORM),   u_k = x_k * g_k / r     (g = 1 if NULL)
 * ------------------------------------------------------------------------- */
int oracle_rmsnorm(const float *x, const float *g, int64_t K, double *u)
{
    if (!x || !u || K <= 0) return -1;
    double ss = 0.0;
    for (int64_t k = 0; k < K; ++k) ss += (double)x[k] * (double)x[k];
    double r = sqrt(ss / (double)K + EPS_NORM);
    for (int64_t k = 0; k < K; ++k) {
        double gk = g ? (double)g[k] : 1.0;
        u[k] = (double)x[k] * gk / r;
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Walsh-Hadamard transform by its recursive definition (Sylvester order):
 *   F(v) = v                         if len(v) == 1
 *   F(v) = [F(a) + F(b), F(a) - F(b)] with a, b the first and second halves.
 * This is H_n v with H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]], i.e.
 * H[i][j] = (-1)^popcount(i & j); entries +-1 and H H^T = n I
 * [XZY §H-BitLinear模块] (entries +-1, rows mutually orthogonal, computed by the
 * fast O(n log n) transform).  Unnormalised; in place; n a power of two.
 * ------------------------------------------------------------------------- */
static void fwht_rec(double *v, int64_t n)
{
    if (n == 1) return;
    int64_t h = n / 2;
    fwht_rec(v, h);
    fwht_rec(v + h, h);
    for (int64_t i = 0; i < h; ++i) {
        double a = v[i], b = v[h + i];
        v[i] = a + b;
        v[h + i] = a - b;
    }
}

static int is_pow2(int64_t n) { return n > 0 && (n & (n - 1)) == 0; }

int oracle_fwht(double *v, int64_t n)
{
    if (!v || !is_pow2(n)) return -1;
    fwht_rec(v, n);
    return 0;
}

/* Online Hadamard rotation applied to the activations before quantisation,
 * scaled to be orthogonal:  xt = H_K u / sqrt(K)
 * [QbitAI §引入H-BitLinear模块], [AINEWS], [DIGEST abstract]. */
int oracle_hadamard_rotate(const double *u, int64_t K, double *xt)
{
    if (!u || !xt || !is_pow2(K)) return -1;
    memcpy(xt, u, (size_t)K * sizeof(double));
    fwht_rec(xt, K);
    double s = sqrt((double)K);
    for (int64_t k = 0; k < K; ++k) xt[k] = xt[k] / s;
    return 0;
}

/* ---------------------------------------------------------------------------
 * Per-token activation quantisation [QbitAI §引入H-BitLinear模块],
 * [XZY §H-BitLinear模块]: 8-bit uses the per-token absmax, 4-bit the per-token
 * absmean.
 *   INT8:  stat = max_k |xt_k|,        Q = 127,     codes in [-128, 127]
 *   INT4:  stat = mean_k |xt_k|,       Q = sqrt(7), codes in [-8, 7]
 *   G = max(stat, EPS_Q);  pre_k = xt_k * (Q / G);  q_k = clamp(round(pre_k));
 *   dequant scale d = G / Q.
 * pre (optional) receives the pre-rounding values (used by the tests to show
 * that code differences sit at rounding ties).
 * ------------------------------------------------------------------------- */
int oracle_quant_act(const double *xt, int64_t K, int bits, int8_t *q, double *d, double *pre)
{
    if (!xt || !q || !d || K <= 0 || (bits != 8 && bits != 4)) return -1;
    double stat = 0.0, Q, lo, hi;
    if (bits == 8) {
        for (int64_t k = 0; k < K; ++k) if (fabs(xt[k]) > stat) stat = fabs(xt[k]);
        Q = Q8; lo = -128.0; hi = 127.0;
    } else {
        for (int64_t k = 0; k < K; ++k) stat += fabs(xt[k]);
        stat = stat / (double)K;
        Q = Q4; lo = -8.0; hi = 7.0;
    }
    double G = stat > EPS_Q ? stat : EPS_Q;
    double s = Q / G;
    for (int64_t k = 0; k < K; ++k) {
        double v = xt[k] * s;
        if (pre) pre[k] = v;
        q[k] = (int8_t)clampd(rne(v), lo, hi);
    }
    *d = G / Q;
    return 0;
}

/* ---------------------------------------------------------------------------
 * Ternary integer matmul: acc[m][n] = sum_k q[m][k] * w_t[n][k]  (exact, int32).
 * Weights are [N][K] (out x in).  Naive triple loop.
 * ------------------------------------------------------------------------- */
int oracle_gemm_ternary(const int8_t *q, const int8_t *wt, int64_t M, int64_t N, int64_t K,
                        int32_t *acc, int nthreads)
{
    if (!q || !wt || !acc || M < 0 || N <= 0 || K <= 0) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int32_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int32_t)q[m * K + k] * (int32_t)wt[n * K + k];
            acc[m * N + n] = s;
        }
    return 0;
}

/* Dequantisation with the activation and weight scales:
 *   y[m][n] = acc[m][n] * d[m] * a,  a = max(alpha, EPS_Q). */
int oracle_dequant(const int32_t *acc, const double *d, float alpha, int64_t M, int64_t N, double *y)
{
    if (!acc || !d || !y || M < 0 || N <= 0) return -1;
    double a = oracle_weight_scale(alpha);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = (double)acc[m * N + n] * d[m] * a;
    return 0;
}

/* ---------------------------------------------------------------------------
 * Whole forward, token by token: RMSNorm -> Hadamard rotation -> quantise ->
 * ternary matmul -> dequantise [QbitAI §引入H-BitLinear模块] (the layer is the
 * quantised matmul of the normalised, rotated activations), [DIGEST 方法详解]
 * (input -> Hadamard -> quantise -> rest).
 * x [M][K] fp32; g [K] or NULL; wt [N][K]; outputs (each optional except y):
 *   xt [M][K] double, q [M][K] int8, d [M] double, pre [M][K] double,
 *   acc [M][N] int32, y [M][N] double.
 * ------------------------------------------------------------------------- */
int oracle_forward_ex(const float *x, const float *g, const int8_t *wt, float alpha,
                      int64_t M, int64_t K, int64_t N, int bits, int rotate,
                      double *xt, int8_t *q, double *d, double *pre, int32_t *acc, double *y,
                      int nthreads)
{
    if (!x || !wt || !y || M < 0 || N <= 0 || !is_pow2(K) || (bits != 8 && bits != 4)) return -1;
    double a = oracle_weight_scale(alpha);
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
#endif
    for (int64_t m = 0; m < M; ++m) {
        double *u = (double *)malloc((size_t)K * sizeof(double));
        double *t = (double *)malloc((size_t)K * sizeof(double));
        int8_t *qm = (int8_t *)malloc((size_t)K);
        if (!u || !t || !qm) { bad = 1; free(u); free(t); free(qm); continue; }
        double dm;
        oracle_rmsnorm(x + m * K, g, K, u);
        if (rotate) oracle_hadamard_rotate(u, K, t);
        else memcpy(t, u, (size_t)K * sizeof(double));
        oracle_quant_act(t, K, bits, qm, &dm, pre ? pre + m * K : NULL);
        for (int64_t n = 0; n < N; ++n) {
            int32_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int32_t)qm[k] * (int32_t)wt[n * K + k];
            if (acc) acc[m * N + n] = s;
            y[m * N + n] = (double)s * dm * a;
        }
        if (xt) memcpy(xt + m * K, t, (size_t)K * sizeof(double));
        if (q) memcpy(q + m * K, qm, (size_t)K);
        if (d) d[m] = dm;
        free(u); free(t); free(qm);
    }
    return bad ? -2 : 0;
}

/* H-BitLinear forward (with the rotation). */
int oracle_forward(const float *x, const float *g, const int8_t *wt, float alpha,
                   int64_t M, int64_t K, int64_t N, int bits,
                   double *xt, int8_t *q, double *d, double *pre, int32_t *acc, double *y,
                   int nthreads)
{
    return oracle_forward_ex(x, g, wt, alpha, M, K, N, bits, 1, xt, q, d, pre, acc, y, nthreads);
}

/* ---------------------------------------------------------------------------
 * Weight + activation rotation [XZY §实验效果] (table 5 compares rotating the
 * activations only with rotating weights and activations).  Reading: each
 * weight row (one output channel over the K inputs) goes through the same
 * orthonormal transform as the activations, so that
 *   (H u / sqrt(K)) . (H w / sqrt(K)) = u . w
 * in exact arithmetic (H symmetric, H H = K I); the rotated rows are then
 * ternarised as usual:
 *   wr[n] = H_K w[n] / sqrt(K)   (double),
 *   S = sum |wr| (each row left to right, then the row sums in row order, double),
 *   alpha = (float)(S / (N K)),  a = max(alpha, EPS_Q),
 *   w_t = clamp(round(wr / a), -1, 1).
 * wr (optional) receives the rotated rows.
 * ------------------------------------------------------------------------- */
int oracle_quantize_weights_rotated(const float *w, int64_t N, int64_t K, int8_t *wt, float *alpha_out,
                                    double *wr_out)
{
    if (!w || !wt || !alpha_out || N <= 0 || !is_pow2(K)) return -1;
    double *wr = (double *)malloc((size_t)N * K * sizeof(double));
    double *row = (double *)malloc((size_t)K * sizeof(double));
    if (!wr || !row) { free(wr); free(row); return -2; }
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) row[k] = (double)w[n * K + k];
        oracle_hadamard_rotate(row, K, wr + n * K);
    }
    double S = 0.0;
    for (int64_t n = 0; n < N; ++n) S += row_abs_sum_d(wr + n * K, K);
    float alpha = (float)(S / ((double)N * (double)K));
    double a = oracle_weight_scale(alpha);
    for (int64_t i = 0; i < N * K; ++i) wt[i] = (int8_t)clampd(rne(wr[i] / a), -1.0, 1.0);
    *alpha_out = alpha;
    if (wr_out) memcpy(wr_out, wr, (size_t)N * K * sizeof(double));
    free(wr); free(row);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Low-bit attention states [XZY §实验效果] (the QKV states are quantised after
 * RoPE; every head is mapped straight to unsigned integers by an absmax
 * function, with no calibration data; tables 2 and 3 vary the bit width, and
 * a 3-bit KV cache matches the full-precision one).  Reading: per head (one
 * token, one head: a row of d values), with b bits,
 *   Qb = 2^(b-1) - 1,  Z = 2^(b-1),
 *   G  = max(max_e |v_e|, eps),     s = G / Qb,   eps = 1e-5 rounded to fp32
 *        (the per-head statistic and its stored scale are fp32 numbers),
 *   u_e = clamp(round(v_e * Qb / G) + Z, 0, 2^b - 1)   (round half to even),
 *   v^_e = (u_e - Z) * s.
 * RoPE itself is applied upstream (the input rows are post-RoPE).
 * x [R][d] fp32 (R = tokens * heads); codes [R][d] one code per byte;
 * scale [R] double; pre [R][d] optional (v * Qb / G before rounding).
 * ------------------------------------------------------------------------- */
int oracle_quant_heads(const float *x, int64_t R, int64_t d, int bits, uint8_t *codes, double *scale,
                       double *pre)
{
    if (!x || !codes || !scale || R < 0 || d <= 0 || bits < 2 || bits > 8) return -1;
    const double Qb = (double)((1 << (bits - 1)) - 1), Z = (double)(1 << (bits - 1));
    const double hi = (double)((1 << bits) - 1);
    for (int64_t r = 0; r < R; ++r) {
        const float *v = x + r * d;
        double G = 0.0;
        for (int64_t e = 0; e < d; ++e) if (fabs((double)v[e]) > G) G = fabs((double)v[e]);
        if (G < (double)(float)EPS_Q) G = (double)(float)EPS_Q;
        for (int64_t e = 0; e < d; ++e) {
            double p = (double)v[e] * Qb / G;
            if (pre) pre[r * d + e] = p;
            codes[r * d + e] = (uint8_t)clampd(rne(p) + Z, 0.0, hi);
        }
        scale[r] = G / Qb;
    }
    return 0;
}

/* v^ = (u - Z) * s for every code of every head. */
int oracle_dequant_heads(const uint8_t *codes, const double *scale, int64_t R, int64_t d, int bits, double *y)
{
    if (!codes || !scale || !y || R < 0 || d <= 0 || bits < 2 || bits > 8) return -1;
    const double Z = (double)(1 << (bits - 1));
    for (int64_t r = 0; r < R; ++r)
        for (int64_t e = 0; e < d; ++e) y[r * d + e] = ((double)codes[r * d + e] - Z) * scale[r];
    return 0;
}

/* ---------------------------------------------------------------------------
 * One decode step of attention over a quantised KV cache.  The method only
 * fixes the states' quantisation; attention itself is the standard scaled
 * dot product with softmax:
 *   q^   = dequant(quant(q, qbits))                     (per head, as above)
 *   k^_t = (uk_t - Z) * sk_t,   v^_t = (uv_t - Z) * sv_t  (Z = 2^(kvbits-1))
 *   l_t  = (q^ . k^_t) / sqrt(d),   p_t = exp(l_t - max l) / sum exp(...)
 *   out  = sum_t p_t v^_t,   t = 0 .. len_b - 1;  len_b = 0 gives out = 0.
 * Grouped heads: query head h reads KV head h / (Hq / Hkv).
 * q [B][Hq][d] fp32 (post-RoPE); kc, vc [B][Hkv][Tmax][d] one code per byte;
 * ks, vs [B][Hkv][Tmax] fp32 (the stored per-row scales); lens [B];
 * out [B][Hq][d] double.
 * ------------------------------------------------------------------------- */
int oracle_attention_decode(const float *q, int qbits, const uint8_t *kc, const float *ks, const uint8_t *vc,
                            const float *vs, int kvbits, const int32_t *lens, int64_t B, int64_t Hq,
                            int64_t Hkv, int64_t d, int64_t Tmax, double *out)
{
    if (!q || !kc || !ks || !vc || !vs || !lens || !out || B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 ||
        Tmax < 0 || Hq % Hkv || kvbits < 2 || kvbits > 8 || qbits < 2 || qbits > 8)
        return -1;
    for (int64_t b = 0; b < B; ++b)
        if (lens[b] < 0 || lens[b] > Tmax) return -2;
    const double Zkv = (double)(1 << (kvbits - 1));
    const int64_t group = Hq / Hkv;
    int rc = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : rc)
    for (int64_t bh = 0; bh < B * Hq; ++bh) {
        const int64_t b = bh / Hq, h = bh % Hq, hk = h / group;
        const int64_t len = lens[b];
        double *o = out + bh * d;
        uint8_t *uq = malloc((size_t)d);
        double *qh = malloc(sizeof(double) * (size_t)d);
        double *lg = malloc(sizeof(double) * (size_t)(len > 0 ? len : 1));
        double sq = 0.0;
        if (!uq || !qh || !lg || oracle_quant_heads(q + bh * d, 1, d, qbits, uq, &sq, NULL) != 0) {
            rc |= 1;
        } else {
            oracle_dequant_heads(uq, &sq, 1, d, qbits, qh);
            const uint8_t *K = kc + (b * Hkv + hk) * Tmax * d, *V = vc + (b * Hkv + hk) * Tmax * d;
            const float *KS = ks + (b * Hkv + hk) * Tmax, *VS = vs + (b * Hkv + hk) * Tmax;
            double mx = -INFINITY;
            for (int64_t t = 0; t < len; ++t) {
                double dot = 0.0;
                for (int64_t e = 0; e < d; ++e) dot += qh[e] * (((double)K[t * d + e] - Zkv) * (double)KS[t]);
                lg[t] = dot / sqrt((double)d);
                if (lg[t] > mx) mx = lg[t];
            }
            double den = 0.0;
            for (int64_t t = 0; t < len; ++t) { lg[t] = exp(lg[t] - mx); den += lg[t]; }
            for (int64_t e = 0; e < d; ++e) o[e] = 0.0;
            for (int64_t t = 0; t < len; ++t)
                for (int64_t e = 0; e < d; ++e) o[e] += lg[t] / den * (((double)V[t * d + e] - Zkv) * (double)VS[t]);
        }
        free(uq); free(qh); free(lg);
    }
    return rc ? -3 : 0;
}

/* ---------------------------------------------------------------------------
 * Backward pass of the layer with the straight-through estimator
 * [QbitAI §引入H-BitLinear模块] (training: the non-differentiable quantiser
 * functions are bypassed; the gradient is transformed with the orthogonal
 * Hadamard matrix).  The forward is y = xh . Wh^T with the quantised operands
 * xh = q * d (per token) and Wh = W_t * a; the estimator treats both
 * quantisers as the identity, so
 *   dxh[m][k] = a * sum_n dy[m][n] W_t[n][k]          (gradient at xt)
 *   du        = H_K dxh / sqrt(K)  (H symmetric and orthonormal after the
 *               scaling, so its transpose is itself); du = dxh unrotated
 *   RMSNorm, u = x g / r, r = sqrt(mean x^2 + EPS_NORM):
 *   dx[m][j]  = g_j du_j / r - x_j / (K r^3) * sum_i du_i g_i x_i
 *   dg[k]     = sum_m du[m][k] x[m][k] / r_m           (tokens in order)
 *   dW[n][k]  = sum_m dy[m][n] q[m][k] d[m]            (latent weights)
 * q, d are the forward's codes and scales; x, g its input and gain.
 * Outputs (double): dxh [M][K] (optional), dx [M][K], dw [N][K], dg [K]
 * (optional; needs g).
 * ------------------------------------------------------------------------- */
int oracle_backward(const float *x, const float *g, const int8_t *q, const double *d, const int8_t *wt,
                    float alpha, const float *dy, int64_t M, int64_t K, int64_t N, int rotate,
                    double *dxh, double *dx, double *dw, double *dg)
{
    if (!x || !q || !d || !wt || !dy || !dx || !dw || M < 0 || N <= 0 || !is_pow2(K) || (dg && !g)) return -1;
    const double a = oracle_weight_scale(alpha);
    double *du_all = dg ? (double *)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1) * (size_t)K) : NULL;
    double *rr = (double *)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
    if ((dg && !du_all) || !rr) { free(du_all); free(rr); return -2; }
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m) {
        double *t = (double *)malloc(sizeof(double) * (size_t)K);
        double *du = (double *)malloc(sizeof(double) * (size_t)K);
        if (!t || !du) { bad = 1; free(t); free(du); continue; }
        for (int64_t k = 0; k < K; ++k) t[k] = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double gy = (double)dy[m * N + n];
            if (gy == 0.0) continue;
            for (int64_t k = 0; k < K; ++k) t[k] += gy * (double)wt[n * K + k];
        }
        for (int64_t k = 0; k < K; ++k) t[k] *= a;
        if (dxh) memcpy(dxh + m * K, t, sizeof(double) * (size_t)K);
        if (rotate) oracle_hadamard_rotate(t, K, du);
        else memcpy(du, t, sizeof(double) * (size_t)K);
        const float *xm = x + m * K;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) ss += (double)xm[k] * (double)xm[k];
        const double r = sqrt(ss / (double)K + EPS_NORM);
        double sdot = 0.0;
        for (int64_t k = 0; k < K; ++k) sdot += du[k] * (g ? (double)g[k] : 1.0) * (double)xm[k];
        for (int64_t k = 0; k < K; ++k)
            dx[m * K + k] = (g ? (double)g[k] : 1.0) * du[k] / r - (double)xm[k] * sdot / ((double)K * r * r * r);
        rr[m] = r;
        if (du_all) memcpy(du_all + m * K, du, sizeof(double) * (size_t)K);
        free(t); free(du);
    }
    if (!bad && dg) {
        for (int64_t k = 0; k < K; ++k) dg[k] = 0.0;
        for (int64_t m = 0; m < M; ++m)
            for (int64_t k = 0; k < K; ++k) dg[k] += du_all[m * K + k] * (double)x[m * K + k] / rr[m];
    }
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) dw[n * K + k] = 0.0;
        for (int64_t m = 0; m < M; ++m) {
            const double gy = (double)dy[m * N + n] * d[m];
            if (gy == 0.0) continue;
            for (int64_t k = 0; k < K; ++k) dw[n * K + k] += gy * (double)q[m * K + k];
        }
    }
    free(du_all); free(rr);
    return bad ? -2 : 0;
}

/* ---------------------------------------------------------------------------
 * Prefill (causal) attention over the quantised cache: Tn new tokens per
 * sequence, token i of sequence b at position start_b + i, its query
 * quantised per head like the decode step's; it attends to the cached tokens
 * 0 .. start_b + i (the new tokens have been appended to the cache first).
 * q [B][Tn][Hq][d] fp32; cache and scales as for the decode step; start [B];
 * out [B][Tn][Hq][d] double.  Each query row is one decode step with length
 * start_b + i + 1.
 * ------------------------------------------------------------------------- */
int oracle_attention_prefill(const float *q, int qbits, const uint8_t *kc, const float *ks, const uint8_t *vc,
                             const float *vs, int kvbits, const int32_t *start, int64_t B, int64_t Tn,
                             int64_t Hq, int64_t Hkv, int64_t d, int64_t Tmax, double *out)
{
    if (!q || !start || !out || B < 0 || Tn < 0) return -1;
    for (int64_t b = 0; b < B; ++b)
        if (start[b] < 0 || start[b] + Tn > Tmax) return -2;
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < Tn; ++i) {
            /* one decode step of this sequence alone: the cache rows of
             * sequence b, length start + i + 1 */
            const int32_t len = (int32_t)(start[b] + i + 1);
            const int64_t hrow = b * Hkv * Tmax;
            int rc = oracle_attention_decode(q + ((b * Tn + i) * Hq) * d, qbits, kc + hrow * d, ks + hrow,
                                             vc + hrow * d, vs + hrow, kvbits, &len, 1, Hq, Hkv, d, Tmax,
                                             out + ((b * Tn + i) * Hq) * d);
            if (rc) return rc;
        }
    }
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
