/* The oracle (oracle/oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every exported function runs on small seeded
 * inputs, at the edge sizes the tests use (K = 64 .. 1024, one token, ragged
 * head counts), with a few properties checked along the way (the transform
 * applied twice is n times the identity, codes inside their ranges, the
 * layer's output equals its own stages).  The sanitizers flag any
 * out-of-bounds access or undefined behaviour.  Prints "ok" and exits 0 when
 * every check holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_quantize_weights(const float *w, int64_t N, int64_t K, int8_t *wt, float *alpha_out);
double oracle_weight_scale(float alpha);
int oracle_rmsnorm(const float *x, const float *g, int64_t K, double *u);
int oracle_fwht(double *v, int64_t n);
int oracle_hadamard_rotate(const double *u, int64_t K, double *xt);
int oracle_quant_act(const double *xt, int64_t K, int bits, int8_t *q, double *d, double *pre);
int oracle_gemm_ternary(const int8_t *q, const int8_t *wt, int64_t M, int64_t N, int64_t K, int32_t *acc,
                        int nthreads);
int oracle_dequant(const int32_t *acc, const double *d, float alpha, int64_t M, int64_t N, double *y);
int oracle_forward_ex(const float *x, const float *g, const int8_t *wt, float alpha, int64_t M, int64_t K, int64_t N,
                      int bits, int rotate, double *xt, int8_t *q, double *d, double *pre, int32_t *acc, double *y,
                      int nthreads);
int oracle_forward(const float *x, const float *g, const int8_t *wt, float alpha, int64_t M, int64_t K, int64_t N,
                   int bits, double *xt, int8_t *q, double *d, double *pre, int32_t *acc, double *y, int nthreads);
int oracle_quantize_weights_rotated(const float *w, int64_t N, int64_t K, int8_t *wt, float *alpha_out,
                                    double *wr_out);
int oracle_quant_heads(const float *x, int64_t R, int64_t d, int bits, uint8_t *codes, double *scale, double *pre);
int oracle_dequant_heads(const uint8_t *codes, const double *scale, int64_t R, int64_t d, int bits, double *y);
int oracle_attention_decode(const float *q, int qbits, const uint8_t *kc, const float *ks, const uint8_t *vc,
                            const float *vs, int kvbits, const int32_t *lens, int64_t B, int64_t Hq, int64_t Hkv,
                            int64_t d, int64_t Tmax, double *out);
int oracle_backward(const float *x, const float *g, const int8_t *q, const double *d, const int8_t *wt, float alpha,
                    const float *dy, int64_t M, int64_t K, int64_t N, int rotate, double *dxh, double *dx,
                    double *dw, double *dg);
int oracle_attention_prefill(const float *q, int qbits, const uint8_t *kc, const float *ks, const uint8_t *vc,
                             const float *vs, int kvbits, const int32_t *start, int64_t B, int64_t Tn, int64_t Hq,
                             int64_t Hkv, int64_t d, int64_t Tmax, double *out);

static int fails = 0;
#define CHECK(c)                                                   \
    do {                                                           \
        if (!(c)) {                                                \
            printf("FAIL line %d: %s\n", __LINE__, #c);            \
            ++fails;                                               \
        }                                                          \
    } while (0)

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double urand(void) /* uniform in [-1, 1) */
{
    state ^= state << 13; state ^= state >> 7; state ^= state << 17;
    return (double)(state >> 11) / 4503599627370496.0 - 1.0;
}
static void fill(float *v, int64_t n, double scale)
{
    for (int64_t i = 0; i < n; ++i) v[i] = (float)(scale * urand());
}

static void layer(int64_t M, int64_t K, int64_t N)
{
    float *x = malloc(sizeof(float) * M * K), *g = malloc(sizeof(float) * K), *w = malloc(sizeof(float) * N * K);
    int8_t *wt = malloc(N * K), *q = malloc(M * K), *q2 = malloc(M * K);
    double *xt = malloc(sizeof(double) * M * K), *d = malloc(sizeof(double) * M), *pre = malloc(sizeof(double) * M * K);
    double *y = malloc(sizeof(double) * M * N), *y2 = malloc(sizeof(double) * M * N), *d2 = malloc(sizeof(double) * M);
    int32_t *acc = malloc(sizeof(int32_t) * M * N);
    double *u = malloc(sizeof(double) * K), *t = malloc(sizeof(double) * K), *wr = malloc(sizeof(double) * N * K);
    float alpha = 0.f;
    fill(x, M * K, 3.0); fill(g, K, 1.0); fill(w, N * K, 0.05);
    CHECK(oracle_quantize_weights(w, N, K, wt, &alpha) == 0 && alpha > 0.f);
    for (int64_t i = 0; i < N * K; ++i) CHECK(wt[i] >= -1 && wt[i] <= 1);
    CHECK(oracle_weight_scale(0.f) > 0.0);
    for (int bits = 4; bits <= 8; bits += 4) {
        for (int rotate = 0; rotate <= 1; ++rotate) {
            CHECK(oracle_forward_ex(x, g, wt, alpha, M, K, N, bits, rotate, xt, q, d, pre, acc, y, 2) == 0);
            for (int64_t i = 0; i < M * K; ++i) CHECK(bits == 8 ? (q[i] >= -128) : (q[i] >= -8 && q[i] <= 7));
            /* the same result from the stages */
            for (int64_t m = 0; m < M; ++m) {
                CHECK(oracle_rmsnorm(x + m * K, g, K, u) == 0);
                if (rotate) CHECK(oracle_hadamard_rotate(u, K, t) == 0); else memcpy(t, u, sizeof(double) * K);
                CHECK(oracle_quant_act(t, K, bits, q2 + m * K, d2 + m, NULL) == 0);
            }
            CHECK(memcmp(q, q2, M * K) == 0);
            CHECK(oracle_gemm_ternary(q2, wt, M, N, K, acc, 1) == 0);
            CHECK(oracle_dequant(acc, d2, alpha, M, N, y2) == 0);
            for (int64_t i = 0; i < M * N; ++i) CHECK(y[i] == y2[i]);
        }
        CHECK(oracle_forward(x, NULL, wt, alpha, M, K, N, bits, xt, q, d, pre, acc, y, 1) == 0);
    }
    /* transform twice = K times the identity */
    for (int64_t k = 0; k < K; ++k) t[k] = urand();
    memcpy(u, t, sizeof(double) * K);
    CHECK(oracle_fwht(t, K) == 0 && oracle_fwht(t, K) == 0);
    for (int64_t k = 0; k < K; ++k) CHECK(fabs(t[k] - (double)K * u[k]) <= 1e-9 * K);
    CHECK(oracle_fwht(t, K - 1) != 0);
    CHECK(oracle_quantize_weights_rotated(w, N, K, wt, &alpha, wr) == 0);
    /* backward with and without gain / rotation */
    {
        float *dy = malloc(sizeof(float) * M * N);
        double *dxh = malloc(sizeof(double) * M * K), *dx = malloc(sizeof(double) * M * K);
        double *dw = malloc(sizeof(double) * N * K), *dg = malloc(sizeof(double) * K);
        fill(dy, M * N, 1.0);
        CHECK(oracle_backward(x, g, q, d, wt, alpha, dy, M, K, N, 1, dxh, dx, dw, dg) == 0);
        CHECK(oracle_backward(x, NULL, q, d, wt, alpha, dy, M, K, N, 0, NULL, dx, dw, NULL) == 0);
        CHECK(oracle_backward(x, NULL, q, d, wt, alpha, dy, M, K, N, 0, NULL, dx, dw, dg) != 0); /* dg needs g */
        free(dy); free(dxh); free(dx); free(dw); free(dg);
    }
    free(x); free(g); free(w); free(wt); free(q); free(q2); free(xt); free(d); free(pre); free(y); free(y2);
    free(d2); free(acc); free(u); free(t); free(wr);
}

static void attention(int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t Tmax, int kvbits)
{
    const int64_t rows = B * Hkv * Tmax;
    float *kv = malloc(sizeof(float) * rows * d), *q = malloc(sizeof(float) * B * Hq * d);
    uint8_t *kc = malloc(rows * d), *vc = malloc(rows * d);
    double *ks = malloc(sizeof(double) * rows), *vs = malloc(sizeof(double) * rows);
    float *ksf = malloc(sizeof(float) * rows), *vsf = malloc(sizeof(float) * rows);
    double *yk = malloc(sizeof(double) * rows * d), *out = malloc(sizeof(double) * B * Hq * d);
    int32_t *lens = malloc(sizeof(int32_t) * B), *start = malloc(sizeof(int32_t) * B);
    fill(kv, rows * d, 2.0);
    CHECK(oracle_quant_heads(kv, rows, d, kvbits, kc, ks, NULL) == 0);
    CHECK(oracle_dequant_heads(kc, ks, rows, d, kvbits, yk) == 0);
    for (int64_t i = 0; i < rows * d; ++i) CHECK(kc[i] < (1u << kvbits));
    fill(kv, rows * d, 2.0);
    CHECK(oracle_quant_heads(kv, rows, d, kvbits, vc, vs, NULL) == 0);
    for (int64_t r = 0; r < rows; ++r) { ksf[r] = (float)ks[r]; vsf[r] = (float)vs[r]; }
    fill(q, B * Hq * d, 1.0);
    for (int64_t b = 0; b < B; ++b) { lens[b] = (int32_t)((b * 7) % (Tmax + 1)); start[b] = (int32_t)(b % 2); }
    CHECK(oracle_attention_decode(q, 8, kc, ksf, vc, vsf, kvbits, lens, B, Hq, Hkv, d, Tmax, out) == 0);
    CHECK(oracle_attention_prefill(q, 8, kc, ksf, vc, vsf, kvbits, start, B, 1, Hq, Hkv, d, Tmax, out) == 0);
    lens[0] = (int32_t)Tmax + 1;
    CHECK(oracle_attention_decode(q, 8, kc, ksf, vc, vsf, kvbits, lens, B, Hq, Hkv, d, Tmax, out) != 0);
    free(kv); free(q); free(kc); free(vc); free(ks); free(vs); free(ksf); free(vsf); free(yk); free(out);
    free(lens); free(start);
}

int main(void)
{
    layer(1, 64, 16);
    layer(5, 128, 48);
    layer(3, 1024, 32);
    attention(2, 4, 2, 64, 9, 3);
    attention(3, 2, 1, 128, 5, 8);
    if (fails) {
        printf("%d failures\n", fails);
        return 1;
    }
    printf("ok\n");
    return 0;
}
