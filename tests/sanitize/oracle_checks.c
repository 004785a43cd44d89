/*
 * Runs every function of the CPU oracle (oracle/tg_oracle.c, linked in) under
 * AddressSanitizer and UndefinedBehaviorSanitizer: small problems at the
 * edges of every argument (empty and one-element shapes, row subsets, K = 0,
 * padded pitches, both B layouts, bias and residual present or not, GELU,
 * special values, every 16-bit and 8-bit pattern through the codecs) plus
 * invalid arguments, which must be refused without touching memory.  Buffers
 * are allocated at their exact extents so that any access past them faults.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double tgo_f16_to_double(uint16_t h);
double tgo_bf16_to_double(uint16_t b);
uint16_t tgo_double_to_f16(double x);
uint16_t tgo_double_to_bf16(double x);
double tgo_fp8_to_double(int fmt, uint8_t x);
double tgo_e8m0_to_double(uint8_t e);
double tgo_gelu_tanh(double x);
int tgo_gemm_ex(int dt, int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                const uint16_t *B, int64_t ldb, int trans_b, const uint16_t *bias, int act,
                const uint16_t *R, int64_t ldr, double *out_f64, uint16_t *out_bits, int64_t ldc,
                int64_t row0, int64_t row1, int threads);
int tgo_gemm_ex_sample(int dt, int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                       const uint16_t *B, int64_t ldb, int trans_b, const uint16_t *bias, int act,
                       const uint16_t *R, int64_t ldr, int64_t n, const int64_t *ii,
                       const int64_t *jj, double *out_f64, uint16_t *out_bits, int threads);
int tgo_gemm_qkv(int dt, int64_t M, int64_t N, int64_t K, const uint16_t *X, int64_t ldx,
                 const uint16_t *Wq, const uint16_t *Wk, const uint16_t *Wv, int64_t ldw,
                 double *q_f64, double *k_f64, double *v_f64, uint16_t *q_bits, uint16_t *k_bits,
                 uint16_t *v_bits, int64_t ldo, int64_t row0, int64_t row1, int threads);
int tgo_gemm_mx(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K, const uint8_t *A,
                int64_t lda, const uint8_t *SA, int64_t ldsa, const uint8_t *B, int64_t ldb,
                const uint8_t *SB, int64_t ldsb, const uint16_t *bias, int act, int dt,
                double *out_f64, uint16_t *out_bits, int64_t ldc, int64_t row0, int64_t row1,
                int threads);
int tgo_attention(int dt, int64_t B, int64_t H, int64_t S, int64_t D, const uint16_t *Q,
                  const uint16_t *K, const uint16_t *V, double scale, int causal,
                  double *out_f64, uint16_t *out_bits, double *lse, int threads);
int tgo_decode_array(int dt, int64_t n, const uint16_t *in, double *out);
int tgo_encode_array(int dt, int64_t n, const double *in, uint16_t *out);
int tgo_gelu_array(int64_t n, const double *in, double *out);
int tgo_decode_fp8_array(int fmt, int64_t n, const uint8_t *in, double *out);

static int failures = 0;
#define EXPECT(c)                                                                                \
    do {                                                                                         \
        if (!(c)) {                                                                              \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);                      \
            ++failures;                                                                          \
        }                                                                                        \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)rng_state;
}

/* rows x ld buffer of 16-bit patterns (exact extent: (rows-1)*ld + cols) */
static uint16_t *mat16(int dt, int64_t rows, int64_t cols, int64_t ld, int specials)
{
    const int64_t n = rows > 0 ? (rows - 1) * ld + cols : 0;
    uint16_t *p = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) {
        const double v = (double)((int)(next_u32() % 5) - 2);
        p[i] = dt == 1 ? tgo_double_to_f16(v) : tgo_double_to_bf16(v);
    }
    if (specials && n > 3) {
        p[0] = dt == 1 ? 0x7E00 : 0x7FC0;
        p[n / 2] = dt == 1 ? 0x7C00 : 0x7F80;
        p[n - 1] = dt == 1 ? 0xFC00 : 0xFF80;
    }
    return p;
}

static void gemm_cases(void)
{
    const int64_t shapes[][3] = {{1, 1, 1}, {1, 7, 3}, {5, 1, 9}, {3, 4, 0}, {17, 13, 33},
                                 {8, 8, 8}, {0, 5, 5}, {5, 0, 5}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (int dt = 1; dt <= 2; ++dt)
            for (int tb = 0; tb <= 1; ++tb)
                for (int extra = 0; extra <= 1; ++extra) {
                    const int64_t M = shapes[s][0], N = shapes[s][1], K = shapes[s][2];
                    const int64_t lda = K + 3 * extra, ldb = (tb ? K : N) + 2 * extra;
                    const int64_t ldc = N + extra, ldr = N + 5 * extra;
                    uint16_t *A = mat16(dt, M, K, lda, extra);
                    uint16_t *B = tb ? mat16(dt, N, K, ldb, 0) : mat16(dt, K, N, ldb, 0);
                    uint16_t *bias = extra ? mat16(dt, 1, N, N, 0) : NULL;
                    uint16_t *R = extra ? mat16(dt, M, N, ldr, 0) : NULL;
                    const int64_t nc = M > 0 ? (M - 1) * ldc + N : 0;
                    double *f = (double *)malloc(sizeof(double) * (size_t)(nc > 0 ? nc : 1));
                    uint16_t *b = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(nc > 0 ? nc : 1));
                    for (int threads = 1; threads <= 3; threads += 2) {
                        EXPECT(tgo_gemm_ex(dt, M, N, K, A, lda, B, ldb, tb, bias, extra, R, ldr,
                                           f, b, ldc, 0, M, threads) == 0);
                        if (M > 1)
                            EXPECT(tgo_gemm_ex(dt, M, N, K, A, lda, B, ldb, tb, bias, extra, R,
                                               ldr, NULL, b, ldc, 1, M - 1, threads) == 0);
                    }
                    if (M > 0 && N > 0) {
                        int64_t ii[4] = {0, M - 1, M / 2, 0}, jj[4] = {0, N - 1, N / 2, N - 1};
                        double sf[4];
                        uint16_t sb[4];
                        EXPECT(tgo_gemm_ex_sample(dt, M, N, K, A, lda, B, ldb, tb, bias, 1, R,
                                                  ldr, 4, ii, jj, sf, sb, 2) == 0);
                        int64_t bad[1] = {M};
                        EXPECT(tgo_gemm_ex_sample(dt, M, N, K, A, lda, B, ldb, tb, bias, 1, R,
                                                  ldr, 1, bad, jj, sf, sb, 1) == -1);
                    }
                    /* refused arguments touch nothing */
                    EXPECT(tgo_gemm_ex(3, M, N, K, A, lda, B, ldb, tb, bias, 0, R, ldr, f, b, ldc,
                                       0, M, 1) == -1);
                    EXPECT(tgo_gemm_ex(dt, M, N, K, A, lda, B, ldb, 2, bias, 0, R, ldr, f, b, ldc,
                                       0, M, 1) == -1);
                    EXPECT(tgo_gemm_ex(dt, M, N, K, A, lda, B, ldb, tb, bias, 0, R, ldr, f, b, ldc,
                                       0, M + 1, 1) == -1);
                    EXPECT(tgo_gemm_ex(dt, -1, N, K, A, lda, B, ldb, tb, bias, 0, R, ldr, f, b,
                                       ldc, 0, 0, 1) == -1);
                    free(A), free(B), free(bias), free(R), free(f), free(b);
                }
    /* QKV: three GEMMs sharing X */
    {
        const int64_t M = 6, N = 5, K = 7;
        uint16_t *X = mat16(2, M, K, K, 0), *W[3];
        double *f[3];
        uint16_t *o[3];
        for (int t = 0; t < 3; ++t) {
            W[t] = mat16(2, K, N, N, t == 1);
            f[t] = (double *)malloc(sizeof(double) * M * N);
            o[t] = (uint16_t *)malloc(sizeof(uint16_t) * M * N);
        }
        EXPECT(tgo_gemm_qkv(2, M, N, K, X, K, W[0], W[1], W[2], N, f[0], f[1], f[2], o[0], o[1],
                            o[2], N, 0, M, 2) == 0);
        free(X);
        for (int t = 0; t < 3; ++t)
            free(W[t]), free(f[t]), free(o[t]);
    }
}

static void mx_cases(void)
{
    const int64_t shapes[][3] = {{1, 1, 32}, {3, 5, 64}, {9, 4, 96}, {2, 2, 0}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (int fa = 0; fa <= 1; ++fa)
            for (int fb = 0; fb <= 1; ++fb) {
                const int64_t M = shapes[s][0], N = shapes[s][1], K = shapes[s][2], KB = K / 32;
                const int64_t lda = K + 1, ldb = K + 2, ldsa = M + 1, ldsb = N;
                uint8_t *A = (uint8_t *)malloc((size_t)((M - 1) * lda + K + 1));
                uint8_t *B = (uint8_t *)malloc((size_t)((N - 1) * ldb + K + 1));
                uint8_t *SA = (uint8_t *)malloc((size_t)(KB > 0 ? (KB - 1) * ldsa + M : 1));
                uint8_t *SB = (uint8_t *)malloc((size_t)(KB > 0 ? (KB - 1) * ldsb + N : 1));
                for (int64_t i = 0; i < (M - 1) * lda + K; ++i)
                    A[i] = (uint8_t)next_u32();
                for (int64_t i = 0; i < (N - 1) * ldb + K; ++i)
                    B[i] = (uint8_t)next_u32();
                for (int64_t i = 0; KB > 0 && i < (KB - 1) * ldsa + M; ++i)
                    SA[i] = (uint8_t)(120 + next_u32() % 16);
                for (int64_t i = 0; KB > 0 && i < (KB - 1) * ldsb + N; ++i)
                    SB[i] = (uint8_t)(i == 0 ? 0xFF : 120 + next_u32() % 16);
                uint16_t *bias = mat16(2, 1, N, N, 0);
                double *f = (double *)malloc(sizeof(double) * (size_t)(M * N));
                uint16_t *b = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(M * N));
                EXPECT(tgo_gemm_mx(fa, fb, M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, bias, 1,
                                   2, f, b, N, 0, M, 3) == 0);
                EXPECT(tgo_gemm_mx(fa, fb, M, N, K + 1, A, lda, SA, ldsa, B, ldb, SB, ldsb, bias,
                                   1, 2, f, b, N, 0, M, 1) == -1);
                EXPECT(tgo_gemm_mx(fa, 7, M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, bias, 1, 2,
                                   f, b, N, 0, M, 1) == -1);
                free(A), free(B), free(SA), free(SB), free(bias), free(f), free(b);
            }
}

static void attention_cases(void)
{
    const int64_t shapes[][4] = {{1, 1, 1, 4}, {2, 3, 5, 8}, {1, 2, 17, 16}, {1, 1, 0, 8}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (int causal = 0; causal <= 1; ++causal) {
            const int64_t B = shapes[s][0], H = shapes[s][1], S = shapes[s][2], D = shapes[s][3];
            const int64_t n = B * H * S * D;
            uint16_t *Q = mat16(1, 1, n, n, 0), *K = mat16(1, 1, n, n, 0),
                     *V = mat16(1, 1, n, n, causal);
            double *f = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
            uint16_t *b = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1));
            double *lse = (double *)malloc(sizeof(double) * (size_t)(B * H * S > 0 ? B * H * S : 1));
            EXPECT(tgo_attention(1, B, H, S, D, Q, K, V, 0.125, causal, f, b, lse, 2) == 0);
            EXPECT(tgo_attention(1, B, H, S, 0, Q, K, V, 0.125, causal, f, b, lse, 1) == -1);
            free(Q), free(K), free(V), free(f), free(b), free(lse);
        }
}

static void codec_cases(void)
{
    uint16_t *all = (uint16_t *)malloc(sizeof(uint16_t) * 65536);
    double *d = (double *)malloc(sizeof(double) * 65536);
    uint16_t *back = (uint16_t *)malloc(sizeof(uint16_t) * 65536);
    for (int i = 0; i < 65536; ++i)
        all[i] = (uint16_t)i;
    for (int dt = 1; dt <= 2; ++dt) {
        EXPECT(tgo_decode_array(dt, 65536, all, d) == 0);
        EXPECT(tgo_encode_array(dt, 65536, d, back) == 0);
        for (int i = 0; i < 65536; ++i)
            if (!isnan(d[i]))
                EXPECT(back[i] == all[i]);
    }
    EXPECT(tgo_decode_array(9, 1, all, d) == -1);
    const double edge[] = {0.0, -0.0, 1e-320, -1e-320, 65504.0, 65519.99, 65520.0, 1e300,
                           -1e300, INFINITY, -INFINITY, NAN, 3.3895313892515355e38,
                           3.4e38, 5.9604644775390625e-08, 2.98e-08, 1e-45};
    const int ne = (int)(sizeof edge / sizeof edge[0]);
    uint16_t eb[32];
    double g[32];
    EXPECT(tgo_encode_array(1, ne, edge, eb) == 0);
    EXPECT(tgo_encode_array(2, ne, edge, eb) == 0);
    EXPECT(tgo_gelu_array(ne, edge, g) == 0);
    uint8_t b8[256];
    double d8[256];
    for (int i = 0; i < 256; ++i)
        b8[i] = (uint8_t)i;
    for (int fmt = 0; fmt <= 2; ++fmt)
        EXPECT(tgo_decode_fp8_array(fmt, 256, b8, d8) == 0);
    free(all), free(d), free(back);
}

int main(void)
{
    gemm_cases();
    mx_cases();
    attention_cases();
    codec_cases();
    if (failures)
        fprintf(stderr, "%d check(s) failed\n", failures);
    else
        printf("oracle checks passed\n");
    return failures ? 1 : 0;
}
