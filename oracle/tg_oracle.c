/*
 * tg_oracle.c -- CPU oracle for the tiled dense GEMM  C = epilogue(A . B).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * reference that the GPU path is checked against.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or constant with the HIP library.
 *
 * What it computes (the plain definition, in double precision):
 *
 *   C[i][j] = round_dt( act( sum_{k=0}^{K-1} A[i][k] * B[k][j]  + bias[j] ) )
 *
 * - The matrix product is the operation every tile of the method adds up:
 *   per tile, an A tile and a B tile are loaded and multiplied into an
 *   output tile, marching over K ("TileIR", the matmul inner loop; the
 *   TileLang article, section 4, the FP16 GEMM kernel).  Tiling only changes
 *   the order of the sum, so the oracle is the untiled sum.
 * - The sum over k runs in ascending k, in double.  Products of two f16
 *   (11-bit significand) or bf16 (8-bit) values are exact in double.
 * - bias[j] is added per output column, then the activation is applied
 *   ("TileIR", epilogue fusion: an elementwise op applied to the MMA result).
 *   act is identity or the tanh form of GELU:
 *       gelu(x) = 0.5 x (1 + tanh( sqrt(2/pi) (x + 0.044715 x^3) )).
 * - round_dt is IEEE round-to-nearest, ties-to-even, taken once, directly
 *   from double to f16 or bf16 (the TileLang example copies its f32
 *   fragment to an f16 output; the rounding mode is not stated there and
 *   the IEEE default is taken).
 * - The horizontally fused QKV projection ("TileIR", horizontal fusion:
 *   Q, K and V projections share their input) is three independent GEMMs.
 * - The extended form (tgo_gemm_ex) adds two things:
 *     C[i][j] = round_dt( act( sum_k A[i][k] * opB[k][j] + bias[j] ) + R[i][j] )
 *   R is a residual added after the activation, before the one rounding
 *   ("TileIR", vertical fusion: the next elementwise operation, such as a
 *   residual add, chained onto the product instead of run as a second
 *   pass).  opB[k][j] is B[k][j] (B stored [K,N]) or B[j][k] (B stored
 *   [N,K], one output feature per row): the same logical operand with its
 *   two axes permuted, the placement unchanged ("TIRx", section 5.1,
 *   permute).
 * - The block-scaled low-precision form (tgo_gemm_mx) computes
 *     C[i][j] = round_dt( act( sum_k  a(A[i][k]) 2^(SA[k/32][i] - 127)
 *                                   * b(B[j][k]) 2^(SB[k/32][j] - 127) + bias[j] ) )
 *   with A [M,K] and B [N,K] in an 8-bit float format (e4m3 or e5m2) and
 *   one 8-bit power-of-two scale (e8m0) per 32 consecutive k of each row of
 *   A and each column of B ("TIRx", section 6: the FP8 GEMM with e8m0
 *   block-wise scaling).  The pages fix neither the block length nor the
 *   axes; 32 along K is the block of the OCP microscaling formats and of
 *   the gfx950 matrix cores.  Products of two 8-bit floats and two powers
 *   of two are exact in double.
 * - Attention (tgo_attention) is the plain definition
 *     O[i] = sum_j softmax_j( scale * Q[i] . K[j] + mask[i][j] ) V[j],
 *   scale = 1/sqrt(D) by default, mask[i][j] = -inf for j > i when causal
 *   ("TileIR", Softmax(Q K^T / sqrt(d)) V, which the fused kernel evaluates
 *   with an online softmax; "TIRx", section 6: forward multi-head attention
 *   with head dimension 128, causal and non-causal).  It materialises every
 *   score row, in double: m = max_j s_j, p_j = exp(s_j - m), l = sum_j p_j,
 *   O[i] = (sum_j p_j V[j]) / l, and the log-sum-exp m + log(l).
 *
 * Every output element depends only on its own row of A and column of B,
 * so rows are split across OpenMP threads; the value of each element does
 * not depend on the thread count.
 *
 * Codecs: f16/bf16 <-> double are written here from the IEEE 754 binary16
 * and the bfloat16 (truncated binary32) bit layouts; the 8-bit formats from
 * the OCP 8-bit floating point layouts (e4m3: bias 7, no infinities, NaN
 * at exponent and mantissa all ones; e5m2: bias 15, IEEE-style infinities
 * and NaNs) and e8m0 (an exponent only, bias 127, 0xFF = NaN).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { TGO_F16 = 1, TGO_BF16 = 2 };
enum { TGO_ACT_NONE = 0, TGO_ACT_GELU_TANH = 1 };

/* ---------------------------------------------------------------- codecs */

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double tgo_f16_to_double(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25); /* 1.f * 2^(e-15) */
    return s ? -v : v;
}

/* bfloat16: the top 16 bits of a binary32. */
double tgo_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, 4);
    return (double)x;
}

/*
 * Round a double to a binary format with `p` significand bits (including the
 * implicit one), minimum normal exponent emin, maximum finite exponent emax,
 * ties to even.  Returns the sign-less bit pattern with `fbits` fraction
 * bits and `ebits` exponent bits; overflow gives infinity.
 */
static uint16_t tgo_round_bits(double x, int p, int emin, int emax, int ebits)
{
    int fbits = p - 1;
    uint16_t sign = 0;
    if (signbit(x)) {
        sign = (uint16_t)(1u << (fbits + ebits));
        x = -x;
    }
    uint16_t inf = (uint16_t)(((1u << ebits) - 1) << fbits);
    if (isnan(x))
        return (uint16_t)(inf | (1u << (fbits - 1))); /* canonical quiet NaN, sign dropped */
    if (isinf(x))
        return sign | inf;
    if (x == 0.0)
        return sign;

    int e;
    frexp(x, &e); /* x = m * 2^e, m in [0.5, 1) -> unbiased exponent e-1 */
    int exp = e - 1;
    if (exp < emin)
        exp = emin; /* subnormal range: fixed quantum 2^(emin-fbits) */
    /* quantum (ulp) at this exponent */
    double scaled = ldexp(x, fbits - exp); /* x / ulp; exact (power-of-two scale) */
    double fl = floor(scaled);
    double rem = scaled - fl; /* exact: scaled has at most 53 bits */
    uint64_t q = (uint64_t)fl;
    if (rem > 0.5 || (rem == 0.5 && (q & 1)))
        q += 1;
    /* q is now the significand in units of 2^(exp-fbits); it may have
     * carried into the next binade (q == 2^p). */
    if (q >= (1ull << p)) {
        q >>= 1;
        exp += 1;
    }
    if (exp > emax)
        return sign | inf;
    if (q < (1ull << fbits)) /* subnormal (exp == emin) */
        return sign | (uint16_t)q;
    uint16_t bexp = (uint16_t)(exp - emin + 1);
    return sign | (uint16_t)(bexp << fbits) | (uint16_t)(q & ((1u << fbits) - 1));
}

uint16_t tgo_double_to_f16(double x) { return tgo_round_bits(x, 11, -14, 15, 5); }
uint16_t tgo_double_to_bf16(double x) { return tgo_round_bits(x, 8, -126, 127, 8); }

/* 8-bit floats (OCP).  e4m3: 1 sign, 4 exponent (bias 7), 3 fraction bits;
 * exponent 15 with fraction 7 is NaN, there are no infinities.  e5m2: 1
 * sign, 5 exponent (bias 15), 2 fraction bits, IEEE-style specials. */
enum { TGO_FP8_E4M3 = 0, TGO_FP8_E5M2 = 1 };

double tgo_fp8_to_double(int fmt, uint8_t x)
{
    const int s = (x >> 7) & 1;
    double v;
    if (fmt == TGO_FP8_E4M3) {
        const int e = (x >> 3) & 15, f = x & 7;
        if (e == 15 && f == 7)
            return NAN;
        v = e == 0 ? ldexp((double)f, -9) : ldexp(8.0 + f, e - 10); /* (1 + f/8) 2^(e-7) */
    } else {
        const int e = (x >> 2) & 31, f = x & 3;
        if (e == 31)
            return f ? NAN : (s ? -INFINITY : INFINITY);
        v = e == 0 ? ldexp((double)f, -16) : ldexp(4.0 + f, e - 17); /* (1 + f/4) 2^(e-15) */
    }
    return s ? -v : v;
}

/* e8m0 scale: 2^(e - 127); 0xFF is NaN. */
double tgo_e8m0_to_double(uint8_t e) { return e == 0xFF ? NAN : ldexp(1.0, (int)e - 127); }

static double decode(int dt, uint16_t v)
{
    return dt == TGO_F16 ? tgo_f16_to_double(v) : tgo_bf16_to_double(v);
}

static uint16_t encode(int dt, double x)
{
    return dt == TGO_F16 ? tgo_double_to_f16(x) : tgo_double_to_bf16(x);
}

/* ------------------------------------------------------------ activation */

/* The tanh-form GELU.  With u = sqrt(2/pi) (x + 0.044715 x^3), the identity
 * 1 + tanh(u) = 2 / (1 + exp(-2u)) turns 0.5 x (1 + tanh(u)) into
 * x / (1 + exp(-2u)), the same function.  That form is the one evaluated:
 * in double, 1 + tanh(u) cancels to exactly 0 once u < -19 (x < -6.4),
 * while the function's value there (-2.5e-15 at x = -7) is still far
 * above the smallest bf16 magnitudes. */
double tgo_gelu_tanh(double x)
{
    const double c = sqrt(2.0 / M_PI);
    const double u = c * (x + 0.044715 * x * x * x);
    return x / (1.0 + exp(-2.0 * u));
}

static double activate(int act, double v)
{
    return act == TGO_ACT_GELU_TANH ? tgo_gelu_tanh(v) : v;
}

/* ------------------------------------------------------------------ GEMM */

/* opB[k][j] as stored: B[k][j] in a [K,N] matrix, B[j][k] in an [N,K] one. */
static uint16_t op_b(const uint16_t *B, int64_t ldb, int trans_b, int64_t k, int64_t j)
{
    return trans_b ? B[j * ldb + k] : B[k * ldb + j];
}

/* One output element: the definition, k ascending. */
static double element(int dt, int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B,
                      int64_t ldb, int trans_b, const uint16_t *bias, int act,
                      const uint16_t *R, int64_t ldr, int64_t i, int64_t j)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k)
        s += decode(dt, A[i * lda + k]) * decode(dt, op_b(B, ldb, trans_b, k, j));
    if (bias)
        s += decode(dt, bias[j]);
    double v = activate(act, s);
    if (R)
        v += decode(dt, R[i * ldr + j]);
    return v;
}

/*
 * Full GEMM over output rows [row0, row1).  A is [M,K] row-major with row
 * pitch lda; B is [K,N] with pitch ldb (trans_b = 0) or [N,K] with pitch ldb
 * (trans_b = 1); bias is [N] or NULL; R is [M,N] with pitch ldr, or NULL.
 * Outputs (either may be NULL): out_f64[i*ldc + j] the unrounded double
 * result, out_bits the round-to-nearest-even bits in the same dtype.
 * threads <= 0 means the OpenMP default.  Returns 0, or -1 on a bad
 * argument.
 *
 * For speed only, opB is first decoded into a column-major double copy; each
 * element is still the k-ascending sum of exact products.
 */
int tgo_gemm_ex(int dt, int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                const uint16_t *B, int64_t ldb, int trans_b, const uint16_t *bias, int act,
                const uint16_t *R, int64_t ldr, double *out_f64, uint16_t *out_bits, int64_t ldc,
                int64_t row0, int64_t row1, int threads)
{
    if ((dt != TGO_F16 && dt != TGO_BF16) || (act != TGO_ACT_NONE && act != TGO_ACT_GELU_TANH))
        return -1;
    if (M < 0 || N < 0 || K < 0 || row0 < 0 || row1 > M || row0 > row1 || ldc < N)
        return -1;
    if (trans_b != 0 && trans_b != 1)
        return -1;
    if (row0 == row1 || N == 0)
        return 0;
    double *bt = (double *)malloc(sizeof(double) * (size_t)(N * (K > 0 ? K : 1)));
    double *bs = (double *)malloc(sizeof(double) * (size_t)N);
    if (!bt || !bs) {
        free(bt);
        free(bs);
        return -1;
    }
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j)
            bt[j * K + k] = decode(dt, op_b(B, ldb, trans_b, k, j));
    for (int64_t j = 0; j < N; ++j)
        bs[j] = bias ? decode(dt, bias[j]) : 0.0;

#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#pragma omp parallel
#endif
    {
        double *arow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t i = row0; i < row1; ++i) {
            for (int64_t k = 0; k < K; ++k)
                arow[k] = decode(dt, A[i * lda + k]);
            for (int64_t j = 0; j < N; ++j) {
                const double *bcol = bt + j * K;
                double s = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    s += arow[k] * bcol[k];
                if (bias)
                    s += bs[j];
                double v = activate(act, s);
                if (R)
                    v += decode(dt, R[i * ldr + j]);
                if (out_f64)
                    out_f64[i * ldc + j] = v;
                if (out_bits)
                    out_bits[i * ldc + j] = encode(dt, v);
            }
        }
        free(arow);
    }
    free(bt);
    free(bs);
    return 0;
}

/* The plain form: B [K,N], no residual. */
int tgo_gemm(int dt, int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
             const uint16_t *B, int64_t ldb, const uint16_t *bias, int act, double *out_f64,
             uint16_t *out_bits, int64_t ldc, int64_t row0, int64_t row1, int threads)
{
    return tgo_gemm_ex(dt, M, N, K, A, lda, B, ldb, 0, bias, act, NULL, 0, out_f64, out_bits, ldc,
                       row0, row1, threads);
}

/*
 * Sampled outputs: the n elements (ii[s], jj[s]) of the same GEMM, for
 * checking large problems one element at a time (operands as in
 * tgo_gemm_ex).
 */
int tgo_gemm_ex_sample(int dt, int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                       const uint16_t *B, int64_t ldb, int trans_b, const uint16_t *bias, int act,
                       const uint16_t *R, int64_t ldr, int64_t n, const int64_t *ii,
                       const int64_t *jj, double *out_f64, uint16_t *out_bits, int threads)
{
    if ((dt != TGO_F16 && dt != TGO_BF16) || (act != TGO_ACT_NONE && act != TGO_ACT_GELU_TANH))
        return -1;
    if (trans_b != 0 && trans_b != 1)
        return -1;
    for (int64_t s = 0; s < n; ++s)
        if (ii[s] < 0 || ii[s] >= M || jj[s] < 0 || jj[s] >= N)
            return -1;
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#pragma omp parallel for schedule(dynamic, 16)
#endif
    for (int64_t s = 0; s < n; ++s) {
        double v = element(dt, K, A, lda, B, ldb, trans_b, bias, act, R, ldr, ii[s], jj[s]);
        if (out_f64)
            out_f64[s] = v;
        if (out_bits)
            out_bits[s] = encode(dt, v);
    }
    return 0;
}

int tgo_gemm_sample(int dt, int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                    const uint16_t *B, int64_t ldb, const uint16_t *bias, int act, int64_t n,
                    const int64_t *ii, const int64_t *jj, double *out_f64, uint16_t *out_bits,
                    int threads)
{
    return tgo_gemm_ex_sample(dt, M, N, K, A, lda, B, ldb, 0, bias, act, NULL, 0, n, ii, jj,
                              out_f64, out_bits, threads);
}

/*
 * QKV: out_t = X . W_t for t = 0,1,2 -- three independent GEMMs sharing X.
 * W[t] is [K,N] with pitch ldw; the outputs share pitch ldo.
 */
int tgo_gemm_qkv(int dt, int64_t M, int64_t N, int64_t K, const uint16_t *X, int64_t ldx,
                 const uint16_t *Wq, const uint16_t *Wk, const uint16_t *Wv, int64_t ldw,
                 double *q_f64, double *k_f64, double *v_f64, uint16_t *q_bits, uint16_t *k_bits,
                 uint16_t *v_bits, int64_t ldo, int64_t row0, int64_t row1, int threads)
{
    const uint16_t *W[3] = {Wq, Wk, Wv};
    double *of[3] = {q_f64, k_f64, v_f64};
    uint16_t *ob[3] = {q_bits, k_bits, v_bits};
    for (int t = 0; t < 3; ++t) {
        int rc = tgo_gemm(dt, M, N, K, X, ldx, W[t], ldw, NULL, TGO_ACT_NONE, of[t], ob[t], ldo,
                          row0, row1, threads);
        if (rc)
            return rc;
    }
    return 0;
}

/*
 * Block-scaled 8-bit GEMM over output rows [row0, row1).  A is [M,K] bytes
 * (pitch lda), B is [N,K] bytes (pitch ldb), SA is [K/32][M] scale bytes
 * (pitch ldsa: the M scales of one k-block are contiguous), SB is [K/32][N]
 * (pitch ldsb).  bias is [N] in the output dtype dt, or NULL.  Outputs as in
 * tgo_gemm_ex.  K must be a multiple of 32.  Returns 0, or -1 on a bad
 * argument.
 */
int tgo_gemm_mx(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K, const uint8_t *A,
                int64_t lda, const uint8_t *SA, int64_t ldsa, const uint8_t *B, int64_t ldb,
                const uint8_t *SB, int64_t ldsb, const uint16_t *bias, int act, int dt,
                double *out_f64, uint16_t *out_bits, int64_t ldc, int64_t row0, int64_t row1,
                int threads)
{
    if ((dt != TGO_F16 && dt != TGO_BF16) || (act != TGO_ACT_NONE && act != TGO_ACT_GELU_TANH))
        return -1;
    if ((fmt_a != TGO_FP8_E4M3 && fmt_a != TGO_FP8_E5M2) ||
        (fmt_b != TGO_FP8_E4M3 && fmt_b != TGO_FP8_E5M2))
        return -1;
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || row0 < 0 || row1 > M || row0 > row1 ||
        ldc < N)
        return -1;
    if (row0 == row1 || N == 0)
        return 0;
    /* opB with its scales applied, column-major double copy (speed only) */
    double *bt = (double *)malloc(sizeof(double) * (size_t)(N * (K > 0 ? K : 1)));
    if (!bt)
        return -1;
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k)
            bt[j * K + k] = tgo_fp8_to_double(fmt_b, B[j * ldb + k]) *
                            tgo_e8m0_to_double(SB[(k / 32) * ldsb + j]);
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#pragma omp parallel
#endif
    {
        double *arow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t i = row0; i < row1; ++i) {
            for (int64_t k = 0; k < K; ++k)
                arow[k] = tgo_fp8_to_double(fmt_a, A[i * lda + k]) *
                          tgo_e8m0_to_double(SA[(k / 32) * ldsa + i]);
            for (int64_t j = 0; j < N; ++j) {
                const double *bcol = bt + j * K;
                double sum = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    sum += arow[k] * bcol[k];
                if (bias)
                    sum += decode(dt, bias[j]);
                const double v = activate(act, sum);
                if (out_f64)
                    out_f64[i * ldc + j] = v;
                if (out_bits)
                    out_bits[i * ldc + j] = encode(dt, v);
            }
        }
        free(arow);
    }
    free(bt);
    return 0;
}

/* Decode n 8-bit floats (fmt) or, with fmt = 2, e8m0 scales. */
int tgo_decode_fp8_array(int fmt, int64_t n, const uint8_t *in, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = fmt == 2 ? tgo_e8m0_to_double(in[i]) : tgo_fp8_to_double(fmt, in[i]);
    return 0;
}

/*
 * Attention over Q, K, V of shape [B][H][S][D] (contiguous, dtype dt).  For
 * every (b, h, i): scores s_j = scale * sum_d Q[i][d] K[j][d] for j < S (j <= i
 * when causal), then the softmax-weighted sum of the V rows.  out_f64 /
 * out_bits receive O (same layout; either may be NULL), lse (may be NULL)
 * the [B][H][S] log-sum-exp of the scaled scores.  Returns 0 or -1.
 */
int tgo_attention(int dt, int64_t B, int64_t H, int64_t S, int64_t D, const uint16_t *Q,
                  const uint16_t *K, const uint16_t *V, double scale, int causal,
                  double *out_f64, uint16_t *out_bits, double *lse, int threads)
{
    if ((dt != TGO_F16 && dt != TGO_BF16) || B < 0 || H < 0 || S < 0 || D <= 0)
        return -1;
    const int64_t heads = B * H;
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#pragma omp parallel
#endif
    {
        double *sc = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
        double *q = (double *)malloc(sizeof(double) * (size_t)D);
        double *o = (double *)malloc(sizeof(double) * (size_t)D);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
        for (int64_t row = 0; row < heads * S; ++row) {
            const int64_t hd = row / S, i = row % S;
            const uint16_t *Qh = Q + hd * S * D, *Kh = K + hd * S * D, *Vh = V + hd * S * D;
            const int64_t nkeys = causal ? i + 1 : S;
            for (int64_t d = 0; d < D; ++d)
                q[d] = decode(dt, Qh[i * D + d]);
            double m = -INFINITY;
            for (int64_t j = 0; j < nkeys; ++j) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += q[d] * decode(dt, Kh[j * D + d]);
                sc[j] = scale * dot;
                if (sc[j] > m)
                    m = sc[j];
            }
            double l = 0.0;
            for (int64_t d = 0; d < D; ++d)
                o[d] = 0.0;
            for (int64_t j = 0; j < nkeys; ++j) {
                const double pj = exp(sc[j] - m);
                l += pj;
                for (int64_t d = 0; d < D; ++d)
                    o[d] += pj * decode(dt, Vh[j * D + d]);
            }
            for (int64_t d = 0; d < D; ++d) {
                const double v = o[d] / l;
                if (out_f64)
                    out_f64[row * D + d] = v;
                if (out_bits)
                    out_bits[row * D + d] = encode(dt, v);
            }
            if (lse)
                lse[row] = m + log(l);
        }
        free(sc);
        free(q);
        free(o);
    }
    return 0;
}

int tgo_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Array forms of the codecs (used by the tests to sweep all bit patterns). */
int tgo_decode_array(int dt, int64_t n, const uint16_t *in, double *out)
{
    if (dt != TGO_F16 && dt != TGO_BF16)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        out[i] = decode(dt, in[i]);
    return 0;
}

int tgo_encode_array(int dt, int64_t n, const double *in, uint16_t *out)
{
    if (dt != TGO_F16 && dt != TGO_BF16)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        out[i] = encode(dt, in[i]);
    return 0;
}

int tgo_gelu_array(int64_t n, const double *in, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = tgo_gelu_tanh(in[i]);
    return 0;
}
