/*
 * oracle.c -- the CPU oracle for C = A * B^T.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * load this file's library.  The GPU library shares no code with it: no
 * header, table, helper or constant generator.
 *
 * What it computes.  The pages ("HipKittens: fast and furious AMD kernels",
 * GeekNews summary, section "Performance results") name a GEMM kernel that is
 * fastest "in both BF16 and FP8"; the companion page ("How to make AMD GPUs go
 * brrr", section "Real kernel example") says its hot loop is the BF16 GEMM.
 * Neither page writes the product out, so the oracle is the textbook
 * definition of a matrix product with the second operand stored by rows:
 *
 *     C[i][j] = RNE_bf16( s * sum_{k=0..K-1} dec(A[i*lda+k]) * dec(B[j*ldb+k]) )
 *
 * with s = 1 for BF16 inputs and s = sA*sB for FP8 inputs.  The FP8 format is
 * the OCP E4M3FN encoding with one fp32 scale per tensor; the pages only quote
 * an MXFP8 peak rate and give no scaling scheme, so this is a reading, listed
 * with the others in the design notes.
 *
 * Arithmetic.  Everything is in IEEE double.  Every product of two decoded
 * bf16 (8-bit significand) or e4m3 (4-bit significand) values is exact in
 * double; the sum is taken in ascending k from +0.0 with one rounding per add
 * (compiled without fast-math and without FMA contraction); the scale is
 * applied once, and the result is rounded ONCE from double to bf16 with
 * round-to-nearest-even (no float intermediate, which would round twice).
 *
 * Alongside C the oracle returns S[i][j] = |s| * sum_k |dec(a)*dec(b)|, the
 * magnitude sum that the tolerance |C_gpu - C_ref| <= ulp(C_ref) + 1e-4*S uses.
 *
 * The file also holds the attention-forward oracle (its own section, at the
 * end) and the MXFP8 product.
 *
 * Pins (tests marked "not gpu"): integer-valued inputs against an int64
 * product, exact rational sums with fractions.Fraction on tiny shapes, an
 * identity B, the transpose identity, the e4m3 table against torch's
 * float8_e4m3fn, the rounding function against torch's float->bf16 cast, and
 * hand-derived fixtures under tests/golden/.
 */
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BF16 0
#define ORACLE_E4M3 1

/* bf16 is the top half of an IEEE binary32 word: widen and reinterpret. */
double oracle_bf16_decode(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
 * S.1111.111 is NaN; exponent field 0 encodes subnormals m * 2^-9.
 * Largest finite value 448 = 1.75 * 2^8, smallest subnormal 2^-9.
 */
double oracle_e4m3_decode(uint8_t b)
{
    int s = b >> 7;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/*
 * Round a double to the nearest bf16 value, ties to even, in one step.
 * bf16 keeps 8 significant bits (7 stored), exponent range of binary32.
 * The quantum of the binade of |x| is 2^(max(floor(log2|x|), -126) - 7);
 * below 2^-126 the quantum stays 2^-133 (gradual underflow).  Results of
 * magnitude 2^128 or more are infinities; NaN maps to the quiet NaN 0x7FC0.
 */
uint16_t oracle_bf16_round(double x)
{
    int sign, e, E;
    double ax, q, r;
    float f;
    uint32_t u;
    uint16_t bits;

    if (isnan(x))
        return 0x7FC0;
    sign = signbit(x) ? 1 : 0;
    ax = fabs(x);
    if (isinf(ax))
        return sign ? 0xFF80 : 0x7F80;
    if (ax == 0.0)
        return sign ? 0x8000 : 0x0000;
    frexp(ax, &e);           /* ax = f * 2^e with f in [0.5, 1) */
    E = e - 1;               /* floor(log2 ax) */
    if (E < -126)
        E = -126;
    q = ldexp(1.0, E - 7);
    r = rint(ax / q) * q;    /* ax / q is exact; rint rounds half to even */
    if (r >= ldexp(1.0, 128))
        return sign ? 0xFF80 : 0x7F80;
    f = (float)r;            /* exact: at most 8 significant bits, in range */
    memcpy(&u, &f, sizeof u);
    bits = (uint16_t)(u >> 16);
    return (uint16_t)(sign ? (bits | 0x8000u) : bits);
}

static double decode_elem(int dtype, const void *base, int64_t idx,
                          const double *e4m3_table)
{
    if (dtype == ORACLE_BF16)
        return oracle_bf16_decode(((const uint16_t *)base)[idx]);
    return e4m3_table[((const uint8_t *)base)[idx]];
}

/* One output element: the dot product in ascending k, then the scale. */
static void dot_one(int dtype, const void *A, const void *B, int64_t i, int64_t j,
                    int64_t K, int64_t lda, int64_t ldb, double s,
                    const double *tab, double *c_out, double *s_out)
{
    double acc = 0.0, mag = 0.0;
    int64_t k;
    for (k = 0; k < K; ++k) {
        double a = decode_elem(dtype, A, i * lda + k, tab);
        double b = decode_elem(dtype, B, j * ldb + k, tab);
        double p = a * b;
        acc = acc + p;
        mag = mag + fabs(p);
    }
    *c_out = acc * s;
    *s_out = mag * fabs(s);
}

static int check_args(int dtype, const void *A, const void *B, int64_t M, int64_t N,
                      int64_t K, int64_t lda, int64_t ldb)
{
    if (dtype != ORACLE_BF16 && dtype != ORACLE_E4M3)
        return 1;
    if (M < 0 || N < 0 || K < 0)
        return 1;
    if (K > 0 && ((M > 0 && (A == NULL || lda < K)) || (N > 0 && (B == NULL || ldb < K))))
        return 1;
    return 0;
}

/*
 * Full product.  C (bf16 bits, row stride ldc) and S (double, row stride N,
 * may be NULL) are written for 0 <= i < M, 0 <= j < N; nothing else is
 * touched.  Returns 0 on success, 1 on invalid arguments.
 */
int oracle_gemm(int dtype, const void *A, const void *B, uint16_t *C, double *S,
                int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                double scale_a, double scale_b, int nthreads)
{
    double tab[256];
    double s = (dtype == ORACLE_E4M3) ? scale_a * scale_b : 1.0;
    int64_t i;
    int t;

    if (check_args(dtype, A, B, M, N, K, lda, ldb) || ldc < N || (M > 0 && N > 0 && C == NULL))
        return 1;
    for (t = 0; t < 256; ++t)
        tab[t] = oracle_e4m3_decode((uint8_t)t);
    if (nthreads < 1)
        nthreads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (i = 0; i < M; ++i) {
        int64_t j;
        for (j = 0; j < N; ++j) {
            double c, m;
            dot_one(dtype, A, B, i, j, K, lda, ldb, s, tab, &c, &m);
            C[i * ldc + j] = oracle_bf16_round(c);
            if (S)
                S[i * N + j] = m;
        }
    }
    return 0;
}

/*
 * Selected entries only: for p in [0, n) compute C[rows[p]][cols[p]] and its
 * magnitude sum.  This lets full-size products be checked on a sample.
 */
int oracle_gemm_sampled(int dtype, const void *A, const void *B,
                        int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                        const int64_t *rows, const int64_t *cols, int64_t n,
                        double scale_a, double scale_b,
                        uint16_t *c_out, double *s_out, int nthreads)
{
    double tab[256];
    double s = (dtype == ORACLE_E4M3) ? scale_a * scale_b : 1.0;
    int64_t p;
    int t;

    if (check_args(dtype, A, B, M, N, K, lda, ldb) || n < 0)
        return 1;
    for (p = 0; p < n; ++p)
        if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N)
            return 1;
    for (t = 0; t < 256; ++t)
        tab[t] = oracle_e4m3_decode((uint8_t)t);
    if (nthreads < 1)
        nthreads = 1;

#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
    for (p = 0; p < n; ++p) {
        double c, m;
        dot_one(dtype, A, B, rows[p], cols[p], K, lda, ldb, s, tab, &c, &m);
        c_out[p] = oracle_bf16_round(c);
        if (s_out)
            s_out[p] = m;
    }
    return 0;
}

/* Vector forms of the scalar helpers, for the self-checks. */
void oracle_bf16_round_n(const double *x, uint16_t *out, int64_t n)
{
    int64_t p;
    for (p = 0; p < n; ++p)
        out[p] = oracle_bf16_round(x[p]);
}

void oracle_e4m3_table(double *out256)
{
    int t;
    for (t = 0; t < 256; ++t)
        out256[t] = oracle_e4m3_decode((uint8_t)t);
}

int oracle_num_threads_available(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * ---------------------------------------------------------------- MXFP8
 *
 * Block-scaled FP8 ("MXFP8", the format of the pages' 5.0 PF FP8 peak in "How
 * to make AMD GPUs go brrr", section "AMD CDNA GPU structure").  The pages
 * name the format only; its definition is the OCP Microscaling (MX) Formats
 * specification v1.0: along K, every block of 32 consecutive elements of a
 * row shares one scale X in E8M0, an 8-bit biased exponent (bias 127) with
 * value 2^(x - 127), where x = 255 encodes NaN.  The elements are E4M3FN, and
 * an element's value is X * dec(element).  The product is then
 *
 *     C[i][j] = RNE_bf16( sum_k XA[i][k/32] dec(A[i][k]) * XB[j][k/32] dec(B[j][k]) )
 *
 * with XA stored as an M x ceil(K/32) byte array of row stride ldsa and XB as
 * N x ceil(K/32) of row stride ldsb (a last block shorter than 32 keeps its
 * scale).  Each term is exact in double (the element product has at most 8
 * significant bits, the scales are powers of two far inside double's range),
 * and the sum, the magnitude sum and the rounding follow the plain product
 * above: ascending k from +0.0, one rounding per add, one final rounding.
 */
double oracle_e8m0_decode(uint8_t x)
{
    if (x == 255)
        return NAN;
    return ldexp(1.0, (int)x - 127);
}

static void dot_one_mx(const uint8_t *A, const uint8_t *B, const uint8_t *SA,
                       const uint8_t *SB, int64_t i, int64_t j, int64_t K, int64_t lda,
                       int64_t ldb, int64_t ldsa, int64_t ldsb, const double *tab,
                       const double *xtab, double *c_out, double *s_out)
{
    double acc = 0.0, mag = 0.0;
    int64_t k;
    for (k = 0; k < K; ++k) {
        double a = xtab[SA[i * ldsa + k / 32]] * tab[A[i * lda + k]];
        double b = xtab[SB[j * ldsb + k / 32]] * tab[B[j * ldb + k]];
        double p = a * b;
        acc = acc + p;
        mag = mag + fabs(p);
    }
    *c_out = acc;
    *s_out = mag;
}

static int check_args_mx(const void *A, const void *B, const void *SA, const void *SB,
                         int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                         int64_t ldsa, int64_t ldsb)
{
    int64_t nb = (K + 31) / 32;
    if (check_args(ORACLE_E4M3, A, B, M, N, K, lda, ldb))
        return 1;
    if (K > 0 && ((M > 0 && (SA == NULL || ldsa < nb)) || (N > 0 && (SB == NULL || ldsb < nb))))
        return 1;
    return 0;
}

static void mx_tables(double *tab, double *xtab)
{
    int t;
    for (t = 0; t < 256; ++t) {
        tab[t] = oracle_e4m3_decode((uint8_t)t);
        xtab[t] = oracle_e8m0_decode((uint8_t)t);
    }
}

/* Full MXFP8 product; C, S and the return value as for oracle_gemm. */
int oracle_gemm_mx(const uint8_t *A, const uint8_t *B, const uint8_t *SA, const uint8_t *SB,
                   uint16_t *C, double *S, int64_t M, int64_t N, int64_t K, int64_t lda,
                   int64_t ldb, int64_t ldsa, int64_t ldsb, int64_t ldc, int nthreads)
{
    double tab[256], xtab[256];
    int64_t i;

    if (check_args_mx(A, B, SA, SB, M, N, K, lda, ldb, ldsa, ldsb) || ldc < N ||
        (M > 0 && N > 0 && C == NULL))
        return 1;
    mx_tables(tab, xtab);
    if (nthreads < 1)
        nthreads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (i = 0; i < M; ++i) {
        int64_t j;
        for (j = 0; j < N; ++j) {
            double c, m;
            dot_one_mx(A, B, SA, SB, i, j, K, lda, ldb, ldsa, ldsb, tab, xtab, &c, &m);
            C[i * ldc + j] = oracle_bf16_round(c);
            if (S)
                S[i * N + j] = m;
        }
    }
    return 0;
}

/* Selected entries of the MXFP8 product, as oracle_gemm_sampled. */
int oracle_gemm_mx_sampled(const uint8_t *A, const uint8_t *B, const uint8_t *SA,
                           const uint8_t *SB, int64_t M, int64_t N, int64_t K, int64_t lda,
                           int64_t ldb, int64_t ldsa, int64_t ldsb, const int64_t *rows,
                           const int64_t *cols, int64_t n, uint16_t *c_out, double *s_out,
                           int nthreads)
{
    double tab[256], xtab[256];
    int64_t p;

    if (check_args_mx(A, B, SA, SB, M, N, K, lda, ldb, ldsa, ldsb) || n < 0)
        return 1;
    for (p = 0; p < n; ++p)
        if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N)
            return 1;
    mx_tables(tab, xtab);
    if (nthreads < 1)
        nthreads = 1;

#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
    for (p = 0; p < n; ++p) {
        double c, m;
        dot_one_mx(A, B, SA, SB, rows[p], cols[p], K, lda, ldb, ldsa, ldsb, tab, xtab, &c, &m);
        c_out[p] = oracle_bf16_round(c);
        if (s_out)
            s_out[p] = m;
    }
    return 0;
}

/* ------------------------------------------------------------ attention
 *
 * Attention forward, the second workload of the pages ("How to make AMD GPUs
 * go brrr", section "Real kernel example": its hot loop runs the same wave
 * schedule as the BF16 GEMM; "HipKittens: fast and furious AMD kernels",
 * section "Performance results": causal and non-causal, several head
 * dimensions D and sequence lengths N).  The pages do not write the operation
 * out; the oracle takes textbook scaled dot-product attention over BF16
 * inputs, one query row at a time:
 *
 *     s_j   = scale * sum_{d<D} q[d] * k_j[d]      for j < N (j <= i if causal)
 *     O_i   = RNE_bf16( sum_j exp(s_j - m) * v_j / sum_j exp(s_j - m) ),  m = max_j s_j
 *     LSE_i = m + log(sum_j exp(s_j - m))
 *
 * Query head h reads key/value head h / (Hq / Hkv) (grouped-query attention:
 * each key/value head serves Hq / Hkv consecutive query heads).  Element
 * (b, h, t, d) of a tensor sits at b*s[0] + h*s[1] + t*s[2] + d.
 *
 * In double: exact products, ascending sums, one exp per score, one rounding
 * to bf16 at the end.  Alongside O the oracle returns, per element,
 * A = sum_j p_j |v_j[d]| / sum_j p_j, the magnitude the tolerance uses.
 */
static int check_args_attn(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t B,
                           int64_t Hq, int64_t Hkv, int64_t N, int64_t D, const int64_t *sq,
                           const int64_t *sk, const int64_t *sv)
{
    if (B < 0 || Hq < 1 || Hkv < 1 || N < 0 || D < 1 || Hq % Hkv != 0)
        return 1;
    if (Q == NULL || K == NULL || V == NULL || sq == NULL || sk == NULL || sv == NULL)
        return 1;
    return 0;
}

/* One query row r = (b * Hq + h) * N + i: O[0..D), and optionally its double
 * values, LSE and A.  s is scratch for N scores. */
static void attn_row(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t Hq,
                     int64_t Hkv, int64_t N, int64_t D, const int64_t *sq, const int64_t *sk,
                     const int64_t *sv, double scale, int causal, int64_t r, double *s,
                     uint16_t *o, double *o64, double *lse, double *amag)
{
    const int64_t i = r % N;
    const int64_t h = (r / N) % Hq;
    const int64_t b = r / (N * Hq);
    const int64_t kvh = h / (Hq / Hkv);
    const int64_t nk = causal ? i + 1 : N;
    const uint16_t *q = Q + b * sq[0] + h * sq[1] + i * sq[2];
    double m = -INFINITY, l = 0.0;
    int64_t j, d;

    for (j = 0; j < nk; ++j) {
        const uint16_t *kj = K + b * sk[0] + kvh * sk[1] + j * sk[2];
        double acc = 0.0;
        for (d = 0; d < D; ++d)
            acc += oracle_bf16_decode(q[d]) * oracle_bf16_decode(kj[d]);
        s[j] = scale * acc;
        if (s[j] > m)
            m = s[j];
    }
    for (j = 0; j < nk; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (d = 0; d < D; ++d) {
        double acc = 0.0, mag = 0.0, val;
        for (j = 0; j < nk; ++j) {
            const double v = oracle_bf16_decode(V[b * sv[0] + kvh * sv[1] + j * sv[2] + d]);
            acc += s[j] * v;
            mag += s[j] * fabs(v);
        }
        val = acc / l;
        o[d] = oracle_bf16_round(val);
        if (o64)
            o64[d] = val;
        if (amag)
            amag[d] = mag / l;
    }
    if (lse)
        *lse = m + log(l);
}

/*
 * Attention forward for the query rows listed in rows[0..nrows) (each
 * (b * Hq + h) * N + i), or for every row (B * Hq * N of them, in that order)
 * when rows is NULL.  Q is B x Hq x N x D, K and V are B x Hkv x N x D, with
 * strides sq, sk, sv (batch, head, token; elements).  Outputs, nrows x D
 * (nrows x 1 for lse): o (bf16 bits, required), o64, lse and amag (optional).
 * Returns 0; 1 for invalid arguments (nothing written); 2 if scratch memory
 * for the scores could not be allocated.
 */
int oracle_attn_fwd(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t B,
                    int64_t Hq, int64_t Hkv, int64_t N, int64_t D, const int64_t *sq,
                    const int64_t *sk, const int64_t *sv, double scale, int causal,
                    const int64_t *rows, int64_t nrows, uint16_t *o, double *o64, double *lse,
                    double *amag, int nthreads)
{
    const int64_t total = B * Hq * N;
    int64_t p;
    int failed = 0;

    if (check_args_attn(Q, K, V, B, Hq, Hkv, N, D, sq, sk, sv) || o == NULL)
        return 1;
    if (rows == NULL)
        nrows = total;
    if (nrows < 0)
        return 1;
    if (rows)
        for (p = 0; p < nrows; ++p)
            if (rows[p] < 0 || rows[p] >= total)
                return 1;
    if (nthreads < 1)
        nthreads = 1;

#pragma omp parallel num_threads(nthreads)
    {
        double *s = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (s == NULL) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (p = 0; p < nrows; ++p) {
            const int64_t r = rows ? rows[p] : p;
            if (s)
                attn_row(Q, K, V, Hq, Hkv, N, D, sq, sk, sv, scale, causal, r, s, o + p * D,
                         o64 ? o64 + p * D : NULL, lse ? lse + p : NULL,
                         amag ? amag + p * D : NULL);
        }
        free(s);
    }
    return failed ? 2 : 0;
}
