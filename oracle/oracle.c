/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.  The plain CPU reference for C = A*B.
 *
 * Only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this code.  The GPU library never links, includes or
 * calls it, and it shares no source, header, table or helper with the GPU
 * path.
 *
 * What it computes (the plain definition, nothing else):
 *   For 0 <= i < M and 0 <= j < N,  C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]
 *   with A [M,K], B [K,N], C [M,N] all row-major, i.e. the alpha = 1, beta = 0
 *   case of C <- alpha*A*B + beta*C whose old output is never read
 *   ("GEMM From Naive CUDA to Tensor Cores", opening section and
 *   "Compute one output before launching a warp").
 *
 * Precision contract: the inputs are fp16 or bf16 bit patterns (uint16), or
 * 8-bit float patterns (uint8) in the E4M3 or E5M2 formats of the OCP 8-bit
 * floating point specification (OFP8), the 8-bit float the Ada tensor-core
 * GEMM write-up leaves as its untested next step.  Each one is decoded
 * exactly to a double by the bit-level decoders below, and the dot product is
 * accumulated in double, k ascending for every (i, j).  This is the
 * "arithmetic correctness reference" of the two-reference protocol on the same
 * page (section "The two-reference testing protocol": round the inputs to the
 * half format, then accumulate in FP64).  Products of two fp16 (11-bit
 * significand), two bf16 (8-bit) or two 8-bit float (4- or 3-bit) values are
 * exact in double, so the only rounding is the fp64 summation, bounded by
 * (K-1) * 2^-53 * sum|a*b|.
 *
 * Output rounding: oracle_round_to() rounds a double to fp32, fp16 or bf16
 * with IEEE round-to-nearest, ties to even (the mode the rounding demo in
 * section "What FP32 accumulation preserves, and what it can't recover" of the
 * same page relies on).  It is used to build the expected value of bit-exact
 * fixtures whose exact result is not representable in the output format.
 *
 * General form (oracle_gemm_ex_f64), for the fused-epilogue entry point:
 *   C[i][j] = act( alpha * sum_k A[i][k] * B(k, j) + beta * Cold[i][j] + bias[j] )
 *   - alpha, beta: the general C <- alpha*A*B + beta*C the naive-to-tensor-core
 *     page opens with; with beta == 0 the old output is not read at all, so
 *     whatever it holds (even NaN) cannot leak into the result;
 *   - bias: one value per output column, added before the activation, and
 *     act = ReLU (max(x, 0)) or the identity: the bias + ReLU epilogue that
 *     the Ada tensor-core GEMM write-up folds into the kernel (section on the
 *     fused epilogue), applied once to the unrounded value;
 *   - B(k, j) is B[k*ldb + j] for a row-major K x N operand, or B[j*ldb + k]
 *     when B is stored column-major (its N x K transpose row-major), the "TN"
 *     layout the same write-up chose ("A row-major, B column-major").
 *   Everything after the dot product is done in double, once, without
 *   intermediate rounding.
 *
 * Parity pins (tests/test_oracle_pins.py): the page's 2x3 . 3x2 worked example,
 * exact rational brute force on tiny shapes, closed forms (all-ones,
 * identity, permutation, rank-1), the two-reference example, the fp16 rounding
 * table of the precision section, and numpy's IEEE float16 conversion.  The
 * 8-bit formats (tests/test_oracle_f8_pins.py): every code against torch's
 * float8 types, E5M2 as the top byte of binary16, the OFP8 limits, exact
 * rationals and int64 matmuls.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_IN_F16 = 0, ORACLE_IN_BF16 = 1, ORACLE_IN_E4M3 = 2, ORACLE_IN_E5M2 = 3 };
enum { ORACLE_OUT_F32 = 0, ORACLE_OUT_F16 = 1, ORACLE_OUT_BF16 = 2 };
enum { ORACLE_B_ROW_MAJOR = 0, ORACLE_B_COL_MAJOR = 1 };

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Normal:    (1024 + f) * 2^(e - 25)      Subnormal: f * 2^-24 */
double oracle_decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = (f != 0) ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 * Normal:    (128 + f) * 2^(e - 134)      Subnormal: f * 2^-133 */
double oracle_decode_bf16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);
    else if (e == 255)
        v = (f != 0) ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);
    return sign ? -v : v;
}

/* OFP8 E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits, no
 * infinities; exponent 15 with fraction 7 is NaN, so exponent 15 otherwise
 * holds normal numbers (largest 448).
 * Normal:    (8 + f) * 2^(e - 10)         Subnormal: f * 2^-9 */
double oracle_decode_e4m3(uint8_t b) {
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 0xf;
    int f = b & 0x7;
    double v;
    if (e == 15 && f == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)f, -9);
    else
        v = ldexp((double)(8 + f), e - 10);
    return sign ? -v : v;
}

/* OFP8 E5M2: 1 sign bit, 5 exponent bits (bias 15), 2 fraction bits, IEEE
 * special values (exponent 31: infinity for fraction 0, else NaN).
 * Normal:    (4 + f) * 2^(e - 17)         Subnormal: f * 2^-16 */
double oracle_decode_e5m2(uint8_t b) {
    int sign = (b >> 7) & 1;
    int e = (b >> 2) & 0x1f;
    int f = b & 0x3;
    double v;
    if (e == 0)
        v = ldexp((double)f, -16);
    else if (e == 31)
        v = (f != 0) ? NAN : INFINITY;
    else
        v = ldexp((double)(4 + f), e - 17);
    return sign ? -v : v;
}

/* Element idx of an operand stored as bit patterns of in_fmt: uint16 for
 * the 16-bit formats, uint8 for the 8-bit ones. */
static double load_in(int in_fmt, const void* base, int64_t idx) {
    switch (in_fmt) {
    case ORACLE_IN_BF16: return oracle_decode_bf16(((const uint16_t*)base)[idx]);
    case ORACLE_IN_E4M3: return oracle_decode_e4m3(((const uint8_t*)base)[idx]);
    case ORACLE_IN_E5M2: return oracle_decode_e5m2(((const uint8_t*)base)[idx]);
    default:             return oracle_decode_f16(((const uint16_t*)base)[idx]);
    }
}

/* Round-to-nearest-even of a non-negative double q to an integer, written
 * out: q < 2^53 here, so q - floor(q) is exact. */
static double rne_integer(double q) {
    double fl = floor(q);
    double d = q - fl;
    if (d > 0.5) return fl + 1.0;
    if (d < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* Round x to a binary format with p significand bits (hidden bit included),
 * minimum normal exponent emin and maximum exponent emax, IEEE RNE.
 * Returns the rounded value as a double (+-inf on overflow, NaN kept). */
static double round_generic(double x, int p, int emin, int emax) {
    if (isnan(x)) return x;
    if (x == 0.0 || isinf(x)) return x;
    double a = fabs(x);
    int E;                       /* a = m * 2^E, m in [0.5, 1) */
    frexp(a, &E);
    int e = E - 1;               /* a in [2^e, 2^(e+1)) */
    if (e < emin) e = emin;      /* subnormal range: fixed quantum 2^(emin-p+1) */
    double quantum = ldexp(1.0, e - p + 1);
    double q = rne_integer(a / quantum);   /* exact scaling by a power of two */
    double r = q * quantum;
    /* overflow: anything that rounds to 2^(emax+1) or above is infinite */
    if (r >= ldexp(1.0, emax + 1)) r = INFINITY;
    return x < 0 ? -r : r;
}

double oracle_round_to(int out_fmt, double x) {
    switch (out_fmt) {
    case ORACLE_OUT_F16:  return round_generic(x, 11, -14, 15);
    case ORACLE_OUT_BF16: return round_generic(x, 8, -126, 127);
    default:              return round_generic(x, 24, -126, 127);
    }
}

/* Spacing of the output format at r: 2^(floor(log2|r|) - p + 1), floored at
 * the format's smallest subnormal (also the value used for r == 0). */
double oracle_ulp(int out_fmt, double r) {
    int p, emin;
    switch (out_fmt) {
    case ORACLE_OUT_F16:  p = 11; emin = -14;  break;
    case ORACLE_OUT_BF16: p = 8;  emin = -126; break;
    default:              p = 24; emin = -126; break;
    }
    double a = fabs(r);
    int e = emin;
    if (a != 0.0 && isfinite(a)) {
        int E;
        frexp(a, &E);
        e = E - 1;
        if (e < emin) e = emin;
    }
    return ldexp(1.0, e - p + 1);
}

/* Element-wise forms of the two functions above over n doubles, so that a
 * whole output matrix is rounded or measured in one call. */
void oracle_round_to_array(int out_fmt, const double* x, double* dst, int64_t n) {
    for (int64_t t = 0; t < n; ++t) dst[t] = oracle_round_to(out_fmt, x[t]);
}

void oracle_ulp_array(int out_fmt, const double* r, double* dst, int64_t n) {
    for (int64_t t = 0; t < n; ++t) dst[t] = oracle_ulp(out_fmt, r[t]);
}

void oracle_decode_array(int in_fmt, const void* src, double* dst, int64_t n) {
    for (int64_t t = 0; t < n; ++t) dst[t] = load_in(in_fmt, src, t);
}

/* ------------------------------------------------------------------------
 * The triple loop.  Row i of C (or of the selected rows) is
 *   acc[j] = 0;  for k = 0..K-1: a = A[i][k]; for j: acc[j] += a * B[k][j]
 * which is k ascending for every (i, j).  B is decoded once into doubles.
 * ------------------------------------------------------------------------ */
typedef struct {
    const void* A; int64_t lda;      /* elements of in_fmt */
    const double* Bd;              /* K x N decoded, row-major, stride N */
    double* C; int64_t ldc;
    const int64_t* rows;           /* NULL: rows r0..r1-1 of A; else rows[r] */
    int64_t r0, r1;
    int64_t N, K;
    int in_fmt;
} oracle_job_t;

static void* oracle_worker(void* arg) {
    oracle_job_t* jb = (oracle_job_t*)arg;
    for (int64_t r = jb->r0; r < jb->r1; ++r) {
        int64_t i = jb->rows ? jb->rows[r] : r;
        double* c = jb->C + r * jb->ldc;
        for (int64_t j = 0; j < jb->N; ++j) c[j] = 0.0;
        for (int64_t k = 0; k < jb->K; ++k) {
            double a = load_in(jb->in_fmt, jb->A, i * jb->lda + k);
            const double* b = jb->Bd + k * jb->N;
            for (int64_t j = 0; j < jb->N; ++j) c[j] += a * b[j];
        }
    }
    return NULL;
}

static int run_rows(int in_fmt, int b_layout, int64_t nrows, const int64_t* rows, int64_t N,
                    int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                    double* C, int64_t ldc, int nthreads) {
    if (nrows <= 0 || N <= 0) return 0;
    double* Bd = NULL;
    if (K > 0) {
        Bd = (double*)malloc((size_t)K * (size_t)N * sizeof(double));
        if (!Bd) return -1;
        if (b_layout == ORACLE_B_COL_MAJOR) {
            /* B(k, j) = B[j*ldb + k]: column j of the K x N operand is row j in memory */
            for (int64_t j = 0; j < N; ++j)
                for (int64_t k = 0; k < K; ++k) Bd[k * N + j] = load_in(in_fmt, B, j * ldb + k);
        } else {
            for (int64_t k = 0; k < K; ++k)
                for (int64_t j = 0; j < N; ++j) Bd[k * N + j] = load_in(in_fmt, B, k * ldb + j);
        }
    }
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = (int)nrows;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    oracle_job_t* jobs = (oracle_job_t*)malloc(sizeof(oracle_job_t) * (size_t)nthreads);
    char* spawned = (char*)calloc((size_t)nthreads, 1);
    if (!th || !jobs || !spawned) { free(Bd); free(th); free(jobs); free(spawned); return -1; }
    int64_t per = (nrows + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        oracle_job_t* jb = &jobs[t];
        jb->A = A; jb->lda = lda; jb->Bd = Bd; jb->C = C; jb->ldc = ldc;
        jb->rows = rows; jb->N = N; jb->K = K; jb->in_fmt = in_fmt;
        jb->r0 = t * per;
        jb->r1 = (t + 1) * per < nrows ? (t + 1) * per : nrows;
        if (jb->r0 >= jb->r1) continue;
        if (nthreads > 1 && pthread_create(&th[t], NULL, oracle_worker, jb) == 0)
            spawned[t] = 1;
        else
            oracle_worker(jb);          /* single thread, or could not spawn */
    }
    for (int t = 0; t < nthreads; ++t)
        if (spawned[t]) pthread_join(th[t], NULL);
    free(Bd); free(th); free(jobs); free(spawned);
    return 0;
}

/* Full product: C (M x N doubles, stride ldc) = A (M x K, stride lda) *
 * B (K x N, stride ldb); strides in elements of in_fmt.  Returns 0, or -1 on
 * allocation failure. */
int oracle_gemm_f64(int64_t M, int64_t N, int64_t K, int in_fmt,
                    const void* A, int64_t lda, const void* B, int64_t ldb,
                    double* C, int64_t ldc, int nthreads) {
    return run_rows(in_fmt, ORACLE_B_ROW_MAJOR, M, NULL, N, K, A, lda, B, ldb, C, ldc, nthreads);
}

/* Selected rows only: C is nrows x N (stride ldc); output row r is row rows[r]. */
int oracle_gemm_rows_f64(int64_t nrows, const int64_t* rows, int64_t N, int64_t K, int in_fmt,
                         const void* A, int64_t lda, const void* B, int64_t ldb,
                         double* C, int64_t ldc, int nthreads) {
    return run_rows(in_fmt, ORACLE_B_ROW_MAJOR, nrows, rows, N, K, A, lda, B, ldb, C, ldc, nthreads);
}

/* The general form.  Output row r (0 <= r < nrows) is row i = rows[r] of the
 * result (rows == NULL: i = r).  B is read as B(k, j) per b_layout.  Cold holds
 * the old output values of the same selected rows as doubles (row r at
 * Cold + r*ldcold); it is not read when beta == 0 and may then be NULL.  bias
 * holds N doubles or is NULL (no bias).  relu != 0 applies max(x, 0) last.
 * Returns 0, -1 on allocation failure, -2 on a bad layout code. */
int oracle_gemm_ex_f64(int64_t nrows, const int64_t* rows, int64_t N, int64_t K, int in_fmt,
                       int b_layout, const void* A, int64_t lda, const void* B, int64_t ldb,
                       double alpha, double beta, const double* Cold, int64_t ldcold,
                       const double* bias, int relu, double* C, int64_t ldc, int nthreads) {
    if (b_layout != ORACLE_B_ROW_MAJOR && b_layout != ORACLE_B_COL_MAJOR) return -2;
    int rc = run_rows(in_fmt, b_layout, nrows, rows, N, K, A, lda, B, ldb, C, ldc, nthreads);
    if (rc != 0) return rc;
    for (int64_t r = 0; r < nrows; ++r) {
        double* c = C + r * ldc;
        for (int64_t j = 0; j < N; ++j) {
            double v = alpha * c[j];
            if (beta != 0.0) v += beta * Cold[r * ldcold + j];
            if (bias) v += bias[j];
            if (relu && v < 0.0) v = 0.0;
            c[j] = v;
        }
    }
    return 0;
}
