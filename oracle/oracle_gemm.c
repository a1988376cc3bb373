/*
 * oracle_gemm.c -- plain CPU reference for the tiled GEMM.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark may load
 * this library.  It shares no code, header, table or helper with the HIP library: it
 * is written from the definition of the product, not from the kernels.
 *
 * What it computes (the definition the tiled, pipelined kernels must reproduce up to
 * fp32 rounding):
 *
 *   out[i][j] = alpha * sum_{k=0}^{K-1} A[i][k] * B[k][j]  (+ beta * C0[i][j] if beta != 0)
 *
 * The accumulation "C += A * B", looped over the K tiles, is section 2 ("Thread Block
 * Tile") of the page "CUTLASS-Cute 初步(6)：CUDA GEMM 计算优化、Multi-Stage 与软流水";
 * its displayed GEMM formula did not survive extraction, so the scaled form above is
 * the BLAS convention, with beta == 0 meaning C0 is never read.  Tiling and pipelining
 * (all four pages) change only the order in which the products are formed, never the
 * sum, so the oracle is the definition written out: one running fp64 sum per output,
 * k ascending, no blocking, no reordering.
 *
 * Layout (BLAS index form; these are the storage conventions the library boundary uses):
 *   A is M x K: row-major A[i*lda + k], column-major A[k*lda + i]
 *   B is K x N: row-major B[k*ldb + j], column-major B[j*ldb + k]
 *   C0 and out are row-major: C0[i*ldc0 + j], out[r*ldo + j]
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math), so every fp
 * operation is the IEEE operation written here.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#include <fenv.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static inline double load_a(int a_col, const double* A, int64_t lda, int64_t i, int64_t k) {
    return a_col ? A[k * lda + i] : A[i * lda + k];
}
static inline double load_b(int b_col, const double* B, int64_t ldb, int64_t k, int64_t j) {
    return b_col ? B[j * ldb + k] : B[k * ldb + j];
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Number of OpenMP threads a parallel region would use (for the benchmark's report). */
int oracle_max_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) return nthreads;
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * fp64 GEMM on exactly-widened inputs.
 * rows == NULL: every row 0..M-1 is computed, out row r is row r.
 * rows != NULL: out row r is C row rows[r], r in [0, nrows)  (sampled checks).
 * Returns 0, or -1 on an argument error.
 *
 * Per output element the sum is a single fp64 accumulator, k ascending.  When B is
 * row-major the j loop is innermost (a row of fp64 accumulators streamed over B's rows);
 * when B is column-major the k loop is innermost (a dot product).  Both orders perform,
 * for every element, the same operations in the same sequence.
 */
int oracle_gemm_f64(int a_col, int b_col, int64_t M, int64_t N, int64_t K,
                    double alpha, const double* A, int64_t lda,
                    const double* B, int64_t ldb,
                    double beta, const double* C0, int64_t ldc0,
                    double* out, int64_t ldo,
                    const int64_t* rows, int64_t nrows, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || ldo < N) return -1;
    if (!rows) nrows = M;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    set_threads(nthreads);
#pragma omp parallel
    {
        double* acc = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t i = rows ? rows[r] : r;
            for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
            if (!b_col) {
                for (int64_t k = 0; k < K; ++k) {
                    const double a = load_a(a_col, A, lda, i, k);
                    const double* brow = B + k * ldb;
                    for (int64_t j = 0; j < N; ++j) acc[j] += a * brow[j];
                }
            } else {
                for (int64_t j = 0; j < N; ++j) {
                    double s = 0.0;
                    for (int64_t k = 0; k < K; ++k) s += load_a(a_col, A, lda, i, k) * load_b(1, B, ldb, k, j);
                    acc[j] = s;
                }
            }
            double* o = out + r * ldo;
            for (int64_t j = 0; j < N; ++j) {
                double v = alpha * acc[j];
                if (beta != 0.0) v += beta * C0[i * ldc0 + j];
                o[j] = v;
            }
        }
        free(acc);
    }
    return 0;
}

/*
 * fp32 model of a register-blocked CUDA-core / VALU kernel: each output is ONE chain of
 * fused multiply-adds in fp32, k ascending, starting from +0 (the thread-tile outer
 * product of section 4, "Thread Tile", on the multi-stage page: every accumulator is
 * updated once per k).  Epilogue: beta == 0 -> alpha*acc (C0 not read), otherwise
 * fmaf(alpha, acc, beta*c0).  A kernel that keeps that per-accumulator order must agree
 * with this bit for bit, whatever its tiling and stage count.
 */
int oracle_sgemm_fma_chain(int a_col, int b_col, int64_t M, int64_t N, int64_t K,
                           float alpha, const float* A, int64_t lda,
                           const float* B, int64_t ldb,
                           float beta, const float* C0, int64_t ldc0,
                           float* out, int64_t ldo,
                           const int64_t* rows, int64_t nrows, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || ldo < N) return -1;
    if (!rows) nrows = M;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        for (int64_t j = 0; j < N; ++j) {
            float acc = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                const float a = a_col ? A[k * lda + i] : A[i * lda + k];
                const float b = b_col ? B[j * ldb + k] : B[k * ldb + j];
                acc = fmaf(a, b, acc);
            }
            float v;
            if (beta == 0.0f) v = alpha * acc;
            else v = fmaf(alpha, acc, beta * C0[i * ldc0 + j]);
            out[r * ldo + j] = v;
        }
    }
    return 0;
}

/*
 * Round-to-nearest-even of a double to a binary format with p significand bits
 * (hidden bit included) and normal exponent range [emin, emax], with gradual underflow
 * and overflow to infinity.  IEEE 754 roundTiesToEven, written from the definition:
 * the representable numbers near x are the multiples of q = 2^(e-p+1), where e is the
 * exponent of x's leading bit clamped below at emin; x/q is exact (power-of-two scale)
 * and rint() rounds it to the nearest integer with ties to even.
 */
static double round_to_format(double x, int p, int emin, int emax) {
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    int E;
    (void)frexp(x, &E);          /* |x| = f * 2^E, f in [0.5, 1) -> leading bit 2^(E-1) */
    int e = E - 1;
    if (e < emin) e = emin;
    const double q = ldexp(1.0, e - p + 1);
    double r = rint(x / q) * q;
    const double maxfin = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    if (fabs(r) > maxfin) r = copysign(INFINITY, x);
    return r;
}

/* In-place rounding of n doubles to bfloat16 (p=8, emin=-126, emax=127), binary16
 * (p=11, emin=-14, emax=15) or binary32 (p=24, emin=-126, emax=127) values.
 * fmt: 0 = fp32, 1 = bf16, 2 = f16.  Returns 0, or -1 for an unknown format. */
int oracle_round(double* x, int64_t n, int fmt) {
    int p, emin, emax;
    switch (fmt) {
        case 0: p = 24; emin = -126; emax = 127; break;
        case 1: p = 8;  emin = -126; emax = 127; break;
        case 2: p = 11; emin = -14;  emax = 15;  break;
        default: return -1;
    }
    if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
    for (int64_t i = 0; i < n; ++i) x[i] = round_to_format(x[i], p, emin, emax);
    return 0;
}

/* Bit patterns of already-rounded values (for comparing with device output words). */
static uint16_t encode_bits(double v, int p, int emin, int ebits) {
    const int mbits = p - 1;
    uint16_t sign = (uint16_t)(signbit(v) ? 1u : 0u);
    const uint16_t emask = (uint16_t)((1u << ebits) - 1u);
    if (isnan(v)) return (uint16_t)((sign << 15) | (emask << mbits) | (1u << (mbits - 1)));
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)((sign << 15) | (emask << mbits));
    if (a == 0.0) return (uint16_t)(sign << 15);
    int E;
    double f = frexp(a, &E);     /* a = f * 2^E */
    int e = E - 1;
    uint32_t biased, mant;
    const int bias = 1 - emin;
    if (e < emin) {              /* subnormal: a = mant * 2^(emin - mbits) */
        biased = 0;
        mant = (uint32_t)ldexp(a, mbits - emin);
    } else {
        biased = (uint32_t)(e + bias);
        mant = (uint32_t)(ldexp(f, p) - ldexp(1.0, mbits));  /* drop the hidden bit */
    }
    return (uint16_t)((sign << 15) | (biased << mbits) | mant);
}

/* fmt: 1 = bf16, 2 = f16.  Input values must already be representable (oracle_round). */
int oracle_encode16(const double* x, uint16_t* bits, int64_t n, int fmt) {
    for (int64_t i = 0; i < n; ++i) {
        if (fmt == 1) bits[i] = encode_bits(x[i], 8, -126, 8);
        else if (fmt == 2) bits[i] = encode_bits(x[i], 11, -14, 5);
        else return -1;
    }
    return 0;
}
