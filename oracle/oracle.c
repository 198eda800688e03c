/*
 * oracle.c — plain, slow, obviously correct fp64 CPU reference for the
 * half-precision GEMM and the lower-triangular transposed TRMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no code, header or table
 * with the HIP path.
 *
 * Sources (web pages, cited by title and section):
 *  - "Nvidia Tensor Core-MMA PTX编程入门", §4 (示例): the HGEMM problem
 *    statement, C = A·B with A M×K row-major, B K×N column-major (element
 *    (k, n) at B[k + n·K]) and C M×N row-major, all operands fp16.
 *  - "GPU架构与CUDA", section 共享内存与分块 (tiled matmul): out-of-range
 *    operands contribute nothing and only in-range outputs are written;
 *    section 混合精度核函数: fp16 products accumulated in a wider type; and
 *    section 核函数融合: matmul, bias addition and ReLU as one operation.
 *  - "异构计算中高性能TRMM与TRSM的递归算法实现", §2.1–§2.2: B <- α·Aᵀ·B for
 *    lower-triangular A; §2.3: the triangular solve, here X = α·A⁻ᵀ·B.
 *
 * The oracle computes each output straight from its definition, in fp64
 * (the solve by plain back substitution).
 * fp16 inputs convert to fp64 exactly, every fp16×fp16 product is exact in
 * fp64 (11+11 significand bits), so the only rounding is fp64 summation.
 *
 * Conventions: fp16 operands are passed as their IEEE-754 binary16 bit
 * patterns (uint16_t).  HGEMM matrices use the layouts above with general
 * leading dimensions.  TRMM matrices are column-major: element (r, c) of a
 * column-major matrix X with leading dimension ldx sits at X[r + c·ldx].
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

/* ---- IEEE 754 binary16 decoding, from the format definition ----------------
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 *   exponent 0        : subnormal, value = fraction · 2^-24
 *   exponent 1..30    : normal,    value = (1024 + fraction) · 2^(exponent-25)
 *   exponent 31       : infinity (fraction 0) or NaN
 */
double oracle_half_to_double(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

/* ---- bfloat16 decoding, from the format definition --------------------------
 * 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits (the upper half of an
 * IEEE binary32).
 *   exponent 0        : subnormal, value = fraction · 2^-133
 *   exponent 1..254   : normal,    value = (128 + fraction) · 2^(exponent-134)
 *   exponent 255      : infinity (fraction 0) or NaN
 */
double oracle_bf16_to_double(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 7) & 0xff;
    const int frac = h & 0x7f;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -133);
    else if (expo == 255)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + frac), expo - 134);
    return sign ? -v : v;
}

/* Decoding every pattern once keeps the triple loops below affordable; each
 * entry is exactly oracle_half_to_double of its index. */
static double g_h2d[65536];
static int g_h2d_ready = 0;

static void h2d_init(void)
{
    if (g_h2d_ready)
        return;
    for (int i = 0; i < 65536; ++i)
        g_h2d[i] = oracle_half_to_double((uint16_t)i);
    g_h2d_ready = 1;
}

static double g_b2d[65536];
static int g_b2d_ready = 0;

static void b2d_init(void)
{
    if (g_b2d_ready)
        return;
    for (int i = 0; i < 65536; ++i)
        g_b2d[i] = oracle_bf16_to_double((uint16_t)i);
    g_b2d_ready = 1;
}

/* cin_dtype: 0 fp16, 1 fp32, 2 bf16 */
static double cin_value(const void *Cin, int cin_dtype, int64_t idx)
{
    if (cin_dtype == 0)
        return g_h2d[((const uint16_t *)Cin)[idx]];
    if (cin_dtype == 2)
        return oracle_bf16_to_double(((const uint16_t *)Cin)[idx]);
    return (double)((const float *)Cin)[idx];
}

/* ---- HGEMM: ref = α·A·B + β·C_in ------------------------------------------
 * A   : M×K row-major fp16, element (i,k) at A[i*lda + k]
 * B   : K×N column-major fp16, element (k,j) at B[j*ldb + k]
 * Cin : M×N row-major, fp16 (cin_dtype 0) or fp32 (cin_dtype 1); read only
 *       when beta != 0 (BLAS convention, so a NaN-filled C_in with β = 0
 *       does not leak into the result)
 * ref : M×N row-major fp64, element (i,j) at ref[i*ldr + j]
 * When alpha == 0 the product is not formed (A and B are not read).
 */
void oracle_hgemm(int64_t M, int64_t N, int64_t K, double alpha,
                  const uint16_t *A, int64_t lda,
                  const uint16_t *B, int64_t ldb,
                  double beta, const void *Cin, int64_t ldc, int cin_dtype,
                  double *ref, int64_t ldr)
{
    h2d_init();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0;
            if (alpha != 0.0) {
                for (int64_t k = 0; k < K; ++k)
                    acc += g_h2d[A[i * lda + k]] * g_h2d[B[j * ldb + k]];
            }
            double r = alpha * acc;
            if (beta != 0.0)
                r += beta * cin_value(Cin, cin_dtype, i * ldc + j);
            ref[i * ldr + j] = r;
        }
    }
}

/* Same definition, evaluated only at the listed (rows[s], cols[s]). */
void oracle_hgemm_sampled(int64_t K, double alpha,
                          const uint16_t *A, int64_t lda,
                          const uint16_t *B, int64_t ldb,
                          double beta, const void *Cin, int64_t ldc,
                          int cin_dtype, int64_t nsamp, const int64_t *rows,
                          const int64_t *cols, double *ref)
{
    h2d_init();
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t s = 0; s < nsamp; ++s) {
        const int64_t i = rows[s], j = cols[s];
        double acc = 0.0;
        if (alpha != 0.0) {
            for (int64_t k = 0; k < K; ++k)
                acc += g_h2d[A[i * lda + k]] * g_h2d[B[j * ldb + k]];
        }
        double r = alpha * acc;
        if (beta != 0.0)
            r += beta * cin_value(Cin, cin_dtype, i * ldc + j);
        ref[s] = r;
    }
}

/* ---- GEMM on bf16 operands --------------------------------------------------
 * "GPU架构与CUDA", section 混合精度核函数: the products in a lower-precision type,
 * the sum in a wider one.  The same definition as oracle_hgemm with A and B
 * holding bf16 bit patterns: ref = α·Σ_k A(i,k)·B(k,j) + β·C_in(i,j).
 */
void oracle_gemm_bf16(int64_t M, int64_t N, int64_t K, double alpha,
                      const uint16_t *A, int64_t lda,
                      const uint16_t *B, int64_t ldb,
                      double beta, const void *Cin, int64_t ldc, int cin_dtype,
                      double *ref, int64_t ldr)
{
    h2d_init();
    b2d_init();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0;
            if (alpha != 0.0) {
                for (int64_t k = 0; k < K; ++k)
                    acc += g_b2d[A[i * lda + k]] * g_b2d[B[j * ldb + k]];
            }
            double r = alpha * acc;
            if (beta != 0.0)
                r += beta * cin_value(Cin, cin_dtype, i * ldc + j);
            ref[i * ldr + j] = r;
        }
    }
}

/* The bf16 definition at the listed (rows[s], cols[s]) only. */
void oracle_gemm_bf16_sampled(int64_t K, double alpha,
                              const uint16_t *A, int64_t lda,
                              const uint16_t *B, int64_t ldb,
                              int64_t nsamp, const int64_t *rows,
                              const int64_t *cols, double *ref)
{
    b2d_init();
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t s = 0; s < nsamp; ++s) {
        const int64_t i = rows[s], j = cols[s];
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += g_b2d[A[i * lda + k]] * g_b2d[B[j * ldb + k]];
        ref[s] = alpha * acc;
    }
}

/* ---- HGEMM with a fused bias and activation -------------------------------
 * "GPU架构与CUDA", section 核函数融合: a matmul followed by a bias addition and a
 * ReLU, done as one operation.  Here, per output element
 *   t = α·Σ_k A(i,k)·B(k,j) + β·C_in(i,j) + bias[j],   ref(i,j) = act(t)
 * with bias a length-N vector (one value per column of C; NULL means 0),
 * act 0 = identity and act 1 = ReLU, taken as (t < 0 ? +0 : t) so that a NaN
 * passes through.  Same layouts and α/β conventions as oracle_hgemm.
 */
void oracle_hgemm_bias_act(int64_t M, int64_t N, int64_t K, double alpha,
                           const uint16_t *A, int64_t lda,
                           const uint16_t *B, int64_t ldb,
                           double beta, const void *Cin, int64_t ldc, int cin_dtype,
                           const float *bias, int act, double *ref, int64_t ldr)
{
    h2d_init();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0;
            if (alpha != 0.0) {
                for (int64_t k = 0; k < K; ++k)
                    acc += g_h2d[A[i * lda + k]] * g_h2d[B[j * ldb + k]];
            }
            double t = alpha * acc;
            if (beta != 0.0)
                t += beta * cin_value(Cin, cin_dtype, i * ldc + j);
            if (bias)
                t += (double)bias[j];
            if (act == 1 && t < 0.0)
                t = 0.0;
            ref[i * ldr + j] = t;
        }
    }
}

/* ---- TRMM, left side, A lower triangular, transposed ----------------------
 * ref(i,j) = α · Σ_{k=i}^{n-1} A(k,i) · B(k,j)   for 0 <= i < n, 0 <= j < m
 * This is (α·Aᵀ·B)(i,j) with the strictly upper triangle of A taken as zero:
 * A(k,i) for k < i is never read.
 * A : n×n column-major fp16 (lda >= n); B : n×m column-major fp16 (ldb >= n)
 * ref : n×m column-major fp64, element (i,j) at ref[i + j*ldr]
 */
void oracle_trmm_lower_trans(int64_t n, int64_t m, double alpha,
                             const uint16_t *A, int64_t lda,
                             const uint16_t *B, int64_t ldb,
                             double *ref, int64_t ldr)
{
    h2d_init();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < m; ++j) {
        for (int64_t i = 0; i < n; ++i) {
            double acc = 0.0;
            for (int64_t k = i; k < n; ++k)
                acc += g_h2d[A[k + i * lda]] * g_h2d[B[k + j * ldb]];
            ref[i + j * ldr] = alpha * acc;
        }
    }
}

/* ---- TRMM, left side, any triangle and transposition -----------------------
 * ref(i,j) = α · Σ_k op(A)(i,k) · B(k,j),  op(A) = A or Aᵀ,
 * where only A's stored triangle is read: lower (uplo 0) holds A(r,c) for
 * r >= c, upper (uplo 1) for r <= c; the other triangle counts as zero.
 * ("异构计算中高性能TRMM与TRSM的递归算法实现" §2.1 shows the lower and upper
 * blockings; its §5.1 usage calls the lower, non-transposed product.)
 * A : n×n column-major fp16; B : n×m column-major fp16; ref : n×m column-major.
 */
void oracle_trmm(int uplo, int trans, int64_t n, int64_t m, double alpha,
                 const uint16_t *A, int64_t lda,
                 const uint16_t *B, int64_t ldb,
                 double *ref, int64_t ldr)
{
    h2d_init();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < m; ++j) {
        for (int64_t i = 0; i < n; ++i) {
            double acc = 0.0;
            for (int64_t k = 0; k < n; ++k) {
                const int64_t r = trans ? k : i, c = trans ? i : k;   /* op(A)(i,k) = A(r,c) */
                const int stored = uplo == 0 ? r >= c : r <= c;
                if (stored)
                    acc += g_h2d[A[r + c * lda]] * g_h2d[B[k + j * ldb]];
            }
            ref[i + j * ldr] = alpha * acc;
        }
    }
}

/* oracle_trmm's definition at the listed (rows[s], cols[s]) = (i, j). */
void oracle_trmm_sampled(int uplo, int trans, int64_t n, double alpha,
                         const uint16_t *A, int64_t lda,
                         const uint16_t *B, int64_t ldb,
                         int64_t nsamp, const int64_t *rows,
                         const int64_t *cols, double *ref)
{
    h2d_init();
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t s = 0; s < nsamp; ++s) {
        const int64_t i = rows[s], j = cols[s];
        double acc = 0.0;
        for (int64_t k = 0; k < n; ++k) {
            const int64_t r = trans ? k : i, c = trans ? i : k;
            const int stored = uplo == 0 ? r >= c : r <= c;
            if (stored)
                acc += g_h2d[A[r + c * lda]] * g_h2d[B[k + j * ldb]];
        }
        ref[s] = alpha * acc;
    }
}

/* Same definition at the listed (rows[s], cols[s]) = (i, j) pairs. */
void oracle_trmm_lower_trans_sampled(int64_t n, double alpha,
                                     const uint16_t *A, int64_t lda,
                                     const uint16_t *B, int64_t ldb,
                                     int64_t nsamp, const int64_t *rows,
                                     const int64_t *cols, double *ref)
{
    h2d_init();
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t s = 0; s < nsamp; ++s) {
        const int64_t i = rows[s], j = cols[s];
        double acc = 0.0;
        for (int64_t k = i; k < n; ++k)
            acc += g_h2d[A[k + i * lda]] * g_h2d[B[k + j * ldb]];
        ref[s] = alpha * acc;
    }
}

/* ---- TRSM, left side, A lower triangular, transposed ----------------------
 * "异构计算中高性能TRMM与TRSM的递归算法实现" §2.3 solves X = A\B column by
 * column; this is the transposed lower case, X = α·A⁻ᵀ·B, i.e. the X with
 * Aᵀ·X = α·B.  Aᵀ is upper triangular, so each column j is found by back
 * substitution from the last row:
 *   x(i,j) = (α·B(i,j) − Σ_{k=i+1}^{n-1} A(k,i)·x(k,j)) / A(i,i),
 *   for i = n-1, n-2, …, 0.
 * Only the lower triangle of A is read (A(k,i) with k >= i).  A singular
 * diagonal gives ±inf/NaN as the arithmetic does.
 * A : n×n column-major fp16; B : n×m column-major fp16;
 * ref : n×m column-major fp64, element (i,j) at ref[i + j*ldr]
 */
void oracle_trsm_lower_trans(int64_t n, int64_t m, double alpha,
                             const uint16_t *A, int64_t lda,
                             const uint16_t *B, int64_t ldb,
                             double *ref, int64_t ldr)
{
    h2d_init();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < m; ++j) {
        double *x = ref + j * ldr;
        for (int64_t i = n - 1; i >= 0; --i) {
            double acc = alpha * g_h2d[B[i + j * ldb]];
            for (int64_t k = i + 1; k < n; ++k)
                acc -= g_h2d[A[k + i * lda]] * x[k];
            x[i] = acc / g_h2d[A[i + i * lda]];
        }
    }
}

/* Same solve for the listed columns only: column cols[s] of X goes to
 * ref[0..n-1 + s*ldr]. */
void oracle_trsm_lower_trans_cols(int64_t n, double alpha,
                                  const uint16_t *A, int64_t lda,
                                  const uint16_t *B, int64_t ldb,
                                  int64_t ncols, const int64_t *cols,
                                  double *ref, int64_t ldr)
{
    h2d_init();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t s = 0; s < ncols; ++s) {
        const int64_t j = cols[s];
        double *x = ref + s * ldr;
        for (int64_t i = n - 1; i >= 0; --i) {
            double acc = alpha * g_h2d[B[i + j * ldb]];
            for (int64_t k = i + 1; k < n; ++k)
                acc -= g_h2d[A[k + i * lda]] * x[k];
            x[i] = acc / g_h2d[A[i + i * lda]];
        }
    }
}

/* Number of OpenMP threads a parallel region here would use. */
int oracle_num_threads(void)
{
    int t = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            t = omp_get_num_threads();
#endif
        }
    }
    return t;
}

/* ---- Fused bias and activation on bf16 operands ----------------------------
 * "GPU架构与CUDA", sections 核函数融合 (matmul, bias addition and ReLU as one
 * operation) and 混合精度核函数 (a 16-bit operand type, a wider sum): the
 * definition of oracle_hgemm_bias_act with A and B holding bf16 bit
 * patterns,
 *   v = α·Σ_k A(i,k)·B(k,j) + β·C_in(i,j) + bias[j],   ref(i,j) = act(v)
 * bias NULL adds nothing; act 1 is ReLU (v < 0 becomes +0, NaN passes
 * through); C_in is read only when β != 0 (cin_dtype 1 fp32, 2 bf16).
 */
void oracle_gemm_bf16_bias_act(int64_t M, int64_t N, int64_t K, double alpha,
                               const uint16_t *A, int64_t lda,
                               const uint16_t *B, int64_t ldb,
                               double beta, const void *Cin, int64_t ldc, int cin_dtype,
                               const float *bias, int act, double *ref, int64_t ldr)
{
    h2d_init();
    b2d_init();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double dot = 0.0;
            if (alpha != 0.0) {
                for (int64_t k = 0; k < K; ++k)
                    dot += g_b2d[A[i * lda + k]] * g_b2d[B[j * ldb + k]];
            }
            double v = alpha * dot;
            if (beta != 0.0)
                v += beta * cin_value(Cin, cin_dtype, i * ldc + j);
            if (bias != NULL)
                v += (double)bias[j];
            if (act == 1 && v < 0.0)
                v = 0.0;
            ref[i * ldr + j] = v;
        }
    }
}

/* The fused definition above (and oracle_hgemm_bias_act's) at the listed
 * entries (rows[s], cols[s]) only, for operands of either 16-bit type:
 * in_dtype 0 = fp16, 2 = bf16.  ref[s] = act(α·Σ_k A(i,k)·B(k,j)
 * + β·C_in(i,j) + bias[j]) with i = rows[s], j = cols[s]. */
void oracle_gemm_bias_act_sampled(int in_dtype, int64_t K, double alpha,
                                  const uint16_t *A, int64_t lda,
                                  const uint16_t *B, int64_t ldb,
                                  double beta, const void *Cin, int64_t ldc, int cin_dtype,
                                  const float *bias, int act, int64_t nsamp,
                                  const int64_t *rows, const int64_t *cols, double *ref)
{
    h2d_init();
    b2d_init();
    const double *dec = in_dtype == 2 ? g_b2d : g_h2d;
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t s = 0; s < nsamp; ++s) {
        const int64_t i = rows[s], j = cols[s];
        double dot = 0.0;
        if (alpha != 0.0) {
            for (int64_t k = 0; k < K; ++k)
                dot += dec[A[i * lda + k]] * dec[B[j * ldb + k]];
        }
        double u = alpha * dot;
        if (beta != 0.0)
            u += beta * cin_value(Cin, cin_dtype, i * ldc + j);
        if (bias != NULL)
            u += (double)bias[j];
        if (act == 1 && u < 0.0)
            u = 0.0;
        ref[s] = u;
    }
}

/* Threads for the parallel loops above (n >= 1); the benchmark times the
 * oracle on one thread as well as on all of them.  No arithmetic. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
