/*
 * lse_oracle.c - float64 reference for the row-wise log-sum-exp.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link
 * or call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code with the HIP library.
 *
 * What it computes. For every row r of a row-major matrix x with `cols`
 * elements per row and `row_stride` elements between row starts,
 *
 *     out[r] = LSE(x[r, :]) = log( sum_j exp(x[r, j]) ),
 *
 * the natural-log log-sum-exp that the paper "Speeding up Log-Sum-Exp:
 * Kernel Fusion at the Memory Wall, Integer Arithmetic at the Compute Wall"
 * names as its primitive (title, abstract, §1) and reduces over the last
 * axis of a (B, N) tensor, one scalar per row (§2.1, §3.1). The output is in
 * base e, as the paper's integer variant converts its result back to base-e
 * float32 (§3.2).
 *
 * How. The plain max-subtract definition, the recipe of the PyTorch baseline
 * that the paper profiles (§2.1, Figure 1), in float64 as the paper's
 * accuracy reference is FP64 (§4):
 *     m = max_j x_j,   s = sum_j exp(x_j - m)  (in ascending j),
 *     out = m + log(s).
 * Elements are widened exactly to double: fp32 directly, bf16 by placing its
 * 16 bits in the high half of an fp32 word, fp16 (IEEE binary16) from its
 * fields (sign, 5-bit exponent with bias 15, 10-bit fraction; exponent 0
 * is zero or subnormal, fraction * 2^-24; exponent 31 is inf or NaN).
 * Nothing is flushed to zero. The 16-bit inputs follow the paper's
 * reduced-bit FuseLSE16 (§4.3, Figure 5), read as FuseLSE over 16-bit data;
 * the arithmetic here stays float64.
 *
 * Special cases (the paper lists edge-case handling in its Table 3 without
 * the cells; these follow torch.logsumexp, which it replaces as a drop-in):
 *     any NaN in the row            -> NaN
 *     cols == 0, or every x = -inf  -> -inf
 *     otherwise a +inf in the row   -> +inf
 *
 * Token log-probabilities (lse_oracle_token_logprob_f64). The paper names
 * per-token LLM log-probabilities as a use of LSE (§1) and benchmarks the
 * RLHF log-probability computation over vocabularies of 32K to 256K (§2,
 * §5.1): the log-probability of token t under a softmax over the row,
 *     logp[r] = x[r, t] - LSE(x[r, :]),   t = targets[r],
 * in float64 with the LSE above. A target outside [0, cols) gives NaN; the
 * special values follow from IEEE arithmetic on the definition.
 *
 * Backward pass (lse_oracle_softmax_grad_f64). The gradient of LSE(x[r, :])
 * with respect to x[r, j] is exp(x[r, j] - LSE(x[r, :])), the row's softmax;
 * the paper tabulates backward support for its kernels (Table 3). Given the
 * forward value lse[r] and an incoming gradient grad_out[r] (both fp32, as a
 * caller holds them), the oracle writes
 *     out[r, j] = grad_out[r] * exp(x[r, j] - lse[r])
 * in float64, row r at out + r * cols.
 *
 * Backward of the token log-probability (lse_oracle_token_logprob_grad_f64).
 * logp[r] = x[r, t] - LSE(x[r, :]) has derivative [j == t] - softmax_j with
 * respect to x[r, j]; with the forward LSE lse[r] and an incoming gradient
 * grad_logp[r] (both fp32), the oracle writes
 *     out[r, j] = grad_logp[r] * ([j == t] - exp(x[r, j] - lse[r]))
 * in float64. A target outside [0, cols) (whose log-probability is NaN)
 * gives a row of NaN.
 *
 * The rows are split over `nthreads` POSIX threads; a row's arithmetic does
 * not depend on the thread count.
 *
 * Parity pins: every function here is pinned by tests against closed forms,
 * brute force and a library routine; see tests/test_oracle.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F16 = 2 };

/* IEEE binary16 bits to double, from the format's definition. */
static double half_to_double(uint16_t h)
{
    const int sign = h >> 15;
    const int e = (h >> 10) & 0x1F;
    const int frac = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)frac, -24);                   /* zero, subnormal */
    else if (e == 31)
        v = frac ? NAN : INFINITY;                      /* inf, NaN */
    else
        v = ldexp((double)(1024 + frac), e - 25);       /* (1 + frac/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Exact widening of the element at `index` (in elements from x) to double. */
static double load_elem(const void *x, int dtype, int64_t index)
{
    if (dtype == ORACLE_F32) {
        float f;
        memcpy(&f, (const char *)x + 4 * index, 4);
        return (double)f;
    } else if (dtype == ORACLE_F16) {
        uint16_t h;
        memcpy(&h, (const char *)x + 2 * index, 2);
        return half_to_double(h);
    } else {
        uint16_t h;
        uint32_t w;
        float f;
        memcpy(&h, (const char *)x + 2 * index, 2);
        w = (uint32_t)h << 16;
        memcpy(&f, &w, 4);
        return (double)f;
    }
}

/* The log-sum-exp of one row in float64: max, then the shifted exp-sum. */
static double lse_one_row(const void *x, int dtype, int64_t start, int64_t cols)
{
    double m = -INFINITY;
    double s = 0.0;
    int64_t j;

    if (cols == 0)
        return -INFINITY;

    /* First pass: the row maximum; a NaN anywhere makes the result NaN. */
    for (j = 0; j < cols; ++j) {
        double v = load_elem(x, dtype, start + j);
        if (isnan(v))
            return NAN;
        if (v > m)
            m = v;
    }
    if (m == -INFINITY)
        return -INFINITY;
    if (m == INFINITY)
        return INFINITY;

    /* Second pass: sum of exp(x_j - m); a -inf entry contributes exp(-inf) = 0. */
    for (j = 0; j < cols; ++j)
        s += exp(load_elem(x, dtype, start + j) - m);

    return m + log(s);
}

/* The log-probability of column t of one row: the element minus the row's LSE. */
static double token_logprob_one_row(const void *x, int dtype, int64_t start, int64_t cols,
                                    int64_t t)
{
    if (t < 0 || t >= cols)
        return NAN;
    return load_elem(x, dtype, start + t) - lse_one_row(x, dtype, start, cols);
}

/* One row of the backward pass: grad_out * exp(x_j - lse) for every j. */
static void softmax_grad_one_row(const void *x, int dtype, int64_t start, int64_t cols,
                                 double lse, double grad_out, double *out)
{
    int64_t j;
    for (j = 0; j < cols; ++j)
        out[j] = grad_out * exp(load_elem(x, dtype, start + j) - lse);
}

/* One row of the token log-probability's backward pass:
 * g * ([j == t] - exp(x_j - lse)); a row of NaN when t is outside [0, cols). */
static void token_grad_one_row(const void *x, int dtype, int64_t start, int64_t cols, int64_t t,
                               double lse, double g, double *out)
{
    const int valid = t >= 0 && t < cols;
    int64_t k;
    for (k = 0; k < cols; ++k) {
        const double p = exp(load_elem(x, dtype, start + k) - lse);   /* softmax_k */
        out[k] = valid ? g * ((k == t ? 1.0 : 0.0) - p) : NAN;
    }
}

struct job {
    const void *x;
    int dtype;
    int64_t row_begin, row_end, cols, row_stride;
    const int64_t *targets;  /* NULL: LSE; else the target column of each row */
    const float *lse, *grad_out;  /* non-NULL: the backward pass, out holds rows x cols */
    double *out;
};

static void *run_rows(void *arg)
{
    const struct job *jb = (const struct job *)arg;
    int64_t r;
    for (r = jb->row_begin; r < jb->row_end; ++r) {
        if (jb->lse != NULL && jb->targets != NULL)
            token_grad_one_row(jb->x, jb->dtype, r * jb->row_stride, jb->cols, jb->targets[r],
                               jb->lse[r], jb->grad_out[r], &jb->out[r * jb->cols]);
        else if (jb->lse != NULL)
            softmax_grad_one_row(jb->x, jb->dtype, r * jb->row_stride, jb->cols,
                                 (double)jb->lse[r], (double)jb->grad_out[r],
                                 jb->out + r * jb->cols);
        else if (jb->targets == NULL)
            jb->out[r] = lse_one_row(jb->x, jb->dtype, r * jb->row_stride, jb->cols);
        else
            jb->out[r] = token_logprob_one_row(jb->x, jb->dtype, r * jb->row_stride, jb->cols,
                                               jb->targets[r]);
    }
    return NULL;
}

#define ORACLE_MAX_THREADS 256

static int run_all(const void *x, int dtype, int64_t rows, int64_t cols, int64_t row_stride,
                   const int64_t *targets, const float *lse, const float *grad_out,
                   double *out, int nthreads)
{
    pthread_t tid[ORACLE_MAX_THREADS];
    struct job jobs[ORACLE_MAX_THREADS];
    int64_t per;
    int t, started = 0;

    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F16)
        return -1;
    if (rows < 0 || cols < 0 || (rows > 1 && row_stride < cols))
        return -1;
    if (rows == 0)
        return 0;
    if (out == NULL || (cols > 0 && x == NULL))
        return -1;

    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > ORACLE_MAX_THREADS)
        nthreads = ORACLE_MAX_THREADS;
    if ((int64_t)nthreads > rows)
        nthreads = (int)rows;

    per = (rows + nthreads - 1) / nthreads;
    for (t = 0; t < nthreads; ++t) {
        jobs[t].x = x;
        jobs[t].dtype = dtype;
        jobs[t].row_begin = (int64_t)t * per;
        jobs[t].row_end = jobs[t].row_begin + per < rows ? jobs[t].row_begin + per : rows;
        jobs[t].cols = cols;
        jobs[t].row_stride = row_stride;
        jobs[t].targets = targets;
        jobs[t].lse = lse;
        jobs[t].grad_out = grad_out;
        jobs[t].out = out;
    }
    if (nthreads == 1) {
        run_rows(&jobs[0]);
        return 0;
    }
    for (t = 0; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, run_rows, &jobs[t]) != 0)
            break;
        ++started;
    }
    for (t = started; t < nthreads; ++t)   /* thread creation failed: finish here */
        run_rows(&jobs[t]);
    for (t = 0; t < started; ++t)
        pthread_join(tid[t], NULL);
    return 0;
}

/*
 * out[r] = LSE of row r, r in [0, rows). `x` is a host pointer to the first
 * element; row r starts `r * row_stride` elements after it. Returns 0, or -1
 * for an invalid argument (unknown dtype, negative size, row_stride < cols
 * with more than one row, null pointer with work to do).
 */
int lse_oracle_f64(const void *x, int dtype, int64_t rows, int64_t cols,
                   int64_t row_stride, double *out, int nthreads)
{
    return run_all(x, dtype, rows, cols, row_stride, NULL, NULL, NULL, out, nthreads);
}

/*
 * out[r] = x[r, t] - LSE of row r with t = targets[r] (NaN when t is outside
 * [0, cols)), r in [0, rows). Arguments as lse_oracle_f64; `targets` is a
 * host pointer to rows int64 values and must not be null when rows > 0.
 */
int lse_oracle_token_logprob_f64(const void *x, int dtype, int64_t rows, int64_t cols,
                                 int64_t row_stride, const int64_t *targets, double *out,
                                 int nthreads)
{
    if (rows > 0 && targets == NULL)
        return -1;
    return run_all(x, dtype, rows, cols, row_stride, targets, NULL, NULL, out, nthreads);
}

/*
 * out[r * cols + j] = grad_out[r] * exp(x[r, j] - lse[r]) for r in [0, rows),
 * j in [0, cols). Arguments as lse_oracle_f64; `lse` and `grad_out` are host
 * pointers to rows fp32 values and must not be null when rows > 0.
 */
int lse_oracle_softmax_grad_f64(const void *x, int dtype, int64_t rows, int64_t cols,
                                int64_t row_stride, const float *lse, const float *grad_out,
                                double *out, int nthreads)
{
    if (rows > 0 && (lse == NULL || grad_out == NULL))
        return -1;
    return run_all(x, dtype, rows, cols, row_stride, NULL, lse, grad_out, out, nthreads);
}

/*
 * out[r * cols + j] = grad_logp[r] * ([j == t] - exp(x[r, j] - lse[r])) with
 * t = targets[r], for r in [0, rows), j in [0, cols); a row of NaN when t is
 * outside [0, cols). Arguments as lse_oracle_f64; `targets`, `lse` and
 * `grad_logp` are host pointers to rows values and must not be null when
 * rows > 0.
 */
int lse_oracle_token_logprob_grad_f64(const void *x, int dtype, int64_t rows, int64_t cols,
                                      int64_t row_stride, const int64_t *targets,
                                      const float *lse, const float *grad_logp, double *out,
                                      int nthreads)
{
    if (rows > 0 && (targets == NULL || lse == NULL || grad_logp == NULL))
        return -1;
    return run_all(x, dtype, rows, cols, row_stride, targets, lse, grad_logp, out, nthreads);
}
