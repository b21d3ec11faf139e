/*
 * lse.h - C ABI of the MI355X (gfx950) row-wise log-sum-exp library.
 *
 * The operation. For a row-major matrix x with `rows` rows of `cols`
 * elements, row r starting `r * row_stride` elements after x, the library
 * writes one fp32 scalar per row,
 *
 *     out[r] = log( sum_j exp(x[r, j]) )        (natural log),
 *
 * the log-sum-exp (LSE) that the paper "Speeding up Log-Sum-Exp: Kernel
 * Fusion at the Memory Wall, Integer Arithmetic at the Compute Wall" defines
 * as its primitive (title, abstract, §1) and reduces over the last axis of a
 * (B, N) tensor (§2.1, Figure 1). As in its single-pass fused kernel
 * (§3.1), every input element is read from device memory once, each lane
 * folds its elements into a running (max, exp-sum) pair, the pairs are
 * merged with the associative, commutative pairwise LSE, and one scalar per
 * row is written. The output is base e, as the paper's integer variant also
 * returns base-e float32 (§3.2). Accumulation is fp32 for both input types.
 *
 * Special values follow torch.logsumexp, which the paper's kernels replace
 * as a drop-in (abstract, §6): a NaN anywhere in a row gives NaN; a row of
 * only -inf, or an empty row (cols == 0), gives -inf; otherwise a +inf in the
 * row gives +inf.
 *
 * Streams and ownership. All device work is enqueued on the caller's
 * `stream` and returns without synchronising. `x` and `out` are device
 * pointers owned by the caller and must stay valid until the stream reaches
 * the call. A handle owns a small device workspace for the split-row
 * schedule; calls that share one handle must not run concurrently (use one
 * handle per stream). The compute entry points allocate nothing, never
 * synchronise and enqueue no memset (the split schedules' pair slots and
 * arrival counters are cleared by the kernels that use them), so they may be
 * captured into a HIP graph and the graph replayed.
 *
 * Errors. Every entry point returns an lse_status_t; nothing aborts. The
 * arguments of lse_forward are checked on the host before any HIP call, in
 * this order: dtype, sizes, pointers and alignment, then the handle.
 */
#ifndef ROW_WISE_LOG_AMD_LSE_H
#define ROW_WISE_LOG_AMD_LSE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lse_handle_s *lse_handle_t;

/* Element type of x. The 16-bit types are decoded exactly to fp32 (bf16's
 * 16 bits become the high half of an fp32 word; every IEEE half value,
 * subnormals included, is an fp32 value) and accumulated in fp32, like fp32
 * input. A 16-bit input halves the bytes read, the lever behind the paper's
 * reduced-bit FuseLSE16 (§4.3, Figure 5); the arithmetic stays fp32. */
typedef enum {
    LSE_DTYPE_F32 = 0,
    LSE_DTYPE_BF16 = 1,
    LSE_DTYPE_F16 = 2
} lse_dtype_t;

typedef enum {
    LSE_OK = 0,
    LSE_ERR_INVALID_ARG = 1,       /* a size, pointer, alignment or handle is invalid */
    LSE_ERR_UNSUPPORTED_DTYPE = 2, /* dtype is not one of lse_dtype_t */
    LSE_ERR_NO_DEVICE = 3,         /* no HIP device, or the device is not gfx950 */
    LSE_ERR_ALLOC = 4,             /* device memory for the workspace could not be allocated */
    LSE_ERR_HIP = 5                /* a HIP runtime call or kernel launch failed */
} lse_status_t;

/* Schedules. AUTO picks by shape; the others force one schedule, which the
 * tests and the benchmark use to compare them. Every schedule computes every
 * shape: ROWS_PER_WAVE holds a row in registers and passes rows longer than
 * it holds (4 KiB when rows are 16-byte aligned, else 1024 elements) to
 * ROW_PER_WG; SPLIT_ROW processes at most LSE_SPLIT_MAX_ROWS rows per launch
 * and issues more launches for more rows; an empty row (cols == 0) needs no
 * loads and always runs as ROWS_PER_WAVE. */
typedef enum {
    LSE_SCHED_AUTO = 0,
    LSE_SCHED_ROWS_PER_WAVE = 1, /* short rows held in registers, 64/G rows per wavefront */
    LSE_SCHED_ROW_PER_WG = 2,    /* one workgroup streams one row */
    LSE_SCHED_SPLIT_ROW = 3      /* S workgroups per row, partial (max, sum) pairs merged by the last */
} lse_schedule_t;

/*
 * Create a handle on HIP device `device` (an index as for hipSetDevice).
 * Queries the compute-unit count, allocates the split-row workspace
 * (LSE_SPLIT_MAX_ROWS * LSE_SPLIT_MAX_PARTS (max, sum) pairs plus one
 * counter per row, each in its own 256 bytes, about 0.75 MiB, all zeroed)
 * and lse_forward_dim's workspace (LSE_DIM_MAX_PAIRS pairs, 32 MiB), and
 * synchronises once. On success *out receives the handle; on failure
 * *out is set to NULL.
 * Errors: INVALID_ARG (out NULL, device out of range), NO_DEVICE (no device
 * or not gfx950), ALLOC, HIP.
 */
lse_status_t lse_create(lse_handle_t *out, int device);

/*
 * out[r] = LSE(x[r, 0:cols]) for r in [0, rows), enqueued on `stream`
 * (NULL means the null stream of the handle's device): the paper's fused
 * single-pass LSE (§3.1) over the last axis (§2.1), special values as above.
 * Accuracy: |out[r] - LSE| <= 2e-6 * max(1, |LSE|) for fp32 input and
 * 1e-5 * max(1, |LSE|) for bf16 and fp16 input, against the exact LSE of the
 * decoded elements; the paper reports FuseLSE's error against FP64 in §4.1.
 *   x          device pointer to element (0, 0); aligned to its element size.
 *   dtype      LSE_DTYPE_F32, LSE_DTYPE_BF16 or LSE_DTYPE_F16.
 *   rows       >= 0; rows == 0 is a no-op (x and out may be NULL).
 *   cols       >= 0, < 2^31; cols == 0 writes -inf to every out[r].
 *   row_stride elements between consecutive row starts; >= cols when
 *              rows > 1 (ignored when rows == 1). Rows may be padded.
 *   out        device pointer to rows fp32 values, 4-byte aligned; must not
 *              overlap x.
 * No allocation, no synchronisation. Only bytes inside the rows
 * [x + r*row_stride, x + r*row_stride + cols) are read.
 * Errors: UNSUPPORTED_DTYPE; INVALID_ARG (negative or too large sizes,
 * row_stride < cols, NULL pointer with work to do, misaligned x or out, NULL
 * handle); HIP (launch failure, from hipGetLastError).
 */
lse_status_t lse_forward(lse_handle_t h, const void *x, lse_dtype_t dtype,
                         int64_t rows, int64_t cols, int64_t row_stride,
                         float *out, hipStream_t stream);

/*
 * Token log-probabilities, fused into the same pass over x: for each row r
 * with t = targets[r],
 *
 *     logp[r] = x[r, t] - LSE(x[r, 0:cols])
 *
 * the log-probability of column t under a softmax over the row. This is the
 * quantity behind the paper's motivating workload (§1, §5.1): per generated
 * token in RLHF training, the log-probability of the sampled token under the
 * model's logits over the vocabulary. The subtraction is one fp32 operation on
 * the decoded element and the fp32 LSE; x is read once, as by lse_forward.
 *   targets    device pointer to rows int64 column indices, 8-byte aligned.
 *              A target outside [0, cols) gives logp[r] = NaN.
 *   logp       device pointer to rows fp32 outputs, 4-byte aligned.
 *   lse_out    optional (NULL allowed) device pointer to rows fp32 values that
 *              receive LSE(x[r, :]) exactly as lse_forward writes them.
 * Other arguments, streams and errors as for lse_forward. IEEE arithmetic
 * gives the special values: a target at -inf gives -inf; a row of only -inf
 * gives NaN (-inf - -inf); a +inf elsewhere in the row gives -inf and a +inf
 * at the target NaN; a NaN in the row gives NaN.
 * Errors: as lse_forward, plus INVALID_ARG for NULL or misaligned targets or
 * logp when rows > 0.
 */
lse_status_t lse_token_logprob(lse_handle_t h, const void *x, lse_dtype_t dtype,
                               int64_t rows, int64_t cols, int64_t row_stride,
                               const int64_t *targets, float *logp, float *lse_out,
                               hipStream_t stream);

/*
 * Backward pass: the gradient of lse[r] = LSE(x[r, :]) with respect to x,
 *
 *     grad_x[r, j] = grad_out[r] * exp(x[r, j] - lse[r]),
 *
 * the row's softmax scaled by the incoming gradient; backward support is
 * one of the properties the paper tabulates for its kernels (Table 3). One
 * streaming pass: x is read once and grad_x written once, in x's element
 * type (bf16 and fp16 results are rounded to nearest even from fp32
 * arithmetic).
 *   x, dtype, rows, cols, row_stride   as for lse_forward.
 *   lse        device pointer to rows fp32 values, normally lse_forward's
 *              output for the same x (any values are accepted: the formula is
 *              applied as written, with IEEE special values).
 *   grad_out   device pointer to rows fp32 incoming gradients.
 *   grad_x     device pointer to rows x cols elements of dtype, row r at
 *              grad_x + r * grad_row_stride elements, aligned to its element
 *              size; must not overlap x, lse or grad_out.
 *   grad_row_stride  >= cols when rows > 1.
 * No allocation, no synchronisation; nothing outside the rows of grad_x is
 * written. Errors: as lse_forward, plus INVALID_ARG for NULL or misaligned
 * lse, grad_out or grad_x, or grad_row_stride < cols.
 */
lse_status_t lse_backward(lse_handle_t h, const void *x, lse_dtype_t dtype,
                          int64_t rows, int64_t cols, int64_t row_stride,
                          const float *lse, const float *grad_out, void *grad_x,
                          int64_t grad_row_stride, hipStream_t stream);

/*
 * Backward pass of the token log-probability: the gradient of
 * logp[r] = x[r, t] - LSE(x[r, :]) (t = targets[r]) with respect to x,
 *
 *     grad_x[r, j] = grad_logp[r] * ([j == t] - exp(x[r, j] - lse[r])),
 *
 * what training back-propagates through the per-token log-probabilities of
 * the paper's motivating workload (§1, §5.1): lse_backward's pass with the
 * incoming gradient negated and grad_logp[r] added at the target column.
 *   x, dtype, rows, cols, row_stride   as for lse_forward.
 *   targets    device pointer to rows int64 column indices, 8-byte aligned; a
 *              target outside [0, cols) (whose logp is NaN) gives a row of NaN.
 *   lse        device pointer to rows fp32 values, normally the forward LSE
 *              (lse_token_logprob's lse_out or lse_forward's output).
 *   grad_logp  device pointer to rows fp32 incoming gradients.
 *   grad_x, grad_row_stride   as for lse_backward.
 * One streaming pass, x read once and grad_x written once, in x's element type.
 * No allocation, no synchronisation; nothing outside the rows of grad_x is
 * written. Errors: as lse_backward, plus INVALID_ARG for NULL or misaligned
 * targets.
 */
lse_status_t lse_token_logprob_backward(lse_handle_t h, const void *x, lse_dtype_t dtype,
                                        int64_t rows, int64_t cols, int64_t row_stride,
                                        const int64_t *targets, const float *lse,
                                        const float *grad_logp, void *grad_x,
                                        int64_t grad_row_stride, hipStream_t stream);

/*
 * LSE over the middle axis of a contiguous [outer, n, inner] array:
 *
 *     out[o * inner + i] = log( sum_{j < n} exp(x[(o * n + j) * inner + i]) ),
 *
 * which is torch.logsumexp(x, dim=d) for a contiguous x, with outer the
 * product of the sizes before d, n the size of d and inner the product of
 * the sizes after it; the paper offers its kernels as drop-in replacements
 * for torch.logsumexp (abstract, §6). inner == 1 is lse_forward over rows of
 * n. Same accuracy, special values and stream semantics as lse_forward.
 *   x      device pointer, aligned to its element size.
 *   outer, n, inner  >= 0; n < 2^31; outer * inner < 2^40 and the element
 *          count must fit in int64.
 *   out    device pointer to outer * inner fp32 values, 4-byte aligned, not
 *          overlapping x. n == 0 writes -inf.
 * When there are too few outputs to fill the GPU, several workgroups share
 * each output's n and meet through the handle's workspace and arrival
 * counters (so, like lse_forward, calls sharing a handle must not run
 * concurrently).
 * Errors: UNSUPPORTED_DTYPE; INVALID_ARG (sizes, NULL or misaligned
 * pointers with work to do, NULL handle); HIP.
 */
lse_status_t lse_forward_dim(lse_handle_t h, const void *x, lse_dtype_t dtype,
                             int64_t outer, int64_t n, int64_t inner, float *out,
                             hipStream_t stream);

/*
 * The backward pass of lse_forward_dim over the middle axis of a contiguous
 * [outer, n, inner] array:
 *
 *     grad_x[(o*n + j)*inner + i] = grad_out[o*inner + i]
 *                                   * exp(x[(o*n + j)*inner + i] - lse[o*inner + i]),
 *
 * the gradient of out = LSE over j with respect to x (along j, each column's
 * softmax scaled by its incoming gradient): the backward support the paper
 * lists for its kernels (Table 3), for the torch.logsumexp drop-in (abstract,
 * §6) over any axis. lse_backward is the last-axis case (inner == 1 calls it).
 *   x, dtype, outer, n, inner   as for lse_forward_dim.
 *   lse        device pointer to outer * inner fp32 values, normally
 *              lse_forward_dim's output; 4-byte aligned.
 *   grad_out   device pointer to outer * inner fp32 incoming gradients,
 *              4-byte aligned.
 *   grad_x     device pointer to an array of x's layout and element type
 *              (16-bit results rounded to nearest even), aligned to its
 *              element size; must not overlap x, lse or grad_out.
 * As in lse_backward, the formula is applied as written in fp32 arithmetic
 * (any lse is accepted; IEEE special values). One streaming pass: x read
 * once, grad_x written once, nothing else written; lse and grad_out are read
 * once per column tile, or, on the flat schedule (which the planner takes for
 * widths or bases that do not fit 16-byte column groups, and, while lse and
 * grad_out total at most 16 MiB, for fp32 and for 16-bit rows whose pitch is
 * not a multiple of 128 bytes), once per element from the caches; no
 * workspace, no allocation, no synchronisation. The results do not depend on
 * the schedule.
 * Errors: UNSUPPORTED_DTYPE; INVALID_ARG (sizes, NULL or misaligned pointers
 * with work to do, NULL handle); HIP.
 */
lse_status_t lse_backward_dim(lse_handle_t h, const void *x, lse_dtype_t dtype,
                              int64_t outer, int64_t n, int64_t inner, const float *lse,
                              const float *grad_out, void *grad_x, hipStream_t stream);

/*
 * lse_forward without a handle and without allocating, for callers that
 * cannot call hipMalloc: code under HIP graph capture, tight serving loops,
 * harnesses that forbid device allocation. Same operation, arguments (minus
 * the handle), accuracy, special values and stream semantics as lse_forward,
 * on the current device (`stream` must belong to it), with the planner's
 * automatic schedule (lse_set_schedule / lse_set_tuning do not apply).
 *
 * Scratch. The split-row schedule's (max, sum) pairs and arrival counters
 * live in a fixed device array of 768 KiB that each GPU the library runs on
 * holds until the process ends (room for LSE_SPLIT_MAX_ROWS rows of
 * LSE_SPLIT_MAX_PARTS pairs per launch; longer inputs go in several launches,
 * so every shape fits, and a plan that did not would be rejected with
 * INVALID_ARG before any launch). The first call on a device looks the array
 * up and enqueues one small kernel on `stream` that zeroes it (again
 * on later calls while that kernel was only captured, not run); lse_create on
 * a device does the same set-up. Every call on a GPU shares that GPU's
 * scratch: calls that overlap on one GPU (other streams, threads or graph
 * replays running at the same time) race and give wrong results.
 * No hipMalloc, hipFree or allocating library call; no synchronisation.
 * Errors: as lse_forward (no handle error); NO_DEVICE (no current device, or
 * not gfx950); HIP.
 */
lse_status_t lse_forward_noalloc(const void *x, lse_dtype_t dtype, int64_t rows, int64_t cols,
                                 int64_t row_stride, float *out, hipStream_t stream);

/* Release the handle and its workspace. NULL is allowed and returns LSE_OK.
 * The caller must ensure no work using the handle is still pending. */
lse_status_t lse_destroy(lse_handle_t h);

/* A static, human-readable name for a status code. */
const char *lse_status_string(lse_status_t s);

/* Force a schedule for later lse_forward calls on this handle (AUTO resets).
 * Errors: INVALID_ARG (NULL handle or unknown schedule). */
lse_status_t lse_set_schedule(lse_handle_t h, lse_schedule_t s);

/* Tuning overrides, for measurement. Streaming schedules: threads per
 * workgroup `block` (64, 128, 256, 512 or 1024), 16-byte loads per lane per
 * batch `unroll` (4 or 8), SPLIT_ROW workgroups per row `parts` (1..64;
 * lse_forward uses at most `block` of them, as the last part merges the
 * pairs one per thread; lse_forward_dim takes it as its workgroups per tile
 * along n, and lse_backward_dim as well, where it also selects the column
 * tiles over the flat schedule).
 * ROWS_PER_WAVE: at most `waves_per_cu` wavefronts per compute unit in the
 * grid (1..1024; the wavefronts loop over the rest) and `lanes_per_row` lanes
 * sharing a row (a power of two up to 64; ignored where no kernel instance
 * fits the shape). 0 restores the planner's choice.
 * Errors: INVALID_ARG (NULL handle or a value outside those sets). */
lse_status_t lse_set_tuning(lse_handle_t h, int32_t block, int32_t unroll, int32_t parts,
                            int32_t waves_per_cu, int32_t lanes_per_row);

/* Launch plan chosen for one call: which kernel runs, with what grid. */
typedef struct {
    int32_t schedule;        /* an lse_schedule_t other than AUTO; 0 when rows == 0 */
    int32_t block;           /* threads per workgroup */
    int64_t grid;            /* workgroups launched */
    int32_t vector_loads;    /* 1: 16-byte loads, 0: one element per load */
    int32_t lanes_per_row;   /* ROWS_PER_WAVE: lanes G sharing one row */
    int32_t loads_per_lane;  /* ROWS_PER_WAVE: loads each lane holds for a row */
    int32_t rows_per_wave;   /* ROWS_PER_WAVE: rows a wavefront holds at once */
    int32_t parts;           /* SPLIT_ROW: workgroups per row (1 otherwise) */
    int32_t unroll;          /* ROW_PER_WG / SPLIT_ROW: 16-byte loads per lane per batch */
    int64_t workspace_bytes; /* SPLIT_ROW: workspace bytes the call uses */
} lse_plan_t;

/* Capacity of a handle's split-row workspace. */
#define LSE_SPLIT_MAX_ROWS 1024
#define LSE_SPLIT_MAX_PARTS 64
/* Capacity, in (max, sum) pairs (8 bytes each, 32 MiB), of a handle's
 * workspace for lse_forward_dim's split of the reduced axis. */
#define LSE_DIM_MAX_PAIRS (1 << 22)

/*
 * The launch plan lse_forward would use, computed on the host with no HIP
 * call: for tests and profiling. `x_addr` is the device address of x (only
 * its alignment matters), `n_cu` the compute-unit count, `schedule` an
 * lse_schedule_t (AUTO for the shape-based choice). Arguments are checked as
 * in lse_forward, minus the handle and the pointers' nullness.
 * Errors: UNSUPPORTED_DTYPE, INVALID_ARG (also plan NULL or n_cu < 1).
 */
lse_status_t lse_plan(lse_dtype_t dtype, int64_t rows, int64_t cols, int64_t row_stride,
                      uint64_t x_addr, int32_t n_cu, lse_schedule_t schedule,
                      lse_plan_t *plan);

#ifdef __cplusplus
}
#endif

#endif /* ROW_WISE_LOG_AMD_LSE_H */
