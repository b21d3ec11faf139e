// lse_launch.h - the interface between the host planner (lse_api.cpp) and the
// kernel dispatch (lse_kernels.hip, lse_backward.hip, lse_dim.hip, lse_noalloc.hip).
// Host-only types; no device code.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "lse.h"

namespace lse {

enum : int { kSchedRowsPerWave = 1, kSchedRowPerWG = 2, kSchedSplitRow = 3 };

// Arrival counters (split rows, split dim tiles) sit kCounterWords words, 256
// bytes, apart. Agent-scope atomics that share a cache line are serialised:
// measured on MI355X, 1024 workgroups adding to 16 counters took 13.8 us with
// the counters in one line and 3.0 us with each in its own.
constexpr int kCounterWords = 64;

// Bound on the merging part's reads of one split-row slot (each a memory
// round trip); a pair is expected within the first few.
constexpr int kSplitSpinLimit = 1 << 16;

struct LaunchArgs {
    // what to run
    int schedule;
    int dtype;             // an lse_dtype_t
    int block;
    int64_t grid;
    bool vector_loads;
    int lanes_per_row;
    int loads_per_lane;
    int rows_per_wave;
    int parts;
    int unroll;
    // operands
    const char* x;
    int64_t rows;
    int64_t cols;
    int64_t stride_bytes;
    float* out;          // LSE per row; may be NULL when targets is set
    const int64_t* targets;  // token log-probabilities: target column per row (NULL: LSE only)
    float* logp;         // x[r, targets[r]] - LSE per row (with targets)
    unsigned* ws_pairs;  // split-row (max, sum) pairs, 2 words each, zero between calls
    unsigned* counters;  // split-row arrival counters, one per row (kCounterWords apart), zero between calls
    hipStream_t stream;
};

// Launches the kernel the plan names; returns hipGetLastError() after it.
hipError_t launch(const LaunchArgs& a);

// What a forward call needs besides its operands: the device, its CU count,
// the schedule and tuning overrides (0 = the planner's choice), and the split
// schedule's workspace with its capacity (pairs of 8 bytes; counters
// kCounterWords words apart; both zero between calls). A handle provides them, or
// the no-allocation entry point its per-device scratch.
struct ForwardContext {
    int device;
    int n_cu;
    int schedule;
    int block, unroll, parts, waves_per_cu, lanes_per_row;
    unsigned* ws_pairs;
    unsigned* counters;
    int64_t pair_capacity;
    int64_t counter_capacity;
};

// Argument checks shared by the forward entry points (no HIP call).
lse_status_t check_forward(const void* x, lse_dtype_t dtype, int64_t rows, int64_t cols,
                           int64_t row_stride, const float* out);

// Plan and launch one forward call on `stream` (lse_api.cpp).
lse_status_t run_forward(const ForwardContext& c, const void* x, lse_dtype_t dtype, int64_t rows,
                         int64_t cols, int64_t row_stride, float* out, const int64_t* targets,
                         float* logp, hipStream_t stream);

// The no-allocation entry point's per-device scratch (lse_noalloc.hip): look
// up the current device's copy (once) and clear its pairs and arrival
// counters on `stream` unless a launch already did. ptr and n_cu may be NULL.
lse_status_t noalloc_prepare(int device, hipStream_t stream, unsigned char** ptr, int* n_cu);

// The backward pass, grad_x = grad_out * exp(x - lse) (lse_backward.hip).
struct GradArgs {
    int dtype;             // an lse_dtype_t
    bool vector_units;     // 16-byte units (rows 16-byte aligned, or peel below)
    bool peel;             // each row's units start at its first 16-byte boundary
    int64_t grid;
    int64_t rows_per_wg;   // 1: a workgroup takes one chunk of one row
    int64_t chunks_per_row;
    int64_t chunk_units;   // units per chunk (rows_per_wg == 1)
    const char* x;
    int64_t rows, cols;
    int64_t xs_bytes, gs_bytes;  // bytes between row starts of x and of grad_x
    const float* lse;
    const float* grad_out;
    const int64_t* targets;  // non-NULL: the token log-probability's backward
    char* grad_x;
    hipStream_t stream;
};

hipError_t launch_grad(const GradArgs& a);

// LSE over the middle axis of [outer, n, inner] (lse_dim.hip): one launch
// covers tiles [tile0, tile0 + grid / parts) of gw column groups each; with
// parts > 1 the last workgroup of each tile to arrive merges the parts' pairs
// from ws_pairs in the same launch.
struct DimArgs {
    int dtype;             // an lse_dtype_t
    bool vector_cols;      // 16-byte groups of columns (inner % K == 0, x 16-byte aligned)
    int64_t grid;
    int parts;             // workgroups per tile along the reduced axis (<= 1024)
    int gw;                // column groups per tile (<= 256; 256 / gw steps of j per load)
    const char* x;
    int64_t n, inner;
    int64_t ncv;           // column groups in all (outer * inner / K)
    int64_t tile0;
    float* out;
    unsigned* ws_pairs;    // tiles * gw * K * parts (max, sum) pairs of one launch
    unsigned* counters;    // one arrival counter per tile of a launch (kCounterWords apart),
                           // zero between calls
    bool xcd_runs;         // give each XCD a contiguous run of workgroups (see lse_cols)
    hipStream_t stream;
};

hipError_t launch_cols(const DimArgs& a);

// The backward pass over the middle axis (lse_dim.hip): the same tiles as
// DimArgs, parts along n independent (nothing to merge).
struct DimGradArgs {
    int dtype;             // an lse_dtype_t
    bool vector_cols;      // 16-byte groups of columns (inner % K == 0, x and grad_x 16-byte aligned)
    int64_t grid;
    int parts;             // workgroups per tile along n (<= 65536)
    int gw;                // column groups per tile
    const char* x;
    int64_t n, inner;
    int64_t ncv;           // column groups in all
    int64_t tile0;
    const float* lse;      // [outer, inner] fp32
    const float* grad_out; // [outer, inner] fp32
    char* grad_x;          // x's layout and element type
    bool xcd_runs;
    hipStream_t stream;
};

hipError_t launch_grad_cols(const DimGradArgs& a);

// lse_backward_dim's flat launch: lanes own 16-byte vectors (or single
// elements) of the flat [outer, n, inner] array and look up each element's
// lse and grad_out.
struct DimFlatArgs {
    int dtype;             // an lse_dtype_t
    bool vec;              // x and grad_x share their phase mod 16
    const char* x;
    char* grad_x;
    const float* lse;      // [outer, inner] fp32
    const float* grad_out; // [outer, inner] fp32
    int64_t n, inner;
    int64_t total;         // outer * n * inner elements
    int64_t head;          // elements before x's first 16-byte boundary (0 without vec)
    int64_t nvec;          // whole 16-byte vectors after the head (elements without vec)
    uint64_t m_inner;      // floor((2^64 - 1) / inner) + 1 where inner < 2^32, else 0
    uint64_t m_n;          // the same for n; 0 for n == 1
    hipStream_t stream;
};

hipError_t launch_grad_flat(const DimFlatArgs& a);

}  // namespace lse
