// lse_api.cpp - the C ABI declared in include/lse.h: argument checks, the
// shape-based launch planner, the handle and its split-row workspace.
//
// The planner is a pure host function (lse_plan) so that its choices can be
// tested without a GPU. lse_forward checks its arguments, plans, and launches
// on the caller's stream; it never allocates and never synchronises.
#include "lse.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>

#include "lse_launch.h"

struct lse_handle_s {
    int device;
    int n_cu;
    unsigned* ws_pairs;  // LSE_SPLIT_MAX_ROWS * LSE_SPLIT_MAX_PARTS (max, sum) pairs, zero between calls
    unsigned* counters;  // LSE_SPLIT_MAX_ROWS arrival counters, 256 bytes apart, zero between calls
    unsigned* dim_pairs; // LSE_DIM_MAX_PAIRS (max, sum) pairs for lse_forward_dim's split
    int schedule;        // lse_schedule_t forced for later calls (AUTO = by shape)
    int block, unroll, parts, waves_per_cu, lanes_per_row;  // tuning overrides, 0 = planner default
};

namespace {

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;
constexpr int kRegsMaxVecUnits = 256;  // schedule A: rows of up to 4 KiB in 16-byte loads...
constexpr int kRegsMaxElems = 1024;    // ...or up to 1024 single elements (unaligned rows)
// Schedule A grid cap, in wavefronts per CU (each wavefront loops over the
// rest): 8 when a row needs at most 4 lanes (cheap group reductions), else 16.
// Measured on rows of 16 to 2048 elements, both beat 32 and 64 per CU, and 8
// loses where the 64-lane reductions need more wavefronts to hide them.
constexpr int kWavesPerCUNarrow = 8;
constexpr int kWavesPerCUWide = 16;
// Few long rows (LSE_SCHED_SPLIT_ROW). Rows longer than 64 KiB are split
// when there are at most half as many of them as CUs (fewer than 3/8 for rows
// under 256 KiB), so that each row's share of the budget below is at least
// the 8 wavefronts of a 512-thread workgroup; with more rows one 512-thread
// workgroup per row streams faster (measured at steady state: 150 rows of
// 256 KiB and 1 MiB, 9.4 and 27.2 us against 11.7 and 34.8 us split), as it
// does for rows of up to 64 KiB at any count. A split row gets the
// wavefronts that give each lane one batch of four 16-byte loads, at most its
// share of 4 wavefronts per CU (rounded up): many small workgroups for short inputs
// (launch-latency bound), about 4 wavefronts per CU once the input is large.
// At steady state it beats the previous rule (512-thread parts of ~128 KiB)
// by 1.17x on random shapes, up to 1.8x on small inputs, and loses 5-9 % on
// some inputs of 200 MB and more with 129 to 223 rows.
constexpr int64_t kSplitMinRowBytes = 64 << 10;
constexpr int kSplitWavesPerCU = 4;
// Just over one row per CU (up to 5/4), one workgroup per row leaves most CUs
// one row and some two; rows of 1 MiB and more then split into four parts of
// 256 threads. Measured at steady state with bench.py --ab (257 to 320 rows of
// 1 and 4 MiB, bf16 and fp32): 5-15 % faster than one 256-thread workgroup
// per row, 10-23 % faster than 512 threads; rows of 256 KiB split the same
// way gain nothing or are 2 % slower, so they are not split.
constexpr int64_t kSplitQuarterRowBytes = 1 << 20;
// lse_forward_dim: column groups per workgroup (the other 256 / 32 = 8 lanes
// of each column group take consecutive j), doubled where there are columns
// enough for two 64-group tiles per CU. Measured on [n, inner] of
// [512, 128256] bf16, [4096, 262144] bf16, [65536, 4096] fp32 and
// [16777216, 16] fp32 against 4 to 256 groups and 1 to 1024 parts, the
// fastest plans keep one or two workgroups per CU, each streaming a long
// stretch of j, and split j only when the tiles alone do not reach every CU.
constexpr int kDimGroups = 32;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool valid_dtype(lse_dtype_t d) {
    return d == LSE_DTYPE_F32 || d == LSE_DTYPE_BF16 || d == LSE_DTYPE_F16;
}

int elem_bytes(lse_dtype_t d) { return d == LSE_DTYPE_F32 ? 4 : 2; }

int pow2_at_least(int64_t v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

struct Tuning {
    int block, unroll, parts, waves_per_cu, lanes_per_row;
};

// Register-rows instances (lse_kernels.hip): VPL 1, 2, 4 for G in {1, 2, 4,
// 64}; VPL 1 for G in {8, 16, 32}; scalar rows also VPL 8, 16 for G = 64.
bool regs_instance(int g, int vpl, bool vec) {
    if (vpl == 1) return true;
    if (vpl == 2 || vpl == 4) return g <= 4 || g == 64;
    return !vec && g == 64 && (vpl == 8 || vpl == 16);
}

lse_status_t check_sizes(lse_dtype_t dtype, int64_t rows, int64_t cols, int64_t row_stride,
                         uint64_t x_addr) {
    if (!valid_dtype(dtype)) return LSE_ERR_UNSUPPORTED_DTYPE;
    if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim) return LSE_ERR_INVALID_ARG;
    if (rows > 1 && (row_stride < cols || row_stride > (INT64_MAX / 4) / rows))
        return LSE_ERR_INVALID_ARG;
    const int esize = elem_bytes(dtype);
    if (rows > 0 && cols > 0 && x_addr % esize != 0) return LSE_ERR_INVALID_ARG;
    return LSE_OK;
}

lse_status_t make_plan(lse_dtype_t dtype, int64_t rows, int64_t cols, int64_t row_stride,
                       uint64_t x_addr, int n_cu, int schedule, Tuning tune, lse_plan_t* p) {
    std::memset(p, 0, sizeof(*p));
    if (rows == 0) return LSE_OK;

    const int esize = elem_bytes(dtype);
    const int k = 16 / esize;
    const int64_t stride_bytes = (rows > 1 ? row_stride : cols) * esize;
    const bool aligned16 = x_addr % 16 == 0 && (rows == 1 || stride_bytes % 16 == 0);
    const int64_t vec_units = cols / k;
    const int64_t vec_tail = cols - vec_units * k;
    const bool regs_vec = aligned16 && vec_units >= 1 && vec_units <= kRegsMaxVecUnits;
    const bool regs_scalar = cols <= kRegsMaxElems;

    int sched = schedule;
    bool quarters = false;  // the automatic split of just over one long row per CU
    if (sched == LSE_SCHED_AUTO) {
        const int64_t row_bytes = cols * esize;
        if (regs_vec || (regs_scalar && (!aligned16 || vec_units == 0))) {
            sched = LSE_SCHED_ROWS_PER_WAVE;
        } else if (row_bytes > kSplitMinRowBytes &&
                   (row_bytes >= 4 * kSplitMinRowBytes ? rows * 2 <= n_cu
                                                       : rows * 8 < 3 * int64_t{n_cu})) {
            sched = LSE_SCHED_SPLIT_ROW;  // few long rows: one workgroup per row would idle CUs
        } else if (row_bytes >= kSplitQuarterRowBytes && rows > n_cu &&
                   rows * 4 <= 5 * int64_t{n_cu}) {
            sched = LSE_SCHED_SPLIT_ROW;  // just over one row per CU: quarters even the CUs out
            quarters = true;
        } else {
            sched = LSE_SCHED_ROW_PER_WG;
        }
    }
    // Rows longer than registers hold go to the streaming schedule.
    if (sched == LSE_SCHED_ROWS_PER_WAVE && !regs_vec && !regs_scalar) sched = LSE_SCHED_ROW_PER_WG;
    if (sched != LSE_SCHED_ROWS_PER_WAVE && cols == 0) sched = LSE_SCHED_ROWS_PER_WAVE;  // no loads

    p->schedule = sched;
    if (sched == LSE_SCHED_ROWS_PER_WAVE) {
        const bool vec = regs_vec;
        const int64_t units = vec ? vec_units : cols;
        const int64_t tail = vec ? vec_tail : 0;
        // G lanes cover the row's units (every tail element needs its own lane:
        // G >= tail); VPL loads per lane cover the rest.
        int g = pow2_at_least(std::max<int64_t>({units, tail, 1}));
        if (g > 64) g = 64;
        int vpl = pow2_at_least(ceil_div(units > 0 ? units : 1, g));
        if (tune.lanes_per_row) {
            const int tg = tune.lanes_per_row;
            const int tv = pow2_at_least(ceil_div(units > 0 ? units : 1, tg));
            if (tg >= tail && regs_instance(tg, tv, vec)) {
                g = tg;
                vpl = tv;
            }
        }
        const int rounds = vpl == 1 ? 4 : (vpl == 2 ? 2 : 1);
        p->block = 256;
        p->vector_loads = vec ? 1 : 0;
        p->lanes_per_row = g;
        p->loads_per_lane = vpl;
        p->rows_per_wave = (64 / g) * rounds;
        const int64_t iters = ceil_div(rows, p->rows_per_wave);
        int64_t waves = iters;
        const int wpc = tune.waves_per_cu ? tune.waves_per_cu
                                          : (g <= 4 ? kWavesPerCUNarrow : kWavesPerCUWide);
        const int64_t cap = static_cast<int64_t>(n_cu) * wpc;
        if (waves > cap) waves = cap;
        p->grid = ceil_div(waves, 4);
        p->parts = 1;
        return LSE_OK;
    }

    const int64_t nvec = cols / k;  // 16-byte vectors in a row (one fewer if unaligned)
    p->vector_loads = 1;
    if (sched == LSE_SCHED_ROW_PER_WG) {
        // About 32 fp32 or 64 bf16 elements per lane (one or two batches of
        // four 16-byte loads), 64 to 256 threads. Up to two rows per CU: 512
        // threads, except from 7/8 to 15/8 rows per CU, where some CUs hold
        // two rows and others one and 256 threads stream 5-16 % faster
        // (measured at steady state on 224 to 448 rows of 256 KiB and 1 MiB;
        // at 160 and 200 rows 512 threads are 9-12 % faster, from 480 rows to
        // twice the CUs the two agree). From 15/8 rows per CU, rows of up to
        // 100 KiB also take 256 threads, so that each lane keeps several
        // batches: measured on 480 and 512 rows, 3-4 % faster at 64 and 98
        // KiB (bf16 [512, 50257]: 11.47 -> 11.04 us), while at 128 KiB 512
        // threads were 3-5 % faster and from 160 KiB the two agree within 2 %.
        int block = 256;
        const int64_t cu = n_cu;
        if (rows <= 2 * cu) {
            const bool band = rows * 8 >= 7 * cu && rows * 8 < 15 * cu;
            const bool short_rows = rows * 8 >= 15 * cu && cols * esize <= (100 << 10);
            block = band || short_rows ? 256 : 512;
        } else {
            const int64_t per = nvec / (16 / esize);
            block = 64;
            while (block < 256 && 2 * block <= per) block *= 2;
        }
        p->block = tune.block ? tune.block : block;
        p->unroll = tune.unroll ? tune.unroll : 4;
        p->parts = 1;
        p->grid = rows;
        return LSE_OK;
    }
    // LSE_SCHED_SPLIT_ROW: w wavefronts per row, the fewer of those that give
    // each lane one batch (4 vectors) and the row's share of kSplitWavesPerCU
    // per CU (rounded up to a power of two), at least 2; as up to
    // LSE_SPLIT_MAX_PARTS parts of 64 threads, then wider workgroups (at most
    // 512 threads). The last part to finish merges the row's pairs one per
    // thread, so parts never exceed the block.
    const int64_t r = rows < LSE_SPLIT_MAX_ROWS ? rows : LSE_SPLIT_MAX_ROWS;
    const int64_t w_one = pow2_at_least(ceil_div(nvec > 0 ? nvec : 1, 4 * 64));
    // the share rounds up: rounded down, 40 or 75 rows got only 2.3-2.6
    // wavefronts per CU and ran 22 % slower than with 32 and 16 parts
    const int64_t w_share = pow2_at_least(ceil_div(kSplitWavesPerCU * int64_t{n_cu}, r));
    const int64_t w = std::max<int64_t>(2, std::min(w_one, w_share));
    int64_t parts = std::min<int64_t>(w, LSE_SPLIT_MAX_PARTS);
    int64_t wide = std::min<int64_t>(512, 64 * (w / parts));
    if (quarters) {  // chosen above for rows of 1 MiB and more, n_cu < rows <= 5/4 n_cu
        parts = 4;
        wide = 256;
    }
    p->block = tune.block ? tune.block : static_cast<int32_t>(wide);
    p->unroll = tune.unroll ? tune.unroll : 4;
    if (tune.parts) parts = tune.parts;
    if (parts > LSE_SPLIT_MAX_PARTS) parts = LSE_SPLIT_MAX_PARTS;
    if (parts > p->block) parts = p->block;
    p->parts = static_cast<int32_t>(parts);
    const int64_t batch_rows = rows < LSE_SPLIT_MAX_ROWS ? rows : LSE_SPLIT_MAX_ROWS;
    p->grid = batch_rows * parts;  // per launch; rows beyond LSE_SPLIT_MAX_ROWS take more launches
    p->workspace_bytes = batch_rows * parts * 8 + batch_rows * 4;
    return LSE_OK;
}

// The backward pass's work split: units are 16-byte vectors when every row
// of x and grad_x starts 16-byte aligned; when the rows are not aligned but
// x and grad_x have the same phase mod 16 (same address and same row stride
// mod 16, as contiguous rows of an odd width have), units are 16-byte vectors
// from each row's first 16-byte boundary, (cols - K + 1) / K of them per row,
// with the head and tail elements done singly; else single elements. Rows of at
// least one batch (256 lanes x 4 units) are cut into chunks of 1 to 4
// batches, sized so the grid has about 4 workgroups per CU; shorter rows are
// packed several to a workgroup (up to 4 batches of units). A block's byte
// span stays below 2^30 (its buffer offsets are 32-bit) and its unit count
// below 2^22 (the kernel's float row index is exact there).
lse_status_t make_grad_plan(lse_dtype_t dtype, int64_t rows, int64_t cols, int64_t row_stride,
                            int64_t grad_row_stride, uint64_t x_addr, uint64_t g_addr, int n_cu,
                            lse::GradArgs* a) {
    const int esize = elem_bytes(dtype);
    const int k = 16 / esize;
    const int64_t xs = (rows > 1 ? row_stride : cols) * esize;
    const int64_t gs = (rows > 1 ? grad_row_stride : cols) * esize;
    const bool aligned = cols / k >= 1 && x_addr % 16 == 0 && g_addr % 16 == 0 &&
                         (rows == 1 || (xs % 16 == 0 && gs % 16 == 0));
    const bool peel = !aligned && cols >= 2 * k - 1 && x_addr % 16 == g_addr % 16 &&
                      (rows == 1 || xs % 16 == gs % 16);
    const bool vec = aligned || peel;
    const int64_t units = aligned ? cols / k : peel ? (cols - (k - 1)) / k : cols;
    const int64_t ub = vec ? 16 : esize;
    constexpr int64_t kBatch = 256 * 4;
    a->dtype = dtype;
    a->vector_units = vec;
    a->peel = peel;
    a->rows = rows;
    a->cols = cols;
    a->xs_bytes = xs;
    a->gs_bytes = gs;
    const int64_t target_wgs = 4 * static_cast<int64_t>(n_cu);
    if (units >= kBatch) {
        // Long rows: one batch per workgroup once there are at least 16 per
        // CU (measured on 130 MB to 2 GB inputs, 3-11 % faster than chunks of
        // up to four batches), or at least 4 per CU with rows of four batches
        // and more, whose last, partial chunk wastes little (bf16 [512, 50257]
        // 23.85 -> 20.22 us, [512, 50176] 21.46 -> 18.68 us, fp32 [512, 32000]
        // 25.30 -> 23.48 us; rows of one or two batches lost 2-11 % that way).
        // Smaller inputs keep chunks of one to four batches, about four
        // workgroups per CU.
        int64_t chunk = kBatch;
        if (rows * units < 16 * static_cast<int64_t>(n_cu) * kBatch &&
            (units < 4 * kBatch || rows * units < 4 * static_cast<int64_t>(n_cu) * kBatch)) {
            chunk = ceil_div(ceil_div(rows * units, target_wgs), kBatch) * kBatch;
            chunk = std::min<int64_t>(std::max<int64_t>(chunk, kBatch), 4 * kBatch);
        }
        a->rows_per_wg = 1;
        a->chunk_units = chunk;
        a->chunks_per_row = ceil_div(units, chunk);
        a->grid = rows * a->chunks_per_row;
    } else {
        int64_t r = std::max<int64_t>(1, (4 * kBatch) / units);
        r = std::min<int64_t>(r, std::max<int64_t>(1, ceil_div(rows, target_wgs)));
        const int64_t span = std::max(xs, gs);
        r = std::min<int64_t>(
            r, std::max<int64_t>(1, ((int64_t{1} << 30) - units * ub) / std::max<int64_t>(span, 1)));
        a->rows_per_wg = r;
        a->chunk_units = units;
        a->chunks_per_row = 1;
        a->grid = ceil_div(rows, r);
    }
    return LSE_OK;
}

}  // namespace

extern "C" {

const char* lse_status_string(lse_status_t s) {
    switch (s) {
        case LSE_OK: return "LSE_OK";
        case LSE_ERR_INVALID_ARG: return "LSE_ERR_INVALID_ARG";
        case LSE_ERR_UNSUPPORTED_DTYPE: return "LSE_ERR_UNSUPPORTED_DTYPE";
        case LSE_ERR_NO_DEVICE: return "LSE_ERR_NO_DEVICE";
        case LSE_ERR_ALLOC: return "LSE_ERR_ALLOC";
        case LSE_ERR_HIP: return "LSE_ERR_HIP";
    }
    return "LSE_ERR_UNKNOWN";
}

lse_status_t lse_plan(lse_dtype_t dtype, int64_t rows, int64_t cols, int64_t row_stride,
                      uint64_t x_addr, int32_t n_cu, lse_schedule_t schedule, lse_plan_t* plan) {
    if (plan == nullptr || n_cu < 1) return LSE_ERR_INVALID_ARG;
    lse_status_t st = check_sizes(dtype, rows, cols, row_stride, x_addr);
    if (st != LSE_OK) return st;
    if (schedule < LSE_SCHED_AUTO || schedule > LSE_SCHED_SPLIT_ROW) return LSE_ERR_INVALID_ARG;
    return make_plan(dtype, rows, cols, row_stride, x_addr, n_cu, schedule, Tuning{0, 0, 0, 0, 0}, plan);
}

lse_status_t lse_create(lse_handle_t* out, int device) {
    if (out == nullptr) return LSE_ERR_INVALID_ARG;
    *out = nullptr;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
        (void)hipGetLastError();
        return LSE_ERR_NO_DEVICE;
    }
    if (device < 0 || device >= count) return LSE_ERR_INVALID_ARG;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return LSE_ERR_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return LSE_ERR_NO_DEVICE;

    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) return LSE_ERR_HIP;
    if (hipSetDevice(device) != hipSuccess) return LSE_ERR_HIP;

    lse_handle_s* h = new (std::nothrow) lse_handle_s{};
    lse_status_t st = LSE_OK;
    if (h == nullptr) {
        st = LSE_ERR_ALLOC;
    } else {
        h->device = device;
        h->n_cu = prop.multiProcessorCount;
        const size_t pair_bytes = size_t{LSE_SPLIT_MAX_ROWS} * LSE_SPLIT_MAX_PARTS * 8;
        const size_t count_bytes = size_t{LSE_SPLIT_MAX_ROWS} * lse::kCounterWords * 4;
        const size_t dim_bytes = size_t{LSE_DIM_MAX_PAIRS} * 8;
        void* mem = nullptr;
        if (hipMalloc(&mem, pair_bytes + count_bytes + dim_bytes) != hipSuccess) {
            st = LSE_ERR_ALLOC;
        } else {
            h->ws_pairs = static_cast<unsigned*>(mem);
            h->counters = reinterpret_cast<unsigned*>(static_cast<char*>(mem) + pair_bytes);
            h->dim_pairs = reinterpret_cast<unsigned*>(static_cast<char*>(mem) + pair_bytes +
                                                       count_bytes);
            // The device's scratch for lse_forward_noalloc is set up here too
            // when it can be (its entry point retries and reports otherwise).
            if (lse::noalloc_prepare(device, nullptr, nullptr, nullptr) != LSE_OK)
                (void)hipGetLastError();
            if (hipMemset(h->ws_pairs, 0, pair_bytes + count_bytes) != hipSuccess ||
                hipDeviceSynchronize() != hipSuccess)
                st = LSE_ERR_HIP;
        }
    }
    if (st != LSE_OK && h != nullptr) {
        if (h->ws_pairs) (void)hipFree(h->ws_pairs);
        delete h;
        h = nullptr;
    }
    (void)hipSetDevice(prev);
    *out = h;
    return st;
}

lse_status_t lse_destroy(lse_handle_t h) {
    if (h == nullptr) return LSE_OK;
    lse_status_t st = LSE_OK;
    int prev = 0;
    if (hipGetDevice(&prev) == hipSuccess && hipSetDevice(h->device) == hipSuccess) {
        if (h->ws_pairs && hipFree(h->ws_pairs) != hipSuccess) st = LSE_ERR_HIP;
        (void)hipSetDevice(prev);
    } else {
        st = LSE_ERR_HIP;
    }
    delete h;
    return st;
}

lse_status_t lse_set_schedule(lse_handle_t h, lse_schedule_t s) {
    if (h == nullptr || s < LSE_SCHED_AUTO || s > LSE_SCHED_SPLIT_ROW) return LSE_ERR_INVALID_ARG;
    h->schedule = s;
    return LSE_OK;
}

lse_status_t lse_set_tuning(lse_handle_t h, int32_t block, int32_t unroll, int32_t parts,
                            int32_t waves_per_cu, int32_t lanes_per_row) {
    if (h == nullptr) return LSE_ERR_INVALID_ARG;
    if (block != 0 && block != 64 && block != 128 && block != 256 && block != 512 && block != 1024)
        return LSE_ERR_INVALID_ARG;
    if (unroll != 0 && unroll != 4 && unroll != 8) return LSE_ERR_INVALID_ARG;
    if (parts < 0 || parts > LSE_SPLIT_MAX_PARTS) return LSE_ERR_INVALID_ARG;
    if (waves_per_cu < 0 || waves_per_cu > 1024) return LSE_ERR_INVALID_ARG;
    if (lanes_per_row < 0 || lanes_per_row > 64 || (lanes_per_row & (lanes_per_row - 1)))
        return LSE_ERR_INVALID_ARG;
    h->block = block;
    h->unroll = unroll;
    h->parts = parts;
    h->waves_per_cu = waves_per_cu;
    h->lanes_per_row = lanes_per_row;
    return LSE_OK;
}

}  // extern "C"

namespace lse {

// Plan and launch one forward call (lse_forward, lse_token_logprob and the
// no-allocation entry point); the arguments were checked by the caller. With
// targets set, the kernels also write logp (and write out only if it is not
// NULL).
lse_status_t run_forward(const ForwardContext& c, const void* x, lse_dtype_t dtype, int64_t rows,
                         int64_t cols, int64_t row_stride, float* out, const int64_t* targets,
                         float* logp, hipStream_t stream) {
    lse_plan_t p;
    lse_status_t st = make_plan(dtype, rows, cols, row_stride, reinterpret_cast<uint64_t>(x),
                                c.n_cu, c.schedule,
                                Tuning{c.block, c.unroll, c.parts, c.waves_per_cu, c.lanes_per_row},
                                &p);
    if (st != LSE_OK) return st;
    // The split schedule's pairs and counters of one launch must fit the
    // workspace; launches take at most LSE_SPLIT_MAX_ROWS rows, so a plan
    // never needs more than LSE_SPLIT_MAX_ROWS * LSE_SPLIT_MAX_PARTS pairs and
    // LSE_SPLIT_MAX_ROWS counters.
    if (p.schedule == LSE_SCHED_SPLIT_ROW) {
        const int64_t batch = rows < LSE_SPLIT_MAX_ROWS ? rows : LSE_SPLIT_MAX_ROWS;
        if (batch * p.parts > c.pair_capacity || batch > c.counter_capacity)
            return LSE_ERR_INVALID_ARG;
    }

    const int esize = elem_bytes(dtype);
    LaunchArgs a{};
    a.schedule = p.schedule;
    a.dtype = dtype;
    a.block = p.block;
    a.grid = p.grid;
    a.vector_loads = p.vector_loads != 0;
    a.lanes_per_row = p.lanes_per_row;
    a.loads_per_lane = p.loads_per_lane;
    a.rows_per_wave = p.rows_per_wave;
    a.parts = p.parts;
    a.unroll = p.unroll;
    a.x = static_cast<const char*>(x);
    a.rows = rows;
    a.cols = cols;
    a.stride_bytes = (rows > 1 ? row_stride : cols) * esize;
    a.out = out;
    a.targets = targets;
    a.logp = logp;
    a.ws_pairs = c.ws_pairs;
    a.counters = c.counters;
    a.stream = stream;

    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return LSE_ERR_HIP;
    if (prev != c.device && hipSetDevice(c.device) != hipSuccess) return LSE_ERR_HIP;

    hipError_t err = hipSuccess;
    if (p.schedule == LSE_SCHED_SPLIT_ROW) {
        // The workspace holds LSE_SPLIT_MAX_ROWS rows; larger inputs go in
        // row batches on the same stream (each launch resets its counters).
        for (int64_t r0 = 0; r0 < rows && err == hipSuccess; r0 += LSE_SPLIT_MAX_ROWS) {
            const int64_t n = rows - r0 < LSE_SPLIT_MAX_ROWS ? rows - r0 : LSE_SPLIT_MAX_ROWS;
            LaunchArgs b = a;
            b.x = a.x + r0 * a.stride_bytes;
            b.out = a.out ? a.out + r0 : nullptr;
            b.targets = a.targets ? a.targets + r0 : nullptr;
            b.logp = a.logp ? a.logp + r0 : nullptr;
            b.rows = n;
            b.grid = n * p.parts;
            err = launch(b);
        }
    } else {
        err = launch(a);
    }
    if (prev != c.device) (void)hipSetDevice(prev);
    return err == hipSuccess ? LSE_OK : LSE_ERR_HIP;
}

lse_status_t check_forward(const void* x, lse_dtype_t dtype, int64_t rows, int64_t cols,
                           int64_t row_stride, const float* out) {
    lse_status_t st = check_sizes(dtype, rows, cols, row_stride, reinterpret_cast<uint64_t>(x));
    if (st != LSE_OK || rows == 0) return st;
    if (out == nullptr || (cols > 0 && x == nullptr)) return LSE_ERR_INVALID_ARG;
    if (reinterpret_cast<uint64_t>(out) % 4 != 0) return LSE_ERR_INVALID_ARG;
    return LSE_OK;
}

}  // namespace lse

namespace {

lse::ForwardContext context_of(lse_handle_t h) {
    lse::ForwardContext c{};
    c.device = h->device;
    c.n_cu = h->n_cu;
    c.schedule = h->schedule;
    c.block = h->block;
    c.unroll = h->unroll;
    c.parts = h->parts;
    c.waves_per_cu = h->waves_per_cu;
    c.lanes_per_row = h->lanes_per_row;
    c.ws_pairs = h->ws_pairs;
    c.counters = h->counters;
    c.pair_capacity = int64_t{LSE_SPLIT_MAX_ROWS} * LSE_SPLIT_MAX_PARTS;
    c.counter_capacity = LSE_SPLIT_MAX_ROWS;
    return c;
}

}  // namespace

extern "C" {

lse_status_t lse_forward(lse_handle_t h, const void* x, lse_dtype_t dtype, int64_t rows,
                         int64_t cols, int64_t row_stride, float* out, hipStream_t stream) {
    lse_status_t st = lse::check_forward(x, dtype, rows, cols, row_stride, out);
    if (st != LSE_OK) return st;
    if (h == nullptr) return LSE_ERR_INVALID_ARG;
    if (rows == 0) return LSE_OK;
    return lse::run_forward(context_of(h), x, dtype, rows, cols, row_stride, out, nullptr, nullptr,
                            stream);
}

}  // extern "C"

namespace {

// lse_backward and lse_token_logprob_backward: the same checks and plan; with
// targets the kernels add the one-hot term of the log-probability.
lse_status_t run_backward(lse_handle_t h, const void* x, lse_dtype_t dtype, int64_t rows,
                          int64_t cols, int64_t row_stride, const int64_t* targets,
                          bool with_targets, const float* lse, const float* grad_out,
                          void* grad_x, int64_t grad_row_stride, hipStream_t stream) {
    const uint64_t x_addr = reinterpret_cast<uint64_t>(x);
    lse_status_t st = check_sizes(dtype, rows, cols, row_stride, x_addr);
    if (st != LSE_OK) return st;
    const int esize = elem_bytes(dtype);
    if (rows > 1 && (grad_row_stride < cols || grad_row_stride > (INT64_MAX / 4) / rows))
        return LSE_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return h == nullptr ? LSE_ERR_INVALID_ARG : LSE_OK;
    if (x == nullptr || lse == nullptr || grad_out == nullptr || grad_x == nullptr)
        return LSE_ERR_INVALID_ARG;
    if (with_targets && (targets == nullptr || reinterpret_cast<uint64_t>(targets) % 8 != 0))
        return LSE_ERR_INVALID_ARG;
    const uint64_t g_addr = reinterpret_cast<uint64_t>(grad_x);
    if (reinterpret_cast<uint64_t>(lse) % 4 != 0 || reinterpret_cast<uint64_t>(grad_out) % 4 != 0 ||
        g_addr % esize != 0)
        return LSE_ERR_INVALID_ARG;
    if (h == nullptr) return LSE_ERR_INVALID_ARG;

    lse::GradArgs a{};
    st = make_grad_plan(dtype, rows, cols, row_stride, grad_row_stride, x_addr, g_addr, h->n_cu, &a);
    if (st != LSE_OK) return st;
    a.x = static_cast<const char*>(x);
    a.lse = lse;
    a.grad_out = grad_out;
    a.targets = with_targets ? targets : nullptr;
    a.grad_x = static_cast<char*>(grad_x);
    a.stream = stream;

    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return LSE_ERR_HIP;
    if (prev != h->device && hipSetDevice(h->device) != hipSuccess) return LSE_ERR_HIP;
    const hipError_t err = lse::launch_grad(a);
    if (prev != h->device) (void)hipSetDevice(prev);
    return err == hipSuccess ? LSE_OK : LSE_ERR_HIP;
}

}  // namespace

extern "C" {

lse_status_t lse_backward(lse_handle_t h, const void* x, lse_dtype_t dtype, int64_t rows,
                          int64_t cols, int64_t row_stride, const float* lse,
                          const float* grad_out, void* grad_x, int64_t grad_row_stride,
                          hipStream_t stream) {
    return run_backward(h, x, dtype, rows, cols, row_stride, nullptr, false, lse, grad_out,
                        grad_x, grad_row_stride, stream);
}

lse_status_t lse_token_logprob_backward(lse_handle_t h, const void* x, lse_dtype_t dtype,
                                        int64_t rows, int64_t cols, int64_t row_stride,
                                        const int64_t* targets, const float* lse,
                                        const float* grad_logp, void* grad_x,
                                        int64_t grad_row_stride, hipStream_t stream) {
    return run_backward(h, x, dtype, rows, cols, row_stride, targets, true, lse, grad_logp,
                        grad_x, grad_row_stride, stream);
}

lse_status_t lse_forward_dim(lse_handle_t h, const void* x, lse_dtype_t dtype, int64_t outer,
                             int64_t n, int64_t inner, float* out, hipStream_t stream) {
    if (!valid_dtype(dtype)) return LSE_ERR_UNSUPPORTED_DTYPE;
    const int esize = elem_bytes(dtype);
    if (outer < 0 || n < 0 || inner < 0 || n > kMaxDim) return LSE_ERR_INVALID_ARG;
    constexpr int64_t kMaxOut = int64_t{1} << 40;
    if (inner > 0 && outer > kMaxOut / inner) return LSE_ERR_INVALID_ARG;
    const int64_t nout = outer * inner;
    if (nout > 0 && n > (INT64_MAX / esize) / nout) return LSE_ERR_INVALID_ARG;
    const uint64_t x_addr = reinterpret_cast<uint64_t>(x);
    if (nout == 0) return h == nullptr ? LSE_ERR_INVALID_ARG : LSE_OK;
    if (out == nullptr || (n > 0 && x == nullptr)) return LSE_ERR_INVALID_ARG;
    if ((n > 0 && x_addr % esize != 0) || reinterpret_cast<uint64_t>(out) % 4 != 0)
        return LSE_ERR_INVALID_ARG;
    if (h == nullptr) return LSE_ERR_INVALID_ARG;
    if (inner == 1) return lse_forward(h, x, dtype, outer, n, n, out, stream);

    const int k = 16 / esize;
    const bool vec = inner % k == 0 && x_addr % 16 == 0;
    lse::DimArgs a{};
    a.dtype = dtype;
    a.vector_cols = vec;
    a.x = static_cast<const char*>(x);
    a.n = n;
    a.inner = inner;
    a.ncv = vec ? nout / k : nout;
    a.out = out;
    a.ws_pairs = h->dim_pairs;
    a.counters = h->counters;
    a.stream = stream;
    const int cols_per_lane = vec ? k : 1;
    const int64_t cvs = vec ? inner / k : inner;  // column groups per j-row
    // Column groups per workgroup: 64 when a j-row holds that many and that
    // still leaves two tiles per CU, else 32 (or the whole j-row when it is
    // shorter, so that a workgroup reads consecutive short rows).
    a.gw = static_cast<int>(cvs >= 2 * kDimGroups &&
                                    ceil_div(a.ncv, 2 * kDimGroups) >= 2 * int64_t{h->n_cu}
                                ? 2 * kDimGroups
                                : std::min<int64_t>(kDimGroups, cvs));
    // Tiles whose pieces of a row do not start on 128-byte cache lines share
    // lines with their neighbours; those launches give each XCD a contiguous
    // run of workgroups (lse_cols). Measured with bench.py-style A/B copies
    // on one box: bf16 [512, 50257] over its first axis 24.05 -> 21.23 us,
    // fp32 [2048, 30001] 73.2 -> 51.2 us, bf16 [4096, 4097] 40.1 -> 35.6 us,
    // bf16 [512, 50264] (16-byte path, pitch not a multiple of 128 bytes)
    // 17.05 -> 16.38 us, fp32 [2048, 30004] 48.5 -> 42.7 us; where the pieces
    // are whole lines the mapping made no difference beyond the noise.
    a.xcd_runs = !vec || (int64_t{a.gw} * 16) % 128 != 0 || (inner * esize) % 128 != 0 ||
                 x_addr % 128 != 0;
    const int64_t rw = 256 / a.gw;                // j-rows per load step
    const int64_t tiles = ceil_div(a.ncv, a.gw);
    // Workgroups per tile along n: none while the tiles alone give every CU
    // a workgroup, else enough for about one per CU, each lane keeping at
    // least 16 steps of j, at most 1024 (and one tile's pairs must fit the
    // workspace); a forced value from lse_set_tuning's `parts` wins. Split
    // tiles go in batches whose pairs fit the workspace and whose tiles fit
    // the arrival counters. The one-column path, whose 2- and 4-byte loads
    // keep a quarter to an eighth of the 16-byte path's bytes in flight per
    // workgroup, aims for two workgroups per CU where that leaves at most 64
    // parts per tile (more parts make the tile's merge of their pairs wait
    // longer). Measured as library copies, medians of six alternating blocks,
    // over the first axis, against one per CU: fp32 [65536, 4097] 334 -> 302
    // us, bf16 [65536, 4097] 259 -> 221, fp32 [4096, 12001] (unsplit before)
    // 50.5 -> 45.1, fp32 [4096, 4097] 25.5 -> 22.4, bf16 [20000, 5003] 84.9 ->
    // 76.2; with up to 512 parts per tile, fp32 [1000000, 7] 16.8 -> 18.5 and
    // bf16 [1000000, 7] 15.8 -> 18.1, hence the limit. On the 16-byte path two
    // per CU were 5-15 % slower on every shape timed.
    const int64_t cap_pairs = LSE_DIM_MAX_PAIRS;
    const int64_t tile_pairs = static_cast<int64_t>(a.gw) * cols_per_lane;
    int64_t parts = h->parts;
    if (parts == 0) {
        parts = 1;
        const int64_t want =
            h->n_cu * (!vec && ceil_div(2 * int64_t{h->n_cu}, tiles) <= 64 ? 2 : 1);
        if (tiles < want)
            parts = std::min<int64_t>({ceil_div(want, tiles), int64_t{1024},
                                       std::max<int64_t>(1, n / (16 * rw))});
    }
    parts = std::min<int64_t>({parts, int64_t{1024}, cap_pairs / tile_pairs});
    const int64_t batch =
        parts > 1 ? std::min<int64_t>({tiles, cap_pairs / (tile_pairs * parts),
                                       int64_t{LSE_SPLIT_MAX_ROWS}})  // one counter per tile
                  : tiles;
    a.parts = static_cast<int>(parts);

    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return LSE_ERR_HIP;
    if (prev != h->device && hipSetDevice(h->device) != hipSuccess) return LSE_ERR_HIP;
    hipError_t err = hipSuccess;
    for (int64_t t0 = 0; t0 < tiles && err == hipSuccess; t0 += batch) {
        a.tile0 = t0;
        a.grid = std::min<int64_t>(batch, tiles - t0) * parts;
        err = lse::launch_cols(a);
    }
    if (prev != h->device) (void)hipSetDevice(prev);
    return err == hipSuccess ? LSE_OK : LSE_ERR_HIP;
}

lse_status_t lse_backward_dim(lse_handle_t h, const void* x, lse_dtype_t dtype, int64_t outer,
                              int64_t n, int64_t inner, const float* lse, const float* grad_out,
                              void* grad_x, hipStream_t stream) {
    if (!valid_dtype(dtype)) return LSE_ERR_UNSUPPORTED_DTYPE;
    const int esize = elem_bytes(dtype);
    if (outer < 0 || n < 0 || inner < 0 || n > kMaxDim) return LSE_ERR_INVALID_ARG;
    constexpr int64_t kMaxOut = int64_t{1} << 40;
    if (inner > 0 && outer > kMaxOut / inner) return LSE_ERR_INVALID_ARG;
    const int64_t nout = outer * inner;
    if (nout > 0 && n > (INT64_MAX / esize) / nout) return LSE_ERR_INVALID_ARG;
    if (nout == 0 || n == 0) return h == nullptr ? LSE_ERR_INVALID_ARG : LSE_OK;
    if (x == nullptr || lse == nullptr || grad_out == nullptr || grad_x == nullptr)
        return LSE_ERR_INVALID_ARG;
    const uint64_t x_addr = reinterpret_cast<uint64_t>(x);
    const uint64_t g_addr = reinterpret_cast<uint64_t>(grad_x);
    if (x_addr % esize != 0 || g_addr % esize != 0 ||
        reinterpret_cast<uint64_t>(lse) % 4 != 0 || reinterpret_cast<uint64_t>(grad_out) % 4 != 0)
        return LSE_ERR_INVALID_ARG;
    if (h == nullptr) return LSE_ERR_INVALID_ARG;
    // inner == 1: rows of n elements with one (lse, grad_out) pair each
    if (inner == 1)
        return lse_backward(h, x, dtype, outer, n, n, lse, grad_out, grad_x, n, stream);

    const int k = 16 / esize;
    const bool vec = inner % k == 0 && x_addr % 16 == 0 && g_addr % 16 == 0;
    // The flat kernel (lanes own 16-byte vectors of memory, or elements, and
    // stage their lse and grad_out through LDS) where the column tiles would
    // take one column per lane; and, while lse and grad_out total at most
    // 16 MiB (the flat kernel reads them again for every j, from L2 or the
    // Infinity Cache), for fp32, and
    // for 16-bit types whose row pitch is not a multiple of 128 bytes (the
    // tiles' row pieces then straddle cache lines) unless a tile spans whole
    // rows (32 column groups or fewer: consecutive rows, contiguous). The
    // column tiles otherwise, and whenever lse_set_tuning forces `parts`.
    // Measured as library copies over the first axis (flat against tiles):
    // fp32 [65536, 4097] 364 against 1316 us, bf16 [512, 50257] 28.0 against
    // 48.5, fp32 [65536, 4096] 359 against 417; bf16 [65536, 4104] 240
    // against 318, f16 [16384, 4104] 60.0 against 80.1, bf16 [512, 128264]
    // 59.7 against 66.8, bf16 [100000, 72] 9.2 against 8.0; fp32 [512,
    // 1048576] (8 MiB of lse and grad_out) 729 against 834, fp32 [64, 2000000]
    // (16 MB) 186 against 189, but fp32 [16, 4000000] and [32, 4000000] (32
    // MB) 132 against 98 and 263 against 189; bf16 [512, 128256] 58.7 against
    // 49.3, bf16 [65536, 4096] 261 against 235.
    constexpr int64_t kFlatTableBytes = int64_t{16} << 20;
    const bool table_cached = nout <= kFlatTableBytes / 8;
    const bool pitch_off_lines = (inner * esize) % 128 != 0 && inner / k > kDimGroups;
    if (h->parts == 0 &&
        (!vec || (table_cached && (dtype == LSE_DTYPE_F32 || pitch_off_lines)))) {
        lse::DimFlatArgs f{};
        f.dtype = dtype;
        f.x = static_cast<const char*>(x);
        f.grad_x = static_cast<char*>(grad_x);
        f.lse = lse;
        f.grad_out = grad_out;
        f.n = n;
        f.inner = inner;
        f.total = nout * n;  // below INT64_MAX / esize by the checks above
        f.vec = x_addr % 16 == g_addr % 16;
        f.head = f.vec ? std::min<int64_t>(static_cast<int64_t>((16 - x_addr % 16) % 16) / esize,
                                           f.total)
                       : 0;
        f.nvec = f.vec ? (f.total - f.head) / k : f.total;
        f.m_inner = inner < (int64_t{1} << 32) ? UINT64_MAX / static_cast<uint64_t>(inner) + 1 : 0;
        f.m_n = n == 1 ? 0 : UINT64_MAX / static_cast<uint64_t>(n) + 1;
        f.stream = stream;
        int prev = -1;
        if (hipGetDevice(&prev) != hipSuccess) return LSE_ERR_HIP;
        if (prev != h->device && hipSetDevice(h->device) != hipSuccess) return LSE_ERR_HIP;
        const hipError_t err = lse::launch_grad_flat(f);
        if (prev != h->device) (void)hipSetDevice(prev);
        return err == hipSuccess ? LSE_OK : LSE_ERR_HIP;
    }
    lse::DimGradArgs a{};
    a.dtype = dtype;
    a.vector_cols = vec;
    a.x = static_cast<const char*>(x);
    a.n = n;
    a.inner = inner;
    a.ncv = vec ? nout / k : nout;
    a.lse = lse;
    a.grad_out = grad_out;
    a.grad_x = static_cast<char*>(grad_x);
    a.stream = stream;
    // Tiles of 32 column groups (or the whole j-row when it is shorter), XCD
    // runs where tiles share cache lines; n is split until there are about
    // two workgroups per CU, each lane keeping at least 16 steps of j
    // (nothing is merged). Measured at steady state against 64, 128 and 256
    // groups and against splits up to 8 and 32 workgroups per CU on
    // workloads 2-5 reduced over their first axis: 32 groups were as fast
    // as the best on four and 11 % faster on bf16 [4096, 262144] (846
    // against 955 us with 64); wider tiles lost up to 20 %, and more parts
    // won 4 % on fp32 [16777216, 16] but lost 6-10 % on the others.
    const int64_t cvs = vec ? inner / k : inner;
    a.gw = static_cast<int>(std::min<int64_t>(kDimGroups, cvs));
    a.xcd_runs = !vec || (int64_t{a.gw} * 16) % 128 != 0 || (inner * esize) % 128 != 0 ||
                 x_addr % 128 != 0 || g_addr % 128 != 0;
    const int64_t rw = 256 / a.gw;
    const int64_t tiles = ceil_div(a.ncv, a.gw);
    // Where a tile spans whole j-rows (inner of at most 32 column groups),
    // consecutive rows are contiguous and the launch is a copy in all but
    // its arithmetic: parts of one batch per lane, as many as that takes (at
    // most 65536 per tile), as the copy's short chunks; measured on fp32
    // [16777216, 16] over its first axis, 437 -> 357 us (its copy control:
    // 350 us). On wider rows the same split was 3-11 % faster where the plan
    // above launches 600 workgroups or fewer and 8 % slower on bf16
    // [512, 128256], so those keep it.
    int64_t parts = h->parts;
    if (parts == 0) {
        parts = 1;
        const int64_t want = 2 * int64_t{h->n_cu};
        if (cvs <= a.gw)
            parts = std::min<int64_t>(ceil_div(n, rw * 4), int64_t{65536});
        else if (tiles < want)
            parts = std::min<int64_t>({ceil_div(want, tiles), int64_t{1024},
                                       std::max<int64_t>(1, n / (16 * rw))});
    }
    parts = std::min<int64_t>(parts, int64_t{65536});
    a.parts = static_cast<int>(parts);
    const int64_t batch = std::min<int64_t>(tiles, (int64_t{1} << 30) / parts);

    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return LSE_ERR_HIP;
    if (prev != h->device && hipSetDevice(h->device) != hipSuccess) return LSE_ERR_HIP;
    hipError_t err = hipSuccess;
    for (int64_t t0 = 0; t0 < tiles && err == hipSuccess; t0 += batch) {
        a.tile0 = t0;
        a.grid = std::min<int64_t>(batch, tiles - t0) * parts;
        err = lse::launch_grad_cols(a);
    }
    if (prev != h->device) (void)hipSetDevice(prev);
    return err == hipSuccess ? LSE_OK : LSE_ERR_HIP;
}

lse_status_t lse_token_logprob(lse_handle_t h, const void* x, lse_dtype_t dtype, int64_t rows,
                               int64_t cols, int64_t row_stride, const int64_t* targets,
                               float* logp, float* lse_out, hipStream_t stream) {
    const uint64_t x_addr = reinterpret_cast<uint64_t>(x);
    lse_status_t st = check_sizes(dtype, rows, cols, row_stride, x_addr);
    if (st != LSE_OK) return st;
    if (rows == 0) return h == nullptr ? LSE_ERR_INVALID_ARG : LSE_OK;
    if (targets == nullptr || logp == nullptr || (cols > 0 && x == nullptr))
        return LSE_ERR_INVALID_ARG;
    if (reinterpret_cast<uint64_t>(targets) % 8 != 0 || reinterpret_cast<uint64_t>(logp) % 4 != 0 ||
        reinterpret_cast<uint64_t>(lse_out) % 4 != 0)
        return LSE_ERR_INVALID_ARG;
    if (h == nullptr) return LSE_ERR_INVALID_ARG;
    return lse::run_forward(context_of(h), x, dtype, rows, cols, row_stride, lse_out, targets,
                            logp, stream);
}

}  // extern "C"
