// lse_kernels.hip - the row-wise log-sum-exp kernels for gfx950 and their
// launch dispatch.
//
// One pass over the input, one fp32 scalar out per row: the single-pass fused
// LSE of "Speeding up Log-Sum-Exp: Kernel Fusion at the Memory Wall, Integer
// Arithmetic at the Compute Wall" (§3, §3.1), laid out for CDNA4. The work is
// bound by HBM bandwidth (the paper's §4.2 finds fused LSE time approaching
// the memory lower bound), so the kernels aim at full 16-byte coalesced,
// non-temporal loads with many bytes in flight per compute unit, and keep the
// per-element VALU work to decode, max, one fma, one v_exp_f32 and one add.
//
// Three schedules, picked on the host by shape (lse_api.cpp):
//
//  rows_in_registers  short rows. A group of G lanes (G = 1..64) holds a
//                     whole row in registers, so a wavefront holds 64/G rows
//                     per round and loads ROUNDS rounds before computing.
//                     With the row resident, the (max, sum) recursion
//                     collapses to one group max and one rescaled group sum.
//  stream_rows        long rows, one workgroup per row. Each lane folds
//                     batches of U 16-byte loads into its (m, c, s), the
//                     workgroup merges the lanes' pairs.
//  stream_rows<SPLIT> too few rows to fill the GPU. Each row is cut into P
//                     parts, one workgroup each; every part writes its
//                     (m, s) pair to a workspace, and the last workgroup of
//                     a row to arrive (an agent-scope counter) merges the P
//                     pairs in part order and resets the counter.
#include "lse_device.h"
#include "lse_launch.h"

namespace lse {

// s_waitcnt immediate for gfx9: vmcnt = 0, expcnt and lgkmcnt left at their
// maxima (not waited on).
constexpr int kWaitVmcnt0 = 0x0F70;

// ---------------------------------------------------------------------------
// Slow pass for rows whose maximum m is finite but beyond +-2^30: the sum of
// 2^((x - m) * log2 e) in natural units. Each lane sums elements j = first,
// first + step, ...; the caller reduces across lanes.
template <DType D>
__device__ float natural_units_sum(const char* rp, int64_t cols, float m, int64_t first,
                                   int64_t step) {
    float s = 0.0f;
    for (int64_t j = first; j < cols; j += step)
        s += exp2_hw((load_scalar<D>(rp + j * Elem<D>::kBytes) - m) * kLog2e);
    return s;
}

// ---------------------------------------------------------------------------
// Schedule A: rows held in registers.
//
// Lane l of a wavefront belongs to group l / G and is member g = l % G. In
// round q, group r of wavefront w holds row (w * ROUNDS + q) * (64/G) + r.
// Member g loads the row's units g, g + G, ..., g + (VPL-1) * G, where a unit
// is 16 bytes (VEC) or one element (rows not 16-byte aligned); members
// g < tail also load the tail element units*K + g (a row's last cols % K
// elements). Loads outside the row are replaced by -inf, which changes
// neither the max nor the sum.
template <DType D, int G, int VPL, bool VEC, int ROUNDS>
__global__ __launch_bounds__(256) void rows_in_registers(const char* __restrict__ x,
                                                         int64_t rows, int64_t cols,
                                                         int64_t stride_bytes,
                                                         float* __restrict__ out) {
    constexpr int EB = Elem<D>::kBytes;
    constexpr int K = VEC ? Elem<D>::kPerVec : 1;  // elements per unit
    constexpr int R = 64 / G;                      // rows per wavefront per round
    constexpr int NV = VPL * K;                    // values per lane per round

    const int lane = threadIdx.x & 63;
    const int g = lane & (G - 1);
    const int sub = lane / G;
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
    const int64_t units = cols / K;
    const int tail = static_cast<int>(cols - units * K);

    for (int64_t it = wave; it * (R * ROUNDS) < rows; it += nwaves) {
        float v[ROUNDS][NV];
        float tv[ROUNDS];
        int64_t row[ROUNDS];
#pragma unroll
        for (int q = 0; q < ROUNDS; ++q) {
            row[q] = (it * ROUNDS + q) * R + sub;
            const bool live = row[q] < rows;
            const char* rp = x + (live ? row[q] : 0) * stride_bytes;
#pragma unroll
            for (int u = 0; u < VPL; ++u) {
                const int64_t unit = g + static_cast<int64_t>(u) * G;
                if constexpr (VEC) {
                    u32x4 w = neg_inf_vec<D>();
                    if (live && unit < units)
                        w = load_vec(reinterpret_cast<const u32x4*>(rp + unit * 16));
                    decode<D>(w, &v[q][u * K]);
                } else {
                    v[q][u] = (live && unit < units) ? load_scalar<D>(rp + unit * EB) : -kInf;
                }
            }
            tv[q] = (live && g < tail) ? load_scalar<D>(rp + (units * K + g) * EB) : -kInf;
        }
#pragma unroll
        for (int q = 0; q < ROUNDS; ++q) {
            float mx = max_of<NV>(tv[q], v[q]);
            mx = group_reduce<G>(mx, OpMax{});
            const float c = base2_ref(mx);
            float s = sum_exp_of<NV>(v[q], c) + exp2_hw(__builtin_fmaf(tv[q], kLog2e, -c));
            s = group_reduce<G>(s, OpSum{});
            bool slow;
            float r = finish(mx, c, s, slow);
            if (slow) {  // uniform within the group: mx and s are group-reduced
                float s2 = exp2_hw((tv[q] - mx) * kLog2e);
#pragma unroll
                for (int j = 0; j < NV; ++j) s2 += exp2_hw((v[q][j] - mx) * kLog2e);
                s2 = group_reduce<G>(s2, OpSum{});
                r = __builtin_fmaf(log2_hw(s2), kLn2, mx);
            }
            if (g == 0 && row[q] < rows) out[row[q]] = r;
        }
    }
}

// ---------------------------------------------------------------------------
// Schedules B and C: one workgroup streams a row, or one part of a row.
//
// A row starting at rp splits into a head of elements before the first
// 16-byte boundary (rows not 16-byte aligned), nvec whole 16-byte vectors,
// and a tail of fewer than K elements. Part p of P takes vectors
// [nvec*p/P, nvec*(p+1)/P); part 0 also takes the head, part P-1 the tail.
// Lane t takes vectors t, t + BLOCK, ... in batches of U loads issued before
// any is used.
template <DType D, int BLOCK, int U, bool SPLIT>
__global__ __launch_bounds__(BLOCK) void stream_rows(const char* __restrict__ x,
                                                     int64_t rows, int64_t cols,
                                                     int64_t stride_bytes,
                                                     float* __restrict__ out, int parts,
                                                     unsigned* __restrict__ ws_pairs,
                                                     unsigned* __restrict__ counters) {
    constexpr int EB = Elem<D>::kBytes;
    constexpr int K = Elem<D>::kPerVec;
    __shared__ float scratch[BLOCK / 64];
    __shared__ int is_last;

    const int tid = threadIdx.x;
    const int64_t wg = blockIdx.x;
    const int64_t row = SPLIT ? wg / parts : wg;
    const int part = SPLIT ? static_cast<int>(wg % parts) : 0;
    const int nparts = SPLIT ? parts : 1;

    const char* rp = x + row * stride_bytes;
    const int mis = static_cast<int>(reinterpret_cast<uintptr_t>(rp) & 15);
    const int64_t head = mis ? (cols < (16 - mis) / EB ? cols : (16 - mis) / EB) : 0;
    const int64_t nvec = (cols - head) / K;
    const int64_t tail = cols - head - nvec * K;
    const u32x4* vp = reinterpret_cast<const u32x4*>(rp + head * EB);

    int64_t v0 = 0, v1 = nvec;
    if constexpr (SPLIT) {
        v0 = nvec * part / nparts;
        v1 = nvec * (part + 1) / nparts;
    }

    Acc a = acc_empty();
    if (part == 0 && tid < head) {
        float f = load_scalar<D>(rp + tid * EB);
        fold<1>(a, &f);
    }
    if (part == nparts - 1 && tid < tail) {
        float f = load_scalar<D>(rp + (head + nvec * K + tid) * EB);
        fold<1>(a, &f);
    }

    // Batches of U vectors per lane: nfull whole batches, then one guarded
    // batch holding the last rem < U * BLOCK vectors. Software-pipelined:
    // the loads of the next batch are in flight while a batch is folded, so
    // the fold's VALU time stays off each wavefront's load-to-load path. All
    // branches are uniform; in the guarded batch, lanes past the end load the
    // part's last vector (in bounds) and replace it by -inf, so the loads
    // need no divergent control flow and the hardware wait counts stay exact.
    const int64_t n = v1 - v0;
    const u32x4* p0 = vp + v0 + tid;
    const int64_t nfull = n / (static_cast<int64_t>(U) * BLOCK);
    const int64_t rem = n - nfull * U * BLOCK;

    auto load_full = [&](u32x4 (&w)[U], int64_t k) {
        const u32x4* q = p0 + k * (U * BLOCK);
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = load_vec(q + u * BLOCK);
    };
    auto load_guarded = [&](u32x4 (&w)[U]) {
        const u32x4* q = vp + v0;
        const int64_t base = nfull * U * BLOCK;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = base + tid + u * BLOCK;
            const u32x4 v = load_vec(q + (j < n ? j : n - 1));
            w[u] = j < n ? v : neg_inf_vec<D>();
        }
    };
    auto fold_batch = [&](const u32x4 (&w)[U]) {
        float f[U * K];
#pragma unroll
        for (int u = 0; u < U; ++u) decode<D>(w[u], &f[u * K]);
        fold<U * K>(a, f);
    };

    if (n > 0) {
        u32x4 wa[U], wb[U], wc[U];
        if (nfull == 0) {
            load_guarded(wc);
            fold_batch(wc);
        } else {
            load_full(wa, 0);
            int64_t k = 0;
            for (; k + 2 < nfull; k += 2) {
                load_full(wb, k + 1);
                fold_batch(wa);
                load_full(wa, k + 2);
                fold_batch(wb);
            }
            if (k + 1 < nfull) {
                load_full(wb, k + 1);
                load_guarded(wc);
                fold_batch(wa);
                fold_batch(wb);
            } else {
                load_guarded(wc);
                fold_batch(wa);
            }
            if (rem > 0) fold_batch(wc);
        }
    }

    // Merge the lanes: common maximum first, then each lane's sum rescaled to it.
    float m = block_reduce<BLOCK>(a.m, OpMax{}, scratch);
    float c = base2_ref(m);
    float s = block_reduce<BLOCK>(acc_sum(a) * exp2_hw(a.c - c), OpSum{}, scratch);

    if constexpr (SPLIT) {
        // Publish this part's pair, then count the part in. The pair is
        // written with agent-scope (sc1) stores, which are coherent across
        // the XCDs' L2s; waiting for them to complete before the counter add
        // orders them before it. The last part to arrive reads the pairs
        // with agent-scope loads after its add returns. No L2-wide writeback
        // or invalidate is needed, as every access involved is agent-scope.
        if (tid == 0) {
            unsigned* slot = ws_pairs + 2 * (row * nparts + part);
            __hip_atomic_store(slot, __float_as_uint(m), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(slot + 1, __float_as_uint(s), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            const unsigned prev = __hip_atomic_fetch_add(counters + row, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            is_last = (prev == static_cast<unsigned>(nparts - 1));
        }
        __syncthreads();
        if (!is_last) return;
        float pm = -kInf, ps = 0.0f;
        if (tid < nparts) {
            const unsigned* slot = ws_pairs + 2 * (row * nparts + tid);
            pm = __uint_as_float(__hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            ps = __uint_as_float(
                __hip_atomic_load(slot + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        }
        const float pc = base2_ref(pm);
        m = block_reduce<BLOCK>(pm, OpMax{}, scratch);
        c = base2_ref(m);
        s = block_reduce<BLOCK>(ps * exp2_hw(pc - c), OpSum{}, scratch);
        if (tid == 0)
            __hip_atomic_store(counters + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    bool slow;
    float r = finish(m, c, s, slow);
    if (slow) {  // uniform: m and s are block-reduced
        float s2 = natural_units_sum<D>(rp, cols, m, tid, BLOCK);
        s2 = block_reduce<BLOCK>(s2, OpSum{}, scratch);
        r = __builtin_fmaf(log2_hw(s2), kLn2, m);
    }
    if (tid == 0) out[row] = r;
}

// ---------------------------------------------------------------------------
// Dispatch from a host launch plan to a template instance.

namespace {

template <DType D, int G, int VPL, bool VEC>
hipError_t launch_regs(const LaunchArgs& a) {
    // More rounds in flight when each lane's share of a row is small.
    constexpr int ROUNDS = VPL == 1 ? 4 : (VPL == 2 ? 2 : 1);
    if (a.rows_per_wave != (64 / G) * ROUNDS) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((rows_in_registers<D, G, VPL, VEC, ROUNDS>), dim3(a.grid), dim3(256), 0,
                       a.stream, a.x, a.rows, a.cols, a.stride_bytes, a.out);
    return hipGetLastError();
}

template <DType D, int G, bool VEC>
hipError_t launch_regs_vpl(const LaunchArgs& a) {
    switch (a.loads_per_lane) {
        case 1: return launch_regs<D, G, 1, VEC>(a);
        case 2: if constexpr (G == 64) return launch_regs<D, G, 2, VEC>(a); break;
        case 4: if constexpr (G == 64) return launch_regs<D, G, 4, VEC>(a); break;
        case 8: if constexpr (G == 64) return launch_regs<D, G, 8, VEC>(a); break;
        case 16: if constexpr (G == 64) return launch_regs<D, G, 16, VEC>(a); break;
    }
    return hipErrorInvalidConfiguration;
}

template <DType D, bool VEC>
hipError_t launch_regs_g(const LaunchArgs& a) {
    switch (a.lanes_per_row) {
        case 1: return launch_regs_vpl<D, 1, VEC>(a);
        case 2: return launch_regs_vpl<D, 2, VEC>(a);
        case 4: return launch_regs_vpl<D, 4, VEC>(a);
        case 8: return launch_regs_vpl<D, 8, VEC>(a);
        case 16: return launch_regs_vpl<D, 16, VEC>(a);
        case 32: return launch_regs_vpl<D, 32, VEC>(a);
        case 64: return launch_regs_vpl<D, 64, VEC>(a);
    }
    return hipErrorInvalidConfiguration;
}

template <DType D, int BLOCK, int U, bool SPLIT>
hipError_t launch_stream(const LaunchArgs& a) {
    hipLaunchKernelGGL((stream_rows<D, BLOCK, U, SPLIT>), dim3(a.grid), dim3(BLOCK), 0, a.stream,
                       a.x, a.rows, a.cols, a.stride_bytes, a.out, a.parts, a.ws_pairs,
                       a.counters);
    return hipGetLastError();
}

template <DType D, bool SPLIT>
hipError_t launch_stream_cfg(const LaunchArgs& a) {
    const int key = a.block * 100 + a.unroll;
    switch (key) {
        case 25604: return launch_stream<D, 256, 4, SPLIT>(a);
        case 25608: return launch_stream<D, 256, 8, SPLIT>(a);
        case 51204: return launch_stream<D, 512, 4, SPLIT>(a);
        case 51208: return launch_stream<D, 512, 8, SPLIT>(a);
        case 102404: return launch_stream<D, 1024, 4, SPLIT>(a);
        case 102408: return launch_stream<D, 1024, 8, SPLIT>(a);
    }
    return hipErrorInvalidConfiguration;
}

template <DType D>
hipError_t launch_dtype(const LaunchArgs& a) {
    switch (a.schedule) {
        case kSchedRowsPerWave:
            return a.vector_loads ? launch_regs_g<D, true>(a) : launch_regs_g<D, false>(a);
        case kSchedRowPerWG:
            return launch_stream_cfg<D, false>(a);
        case kSchedSplitRow:
            return launch_stream_cfg<D, true>(a);
    }
    return hipErrorInvalidConfiguration;
}

}  // namespace

hipError_t launch(const LaunchArgs& a) {
    if (a.grid <= 0) return hipSuccess;
    return a.bf16 ? launch_dtype<DType::BF16>(a) : launch_dtype<DType::F32>(a);
}

}  // namespace lse
