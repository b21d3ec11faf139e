// lse_kernels.h - the row-wise log-sum-exp kernels for gfx950 and their
// launch dispatch per element type. Each element type's instances are built in
// a translation unit of their own (lse_kernels_f32.hip, lse_kernels_bf16.hip,
// lse_kernels_f16.hip); lse_kernels.hip holds the entry of the dispatch.
//
// One pass over the input, one fp32 scalar out per row: the single-pass fused
// LSE of "Speeding up Log-Sum-Exp: Kernel Fusion at the Memory Wall, Integer
// Arithmetic at the Compute Wall" (§3, §3.1), laid out for CDNA4. The work is
// bound by HBM bandwidth (the paper's §4.2 finds fused LSE time approaching
// the memory lower bound), so the kernels aim at full 16-byte coalesced,
// non-temporal loads with many bytes in flight per compute unit, and keep the
// per-element VALU work of the streaming loop to decode, one fma, one
// v_exp_f32 and one add (the running maximum is only refreshed when a batch
// outgrows it: fold_lazy_vecs).
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
//                     (m, s) pair to a workspace slot, and the last
//                     workgroup of a row to arrive (an agent-scope counter)
//                     merges the P pairs in part order and clears the slots
//                     and the counter.
#pragma once

#include "lse_device.h"
#include "lse_launch.h"

namespace lse {

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
// round q of iteration i, group r of the wavefront holds row
// i * RW + q * (64/G) + r, RW = (64/G) * ROUNDS rows per iteration. Member g
// loads the row's units g, g + G, ..., g + (VPL-1) * G, where a unit is 16
// bytes (VEC) or one element (rows not 16-byte aligned); with TAIL, members
// g < tail also load the element units*K + g (the row's last cols % K
// elements). A wavefront handles iterations wave, wave + nwaves, ... and loads
// its next iteration while it folds the current one.
//
// Loads never branch. FAST launches (every row has exactly G * VPL units and
// the rows fill whole iterations) need no index checks at all; otherwise a
// unit index past the row, or a row past the last, is clamped to one in
// bounds and its value replaced by -inf, which changes neither the max nor
// the sum. The prefetch of an iteration past the last reloads the last one.
// The planner guarantees units >= 1 for VEC and cols >= 1 (cols == 0 is
// written directly).
template <DType D, int VPL, bool VEC, int ROUNDS>
struct RegTile {
    u32x4 w[ROUNDS][VEC ? VPL : 1];  // 16-byte units (VEC)
    float e[ROUNDS][VEC ? 1 : VPL];  // single elements (not VEC)
    float tv[ROUNDS];                // tail element (TAIL)
    int64_t tg[ROUNDS];              // target column of the round's row (TOK)
};

// What every iteration of one wavefront shares.
struct RegRows {
    const char* x;     // element (0, 0)
    int64_t rows;
    int64_t cols;
    int64_t units;     // whole units per row
    int64_t stride;    // bytes between row starts
    int64_t last_it;   // index of the last iteration
    int64_t lane_off;  // sub * stride + g * (bytes per unit): this lane's first unit in round 0
    const int64_t* targets;  // TOK: target column per row
    int g, sub, tail;
};

template <DType D, int G, int VPL, bool VEC, bool TAIL, bool FAST, int ROUNDS, bool TOK>
__device__ __forceinline__ void load_tile(RegTile<D, VPL, VEC, ROUNDS>& t, const RegRows& rr,
                                          int64_t it) {
    constexpr int EB = Elem<D>::kBytes;
    constexpr int K = VEC ? Elem<D>::kPerVec : 1;
    constexpr int UB = VEC ? 16 : EB;  // bytes per unit
    constexpr int R = 64 / G;
    constexpr int RW = R * ROUNDS;
    const char* base = rr.x + it * RW * rr.stride;  // uniform
#pragma unroll
    for (int q = 0; q < ROUNDS; ++q) {
        const char* row_start;
        int64_t row = it * RW + q * R + rr.sub;
        if constexpr (FAST) {
            row_start = base + q * R * rr.stride + rr.lane_off - rr.g * UB;
        } else {
            row = row < rr.rows ? row : rr.rows - 1;
            row_start = rr.x + row * rr.stride;
        }
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
            int64_t unit = rr.g + static_cast<int64_t>(u) * G;
            if constexpr (!FAST) unit = unit < rr.units ? unit : rr.units - 1;
            const char* p = row_start + unit * UB;
            if constexpr (VEC)
                t.w[q][u] = load_vec(reinterpret_cast<const u32x4*>(p));
            else
                t.e[q][u] = load_scalar<D>(p);
        }
        if constexpr (TAIL)
            t.tv[q] = load_scalar<D>(row_start + (rr.units * K + (rr.g < rr.tail ? rr.g : 0)) * EB);
        if constexpr (TOK) t.tg[q] = rr.targets[row];
    }
}

// v[idx] for a power-of-two N and 0 <= idx < N, by a select tree on the bits
// of idx (N - 1 selects, no indexed register access).
template <int N>
__device__ __forceinline__ float pick(const float* v, int idx) {
    if constexpr (N == 1) {
        return v[0];
    } else {
        constexpr int H = N / 2;
        const float lo = pick<H>(v, idx & (H - 1));
        const float hi = pick<H>(v + H, idx & (H - 1));
        return (idx & H) ? hi : lo;
    }
}

// Fold one tile: every round's row max and rescaled sum, then the finish of
// each row into `stage` (and, with TOK, its token log-probability into
// `stage_lp`), RW slots in row order.
template <DType D, int G, int VPL, bool VEC, bool TAIL, bool FAST, int ROUNDS, bool TOK>
__device__ __forceinline__ void fold_tile(const RegTile<D, VPL, VEC, ROUNDS>& t,
                                          const RegRows& rr, float* stage, float* stage_lp) {
    constexpr int K = VEC ? Elem<D>::kPerVec : 1;
    constexpr int R = 64 / G;
    constexpr int NV = VPL * K;
    const int g = rr.g;
    // Decode, with -inf in place of every clamped unit.
    float v[ROUNDS][NV];
    float tv[ROUNDS];
#pragma unroll
    for (int q = 0; q < ROUNDS; ++q) {
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
            const bool ok = FAST || g + static_cast<int64_t>(u) * G < rr.units;
            if constexpr (VEC) {
                float f[K];
                decode<D>(t.w[q][u], f);
#pragma unroll
                for (int k = 0; k < K; ++k) v[q][u * K + k] = ok ? f[k] : -kInf;
            } else {
                v[q][u] = ok ? t.e[q][u] : -kInf;
            }
        }
        tv[q] = -kInf;
        if constexpr (TAIL) tv[q] = g < rr.tail ? t.tv[q] : -kInf;
    }
    // Per round: the group's max, then the group's sum rescaled to it.
    float mx[ROUNDS], sq[ROUNDS];
    bool any_slow = false;
#pragma unroll
    for (int q = 0; q < ROUNDS; ++q) {
        mx[q] = group_reduce<G>(TAIL ? max_of<NV>(tv[q], v[q]) : max_of<NV - 1>(v[q][0], v[q] + 1),
                                OpMax{});
        const float c = base2_ref(mx[q]);
        float sum = sum_exp_of<NV>(v[q], c);
        if constexpr (TAIL) sum += exp2_hw(__builtin_fmaf(tv[q], kLog2e, -c));
        sq[q] = group_reduce<G>(sum, OpSum{});
        any_slow |= beyond_clamp(mx[q]);
    }
    // TOK: the target element of each round's row. Column c lies in unit
    // c / K, held by member (c / K) % G as its unit (c / K) / G, or in the
    // tail (member c - units*K). The holder contributes the element and the
    // other members +0, so the group sum is the element itself (+-inf and
    // NaN included). A target outside [0, cols) is flagged for NaN.
    float xt[ROUNDS];
    bool tok_ok[ROUNDS];
    if constexpr (TOK) {
#pragma unroll
        for (int q = 0; q < ROUNDS; ++q) {
            const int64_t c = t.tg[q];
            tok_ok[q] = c >= 0 && c < rr.cols;
            const int64_t unit = c / K;
            float mine = 0.0f;
            if (tok_ok[q] && unit < rr.units && static_cast<int>(unit % G) == g)
                mine = pick<NV>(v[q], static_cast<int>(unit / G) * K + static_cast<int>(c - unit * K));
            if constexpr (TAIL) {
                if (tok_ok[q] && c >= rr.units * K && c - rr.units * K == g) mine = tv[q];
            }
            xt[q] = group_reduce<G>(mine, OpSum{});
        }
    }
    if (any_slow) {  // rare: a row's max is finite and beyond +-2^30
#pragma unroll
        for (int q = 0; q < ROUNDS; ++q) {
            if (needs_natural_units(mx[q], sq[q])) {  // uniform within the group
                float s2 = exp2_hw((tv[q] - mx[q]) * kLog2e);
#pragma unroll
                for (int j = 0; j < NV; ++j) s2 += exp2_hw((v[q][j] - mx[q]) * kLog2e);
                s2 = group_reduce<G>(s2, OpSum{});
                // The result is then m + ln2 * log2(s2), s2 >= 1; a sum is never
                // negative otherwise, so -s2 marks the round for the finish.
                sq[q] = -s2;
            }
        }
    }
    // Every lane of a group holds every round's result; member g finishes
    // rounds g, g + G, ..., so the log and the special-value checks run once
    // per row. The results go to this wavefront's LDS slots in row order.
#pragma unroll
    for (int j = 0; j < (ROUNDS + G - 1) / G; ++j) {
        const int q = g + j * G;
        float m = mx[0], sum = sq[0], x_t = 0.0f;
        bool ok_t = false;
#pragma unroll
        for (int k = 0; k < ROUNDS; ++k) {
            m = q == k ? mx[k] : m;
            sum = q == k ? sq[k] : sum;
            if constexpr (TOK) {
                x_t = q == k ? xt[k] : x_t;
                ok_t = q == k ? tok_ok[k] : ok_t;
            }
        }
        if (G <= ROUNDS || q < ROUNDS) {
            const float r = sum < 0.0f ? __builtin_fmaf(log2_hw(-sum), kLn2, m)
                                       : finish(m, base2_ref(m), sum);
            stage[q * R + rr.sub] = r;
            if constexpr (TOK) stage_lp[q * R + rr.sub] = ok_t ? x_t - r : __builtin_nanf("");
        }
    }
}

// Store one iteration's RW staged results: lane l writes row it*RW + l, so
// consecutive lanes write consecutive words. `out` may be NULL (TOK only).
template <int RW, bool FAST, bool TOK, bool NT>
__device__ __forceinline__ void store_stage(const float* stage, const float* stage_lp, int64_t it,
                                            int64_t rows, float* out, float* logp) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < (RW + 63) / 64; ++i) {
        const int slot = lane + 64 * i;
        const int64_t r = it * RW + slot;
        if ((RW % 64 == 0 || slot < RW) && (FAST || r < rows)) {
            if constexpr (NT) {
                if (!TOK || out != nullptr) __builtin_nontemporal_store(stage[slot], out + r);
                if constexpr (TOK) __builtin_nontemporal_store(stage_lp[slot], logp + r);
            } else {
                if (!TOK || out != nullptr) out[r] = stage[slot];
                if constexpr (TOK) logp[r] = stage_lp[slot];
            }
        }
    }
}

// Where a wavefront's iterations hold at least 64 rows (rows of up to 64
// bytes), the results are not stored iteration by iteration: each
// wavefront keeps the results of up to F iterations in its LDS slots and
// stores them together (non-temporal), so the output stream reaches memory
// in bursts instead of one 256-byte store between every two 4 KiB reads.
// Measured on fp32 [16777216, 16]: a read + write kernel of this geometry
// took 186.7 us storing every iteration and 174.4 us flushing 64 iterations
// at a time (the same reads alone: 154.8 us). F fills 64 KiB of LDS per
// 256-thread workgroup (two workgroups per CU).
template <int RW, bool TOK>
struct Deferral {
    static constexpr bool kOn = RW >= 64;
    static constexpr int kF = kOn ? 4096 / (RW * (TOK ? 2 : 1)) : 1;
};

// The wavefront's loop over iterations wave, wave + nwaves, ...: the next
// iteration's tile is loaded (into the other buffer) before this one is folded.
// `stage` (and, with TOK, `stage_lp`) are this wavefront's F * RW LDS slots.
template <DType D, int G, int VPL, bool VEC, bool TAIL, bool FAST, int ROUNDS, bool TOK>
__device__ __forceinline__ void fold_rows(const RegRows& rr, float* out, float* logp, int64_t wave,
                                          int64_t nwaves, float* stage, float* stage_lp) {
    constexpr int RW = (64 / G) * ROUNDS;
    constexpr bool DEFER = Deferral<RW, TOK>::kOn;
    constexpr int F = Deferral<RW, TOK>::kF;
    RegTile<D, VPL, VEC, ROUNDS> ta, tb;
    int64_t it = wave;
    if (it > rr.last_it) return;
    int slot = 0;             // DEFER: iterations staged so far
    int64_t first_it = it;    // DEFER: the iteration in slot 0
    // Store the staged slots: slot j holds iteration first_it + j * nwaves.
    auto flush = [&]() {
        __builtin_amdgcn_wave_barrier();
        for (int j = 0; j < slot; ++j)
            store_stage<RW, FAST, TOK, true>(stage + j * RW, stage_lp + (TOK ? j * RW : 0),
                                             first_it + j * nwaves, rr.rows, out, logp);
        __builtin_amdgcn_wave_barrier();
        slot = 0;
    };
    auto fold_store = [&](const RegTile<D, VPL, VEC, ROUNDS>& t, int64_t cur) {
        if constexpr (DEFER) {
            if (slot == 0) first_it = cur;
            fold_tile<D, G, VPL, VEC, TAIL, FAST, ROUNDS, TOK>(t, rr, stage + slot * RW,
                                                               stage_lp + (TOK ? slot * RW : 0));
            if (++slot == F) flush();
        } else {
            fold_tile<D, G, VPL, VEC, TAIL, FAST, ROUNDS, TOK>(t, rr, stage, stage_lp);
            __builtin_amdgcn_wave_barrier();
            store_stage<RW, FAST, TOK, false>(stage, stage_lp, cur, rr.rows, out, logp);
            __builtin_amdgcn_wave_barrier();
        }
    };
    load_tile<D, G, VPL, VEC, TAIL, FAST, ROUNDS, TOK>(ta, rr, it);
    while (true) {
        int64_t next = it + nwaves;
        load_tile<D, G, VPL, VEC, TAIL, FAST, ROUNDS, TOK>(tb, rr, next < rr.last_it ? next : rr.last_it);
        fold_store(ta, it);
        it = next;
        if (it > rr.last_it) break;
        next = it + nwaves;
        load_tile<D, G, VPL, VEC, TAIL, FAST, ROUNDS, TOK>(ta, rr, next < rr.last_it ? next : rr.last_it);
        fold_store(tb, it);
        it = next;
        if (it > rr.last_it) break;
    }
    if constexpr (DEFER) {
        if (slot > 0) flush();
    }
}

template <DType D, int G, int VPL, bool VEC, bool TAIL, int ROUNDS, bool TOK>
__global__ __launch_bounds__(256) void rows_in_registers(const char* __restrict__ x,
                                                         int64_t rows, int64_t cols,
                                                         int64_t stride_bytes,
                                                         float* __restrict__ out,
                                                         const int64_t* __restrict__ targets,
                                                         float* __restrict__ logp) {
    constexpr int K = VEC ? Elem<D>::kPerVec : 1;
    constexpr int UB = VEC ? 16 : Elem<D>::kBytes;
    constexpr int RW = (64 / G) * ROUNDS;
    constexpr int F = Deferral<RW, TOK>::kF;
    // per-wavefront output staging (4 wavefronts per block), F iterations each
    __shared__ float stage_all[4][F * RW];
    __shared__ float stage_lp_all[TOK ? 4 : 1][TOK ? F * RW : 1];
    float* stage = stage_all[threadIdx.x >> 6];
    float* stage_lp = stage_lp_all[TOK ? threadIdx.x >> 6 : 0];
    const int lane = threadIdx.x & 63;
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;

    if (cols == 0) {  // the empty sum: every row is -inf, and no target is in range
        for (int64_t r = wave * 64 + lane; r < rows; r += nwaves * 64) {
            if (!TOK || out != nullptr) out[r] = -kInf;
            if constexpr (TOK) logp[r] = __builtin_nanf("");
        }
        return;
    }
    RegRows rr;
    rr.x = x;
    rr.rows = rows;
    rr.cols = cols;
    rr.units = cols / K;
    rr.stride = stride_bytes;
    rr.last_it = (rows + RW - 1) / RW - 1;
    rr.targets = targets;
    rr.g = lane & (G - 1);
    rr.sub = lane / G;
    rr.tail = static_cast<int>(cols - rr.units * K);
    rr.lane_off = rr.sub * stride_bytes + rr.g * UB;
    if (rr.units == G * VPL && rows % RW == 0)
        fold_rows<D, G, VPL, VEC, TAIL, true, ROUNDS, TOK>(rr, out, logp, wave, nwaves, stage,
                                                           stage_lp);
    else
        fold_rows<D, G, VPL, VEC, TAIL, false, ROUNDS, TOK>(rr, out, logp, wave, nwaves, stage,
                                                            stage_lp);
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
template <DType D, int BLOCK, int U, bool SPLIT, bool TOK>
__global__ __launch_bounds__(BLOCK) void stream_rows(const char* __restrict__ x, int64_t cols,
                                                     int64_t stride_bytes,
                                                     float* __restrict__ out, int parts,
                                                     unsigned* __restrict__ ws_pairs,
                                                     unsigned* __restrict__ counters,
                                                     const int64_t* __restrict__ targets,
                                                     float* __restrict__ logp) {
    constexpr int EB = Elem<D>::kBytes;
    constexpr int K = Elem<D>::kPerVec;
    __shared__ float pairs[2 * (BLOCK / 64)];
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

    // TOK: the row's target column and, once the first batches are in flight,
    // the aligned 32-bit word that holds its element. Both are uniform in the
    // workgroup and read through the scalar unit (constant address space), so
    // their wait counter is not the one the streaming loads count on; the word
    // is decoded only by the finish, where its wait costs nothing.
    int64_t tgt = 0;
    unsigned t_word = 0;
    bool t_hi = false, t_ok = false;
    if constexpr (TOK) tgt = targets[row];
    auto fetch_target = [&]() {
        if constexpr (TOK) {
            // The empty asm makes the index opaque here, so the address (and
            // the wait for the index) is not hoisted ahead of the first
            // batches' loads.
            int64_t tg = tgt;
            asm volatile("" : "+s"(tg));
            t_ok = tg >= 0 && tg < cols;
            const uintptr_t ad = reinterpret_cast<uintptr_t>(rp + (t_ok ? tg : 0) * EB);
            // an aligned word never crosses a page, so reading the whole word
            // around a bf16 element stays inside the caller's allocation
            t_word = *reinterpret_cast<const __attribute__((address_space(4))) unsigned*>(
                ad & ~uintptr_t{3});
            t_hi = (ad & 2) != 0;
        }
    };

    Acc a = acc_empty();
    // The head and tail elements of a row that is not 16-byte aligned: loaded
    // here, before the batches, but folded only after them, so their memory
    // round trip overlaps the stream instead of preceding it.
    float ends[2] = {-kInf, -kInf};
    const bool has_head = part == 0 && head > 0;  // uniform
    const bool has_tail = part == nparts - 1 && tail > 0;
    if (has_head && tid < head) ends[0] = load_scalar<D>(rp + tid * EB);
    if (has_tail && tid < tail) ends[1] = load_scalar<D>(rp + (head + nvec * K + tid) * EB);

    // Batches of U vectors per lane: nfull whole batches, then one guarded
    // batch holding the last rem < U * BLOCK vectors. Software-pipelined:
    // the loads of the next batch are issued before a batch is folded, and a
    // scheduling barrier after each group of loads keeps the compiler from
    // moving them into the fold (interleaved, the fold's first wait would
    // also wait for the next batch). Every batch issues exactly U loads with
    // no branch around them, so the hardware wait counts stay exact: in the
    // guarded batch, lanes past the end load the part's last vector (in
    // bounds), and the fold replaces those vectors by -inf.
    const int64_t n = v1 - v0;
    const u32x4* p0 = vp + v0 + tid;
    const int64_t nfull = n / (static_cast<int64_t>(U) * BLOCK);
    const int64_t rem = n - nfull * U * BLOCK;
    const int64_t gbase = nfull * U * BLOCK + tid;  // this lane's first index in the guarded batch

    auto load_full = [&](u32x4 (&w)[U], int64_t k) {
        const u32x4* q = p0 + k * (U * BLOCK);
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = load_vec(q + u * BLOCK);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto load_guarded = [&](u32x4 (&w)[U]) {
        const u32x4* q = vp + v0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = gbase + u * BLOCK;
            w[u] = load_vec(q + (j < n ? j : n - 1));
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto fold_batch = [&](const u32x4 (&w)[U]) { fold_lazy_vecs<D, U>(a, w); };
    auto fold_guarded = [&](const u32x4 (&w)[U]) {
        u32x4 m[U];
#pragma unroll
        for (int u = 0; u < U; ++u) m[u] = gbase + u * BLOCK < n ? w[u] : neg_inf_vec<D>();
        fold_batch(m);
    };

    // TOK: the target's word is fetched at one place, in the first pass of the
    // steady-state loop once two batches are in flight; parts too short to
    // enter that loop fetch it after their loads (no other path holds a
    // pending scalar load, which would make the compiler wait for it early).
    if (n > 0) {
        u32x4 wa[U], wb[U], wc[U];
        if (nfull == 0) {
            load_guarded(wc);
            fold_guarded(wc);
        } else {
            load_full(wa, 0);
            int64_t k = 0;
            for (; k + 2 < nfull; k += 2) {
                load_full(wb, k + 1);
                if (TOK && k == 0) fetch_target();
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
            if (rem > 0) fold_guarded(wc);
        }
    }
    if (TOK && nfull < 3) fetch_target();

    if (has_head || has_tail) fold<2>(a, ends);

    // Merge the lanes (one barrier), then across parts for a split row.
    Merged b = block_merge<BLOCK>(a.m, a.c, acc_sum(a), pairs);

    if constexpr (SPLIT) {
        // Merge across the row's parts in the same launch. Each part's
        // workgroup publishes its (max, sum) as one 64-bit word in the row's
        // slot for that part and counts itself in on the row's counter; the
        // part that counts last merges. Slots hold 0 between launches (the
        // workspace is cleared when it is made, and every launch clears what
        // it used), and no pair is 0: a sum of 0 goes with a maximum of -inf.
        //
        // What this relies on is the gfx942/gfx950 memory model at agent
        // scope: atomic loads, stores and read-modify-writes at agent scope
        // are issued with the sc1 bit and performed at the point of
        // coherence of all the device's L2s, and an aligned 64-bit access is
        // single-copy atomic. So a slot read at agent scope holds either 0
        // or the whole pair its part wrote in this launch. The counter only
        // tells the last part that every part has issued its store, not that
        // the store has been performed (no part waits for its store before
        // counting in: that wait was a memory round trip on the critical
        // path of every split row), so the last part reads each slot until
        // it is not 0. Each slot is cleared by the lane that read it (or, for
        // the last part's own slot, by the thread that wrote it), so that in
        // each slot's modification order the clearing store follows the pair,
        // as it does for the counter, whose clearing follows the last add.
        unsigned long long* slots = reinterpret_cast<unsigned long long*>(ws_pairs) + row * nparts;
        const unsigned long long mine =
            (static_cast<unsigned long long>(__float_as_uint(b.s)) << 32) | __float_as_uint(b.m);
        if (tid == 0) {
            __hip_atomic_store(slots + part, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const unsigned prev = __hip_atomic_fetch_add(counters + row * kCounterWords, 1u,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            is_last = (prev == static_cast<unsigned>(nparts - 1));
        }
        __syncthreads();
        if (!is_last) return;
        const bool other = tid < nparts && tid != part;
        unsigned long long v = tid == part ? mine : 0ull;
        if (other) {
            // A pair's store was issued before its part counted in, so it
            // lands within a memory round trip or so; the bound only makes
            // the wait finite by construction. A slot still empty after it
            // (which the protocol rules out) makes the row's result NaN
            // rather than a silently wrong number.
            for (int i = 0; v == 0 && i < kSplitSpinLimit; ++i)
                v = __hip_atomic_load(slots + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (v == 0) v = 0x7FC000007FC00000ull;  // (NaN, NaN)
        }
        float pm = -kInf, ps = 0.0f;
        if (tid < nparts) {
            pm = __uint_as_float(static_cast<unsigned>(v));
            ps = __uint_as_float(static_cast<unsigned>(v >> 32));
        }
        b = block_merge<BLOCK>(pm, base2_ref(pm), ps, pairs);
        if (other) __hip_atomic_store(slots + tid, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tid == 0) {
            __hip_atomic_store(slots + part, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(counters + row * kCounterWords, 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    float r;
    if (needs_natural_units(b.m, b.s)) {  // uniform: b is the same in every thread
        __syncthreads();                    // `pairs` readers are done before scratch reuse
        float s2 = natural_units_sum<D>(rp, cols, b.m, tid, BLOCK);
        s2 = block_reduce<BLOCK>(s2, OpSum{}, pairs);
        r = __builtin_fmaf(log2_hw(s2), kLn2, b.m);
    } else {
        r = finish(b.m, b.c, b.s);
    }
    if (tid == 0) {
        if (!TOK || out != nullptr) out[row] = r;
        if constexpr (TOK) {
            float x_t;
            if constexpr (D == DType::F32)
                x_t = __uint_as_float(t_word);
            else
                x_t = word_half_to_float<D>(t_word, t_hi);
            logp[row] = t_ok ? x_t - r : __builtin_nanf("");
        }
    }
}

// ---------------------------------------------------------------------------
// Dispatch from a host launch plan to a template instance.

namespace {

template <DType D, int G, int VPL, bool VEC, bool TAIL, int ROUNDS>
hipError_t launch_regs_tok(const LaunchArgs& a) {
    if (a.targets != nullptr)
        hipLaunchKernelGGL((rows_in_registers<D, G, VPL, VEC, TAIL, ROUNDS, true>), dim3(a.grid),
                           dim3(256), 0, a.stream, a.x, a.rows, a.cols, a.stride_bytes, a.out,
                           a.targets, a.logp);
    else
        hipLaunchKernelGGL((rows_in_registers<D, G, VPL, VEC, TAIL, ROUNDS, false>), dim3(a.grid),
                           dim3(256), 0, a.stream, a.x, a.rows, a.cols, a.stride_bytes, a.out,
                           nullptr, nullptr);
    return hipGetLastError();
}

template <DType D, int G, int VPL, bool VEC>
hipError_t launch_regs(const LaunchArgs& a) {
    // More rounds in flight when each lane's share of a row is small.
    constexpr int ROUNDS = VPL == 1 ? 4 : (VPL == 2 ? 2 : 1);
    if (a.rows_per_wave != (64 / G) * ROUNDS) return hipErrorInvalidConfiguration;
    const int k = VEC ? (a.dtype == LSE_DTYPE_F32 ? 4 : 8) : 1;
    const bool tail = a.cols % k != 0;
    if (tail) return launch_regs_tok<D, G, VPL, VEC, VEC, ROUNDS>(a);
    return launch_regs_tok<D, G, VPL, VEC, false, ROUNDS>(a);
}

// Instances: VPL 1, 2, 4 for G = 1, 2, 4 and 64 (G = 64 also holds scalar rows
// of up to 1024 elements with VPL 8 and 16), VPL 1 for G = 8, 16, 32.
template <DType D, int G, bool VEC>
hipError_t launch_regs_vpl(const LaunchArgs& a) {
    constexpr bool kWide = G <= 4 || G == 64;
    switch (a.loads_per_lane) {
        case 1: return launch_regs<D, G, 1, VEC>(a);
        case 2: if constexpr (kWide) return launch_regs<D, G, 2, VEC>(a); break;
        case 4: if constexpr (kWide) return launch_regs<D, G, 4, VEC>(a); break;
        case 8: if constexpr (G == 64 && !VEC) return launch_regs<D, G, 8, VEC>(a); break;
        case 16: if constexpr (G == 64 && !VEC) return launch_regs<D, G, 16, VEC>(a); break;
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
    if (a.targets != nullptr)
        hipLaunchKernelGGL((stream_rows<D, BLOCK, U, SPLIT, true>), dim3(a.grid), dim3(BLOCK), 0,
                           a.stream, a.x, a.cols, a.stride_bytes, a.out, a.parts,
                           a.ws_pairs, a.counters, a.targets, a.logp);
    else
        hipLaunchKernelGGL((stream_rows<D, BLOCK, U, SPLIT, false>), dim3(a.grid), dim3(BLOCK), 0,
                           a.stream, a.x, a.cols, a.stride_bytes, a.out, a.parts,
                           a.ws_pairs, a.counters, nullptr, nullptr);
    return hipGetLastError();
}

template <DType D, bool SPLIT>
hipError_t launch_stream_cfg(const LaunchArgs& a) {
    const int key = a.block * 100 + a.unroll;
    switch (key) {
        case 6404: return launch_stream<D, 64, 4, SPLIT>(a);
        case 6408: return launch_stream<D, 64, 8, SPLIT>(a);
        case 12804: return launch_stream<D, 128, 4, SPLIT>(a);
        case 12808: return launch_stream<D, 128, 8, SPLIT>(a);
        case 25604: return launch_stream<D, 256, 4, SPLIT>(a);
        case 25608: return launch_stream<D, 256, 8, SPLIT>(a);
        case 51204: return launch_stream<D, 512, 4, SPLIT>(a);
        case 51208: return launch_stream<D, 512, 8, SPLIT>(a);
        case 102404: return launch_stream<D, 1024, 4, SPLIT>(a);
        case 102408: return launch_stream<D, 1024, 8, SPLIT>(a);
    }
    return hipErrorInvalidConfiguration;
}

}  // namespace

// The launch of one plan for element type D (instantiated per element type).
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

}  // namespace lse
