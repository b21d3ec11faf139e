// lse_dim.hip - log-sum-exp over the middle axis of a contiguous
// [outer, n, inner] array, for gfx950:
//
//     out[o * inner + i] = log( sum_j exp(x[(o * n + j) * inner + i]) ),
//
// torch.logsumexp(x, dim=d) for a contiguous x (outer = prod(shape[:d]),
// n = shape[d], inner = prod(shape[d+1:])). The paper "Speeding up
// Log-Sum-Exp: Kernel Fusion at the Memory Wall, Integer Arithmetic at the
// Compute Wall" presents its kernels as drop-in replacements for
// torch.logsumexp (abstract, §6); this covers the reduction axes other than
// the last (inner == 1 is lse_forward). Same arithmetic as the row kernels:
// each element read once, a per-lane (max, exp-sum) accumulator folded lazily
// (fold_lazy_terms), pairwise merges, one fp32 per output.
//
// Layout. The reduced elements of one output are inner elements apart, and
// neighbouring outputs are neighbours in memory. A lane owns K adjacent
// outputs (a 16-byte group of columns when inner is a multiple of K and x is
// 16-byte aligned, else one column) and walks j, loading 16 bytes per step;
// no lane talks to another while streaming. The workgroup's 256 lanes cover
// a block of gw column groups x rw = 256 / gw steps of j. The planner takes
// gw = 32 or 64 (a load step reads rw pieces of 512 or 1024 bytes), or the
// whole row (gw = inner / K) when it is shorter, so that rw consecutive rows,
// again contiguous, are read at once (inner = 16 fp32: 64 rows of 64 bytes).
// The lanes that share columns are merged through LDS at the end. When there
// are too few column blocks (tiles) to fill the GPU, P workgroups split j and
// write their (max, sum) pairs to the handle's workspace; the last of a
// tile's P workgroups to arrive (an agent-scope counter per tile) merges the
// tile's pairs in the same launch and resets the counter.
//
// The file also holds the backward pass over the same axis: lse_grad_cols
// (the same tiles, one load and one store per step, nothing merged) and
// lse_grad_flat (lanes own 16-byte vectors of the flat array, for widths that
// do not fit the tiles' 16-byte column groups, and for fp32).
#include "lse_device.h"
#include "lse_launch.h"

namespace lse {

template <DType D, bool VEC, int U, bool SPLIT>
__global__ __launch_bounds__(256) void lse_cols(const char* __restrict__ x, int64_t n,
                                                int64_t inner, int64_t ncv, int gw, int64_t tile0,
                                                float* __restrict__ out, int parts,
                                                unsigned* __restrict__ ws_pairs,
                                                unsigned* __restrict__ counters, int xcd_runs) {
    constexpr int K = VEC ? Elem<D>::kPerVec : 1;
    constexpr int EB = Elem<D>::kBytes;
    __shared__ float lds_m[256 * K];
    __shared__ float lds_s[256 * K];

    const int t = threadIdx.x;
    const int rw = 256 / gw;             // steps of j per load
    const int col = t % gw;
    const int jr = t / gw;               // this lane's step within a load
    const bool active = jr < rw;         // lanes past rw * gw hold nothing
    // Workgroups go to the XCDs in turn (b mod 8), and each XCD has its own
    // L2. When a tile's pieces of a row do not start on 128-byte lines (the
    // one-column path, or a row pitch or base that is not a multiple of 128
    // bytes), neighbouring tiles share lines, and spread over the XCDs each
    // such line is fetched once per XCD that needs it. With xcd_runs (the
    // host's choice for those layouts) each XCD takes a contiguous run of the
    // launch's (tile, part) pairs instead, so that neighbours share an L2.
    // (32-bit arithmetic: the grid is below 2^31 workgroups, and a 64-bit
    // division here delayed every workgroup's first loads.)
    unsigned wgi = blockIdx.x;
    if (xcd_runs) {
        const unsigned b = blockIdx.x, q = gridDim.x / 8, r = gridDim.x % 8, xcd = b % 8;
        wgi = xcd * q + (xcd < r ? xcd : r) + b / 8;
    }
    const unsigned tlu = wgi / static_cast<unsigned>(parts);
    const int64_t tl = tlu;
    const int part = static_cast<int>(wgi - tlu * static_cast<unsigned>(parts));
    // The index arithmetic is 32-bit wherever the sizes allow (n < 2^31 by the
    // entry point's contract; column groups below 2^32 unless the array is
    // larger than that): 64-bit divisions, one per lane for the column, took
    // about a thousand instructions before the first load.
    const int64_t cvs = VEC ? inner / K : inner;  // column groups per outer slice
    const int64_t cv_raw = (tile0 + tl) * gw + col;
    const int64_t cv = cv_raw < ncv ? cv_raw : ncv - 1;  // past the end: read a real column
    int64_t o, iv;
    if (ncv <= 0xFFFFFFFFll) {
        const unsigned c = static_cast<unsigned>(cv), cs = static_cast<unsigned>(cvs);
        const unsigned oo = c / cs;
        o = oo;
        iv = c - oo * cs;
    } else {
        o = cv / cvs;
        iv = cv - o * cvs;
    }
    const char* base = x + (o * n * inner + iv * K) * EB;  // element (o, 0, iv*K)
    const int64_t jstride = inner * EB;

    // This part's j range, [n * part / parts, n * (part + 1) / parts), in
    // 32-bit terms: with n = q * parts + r, n * p / parts = q * p + r * p / parts
    // (r * p < parts^2 <= 2^20). The lane takes j = pj0 + jr + s * rw.
    const unsigned nu = static_cast<unsigned>(n), pu = static_cast<unsigned>(parts);
    const unsigned qn = nu / pu, rn = nu - qn * pu;
    const unsigned partu = static_cast<unsigned>(part);
    const int64_t pj0 = qn * partu + rn * partu / pu;
    const int64_t pj1 = qn * (partu + 1) + rn * (partu + 1) / pu;
    const unsigned lenu = static_cast<unsigned>(pj1 - pj0);
    const int64_t len = lenu;
    const int64_t full_steps = lenu / static_cast<unsigned>(rw);   // every lane's j is in range
    const int64_t steps = (lenu + rw - 1) / static_cast<unsigned>(rw);  // the last may be partial
    const int64_t nfull = full_steps / U;            // whole batches of U steps
    const int64_t rem = steps - nfull * U;           // steps in the guarded batch

    Acc a[K];
#pragma unroll
    for (int k = 0; k < K; ++k) a[k] = acc_empty();

    struct Batch {
        u32x4 w[VEC ? U : 1];
        float e[VEC ? 1 : U];
    };
    auto load_at = [&](Batch& b, int u, int64_t j) {
        const char* p = base + j * jstride;
        if constexpr (VEC)
            b.w[u] = load_vec(reinterpret_cast<const u32x4*>(p));
        else
            b.e[u] = load_scalar<D>(p);
    };
    auto load_full = [&](Batch& b, int64_t kb) {
#pragma unroll
        for (int u = 0; u < U; ++u) load_at(b, u, pj0 + jr + (kb * U + u) * rw);
        __builtin_amdgcn_sched_barrier(0);
    };
    // The guarded batch: steps nfull*U .. steps-1; a step past this lane's
    // range reloads the part's last row (in bounds) and is masked to -inf.
    auto load_guarded = [&](Batch& b) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = pj0 + jr + (nfull * U + u) * rw;
            load_at(b, u, j < pj1 ? j : pj1 - 1);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // Each column's U steps fold lazily, with the terms taken step by step: a
    // step's K exponentials depend only on that step's load and the columns'
    // references, so they start as soon as the load has returned, and the
    // arithmetic overlaps the later steps' loads. The per-column sums (the
    // tree of sum_exp_of<U>) and lazy tests follow the last step.
    auto fold_batch = [&](const Batch& b, bool guarded) {
        float f[U][K], e[U][K];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (VEC)
                decode<D>(b.w[u], f[u]);
            else
                f[u][0] = b.e[u];
            if (guarded && !(u < rem && pj0 + jr + (nfull * U + u) * rw < pj1)) {
#pragma unroll
                for (int k = 0; k < K; ++k) f[u][k] = -kInf;
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
                e[u][k] = exp2_hw(__builtin_fmaf(f[u][k], kLog2e, -a[k].c));
                // Ordered empty asm pins the step's terms here: otherwise the
                // compiler moves each term next to its column's sum, and the
                // first column's sum waits for every step's load.
                asm volatile("" : "+v"(e[u][k]));
            }
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float g[U], h[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                g[u] = f[u][k];
                h[u] = e[u][k];
            }
            fold_lazy_terms<U>(a[k], g, tree_sum<U>(h));
        }
    };

    if (len > 0 && active) {
        Batch ba, bb, bc;
        if (nfull == 0) {
            load_guarded(bc);
            fold_batch(bc, true);
        } else {
            load_full(ba, 0);
            int64_t kb = 0;
            for (; kb + 2 < nfull; kb += 2) {
                load_full(bb, kb + 1);
                fold_batch(ba, false);
                load_full(ba, kb + 2);
                fold_batch(bb, false);
            }
            if (kb + 1 < nfull) {
                load_full(bb, kb + 1);
                load_guarded(bc);
                fold_batch(ba, false);
                fold_batch(bb, false);
            } else {
                load_guarded(bc);
                fold_batch(ba, false);
            }
            if (rem > 0) fold_batch(bc, true);
        }
    }

    // The tile's pairs from all parts, entry q = col * K + k: L lanes per
    // entry (a power of two, L * entries <= 256, L <= 64) take parts l,
    // l + L, ..., and their partial (max, sum) meet in LDS. A merged maximum
    // beyond +-2^30 sums the column's j again, over the same L lanes.
    auto merge_parts = [&](int64_t tlm) {
        const int ent = gw * K;
        const int64_t entries = static_cast<int64_t>(gridDim.x / parts) * ent;
        const unsigned long long* wp = reinterpret_cast<const unsigned long long*>(ws_pairs);
        int L = 1;
        while (L < 64 && 2 * L * ent <= 256) L *= 2;
        const int l = t & (L - 1);
        for (int q0 = 0; q0 < ent; q0 += 256 / L) {
            const int q = q0 + t / L;
            const int c = q / K;
            const int k = q - c * K;
            const int64_t qcv = (tile0 + tlm) * gw + c;
            const bool live = q < ent && qcv < ncv;
            // This lane's parts in batches of 8 loads issued together; each
            // batch raises the running maximum and rescales the sum (and its
            // compensation) once.
            float pm = -kInf;
            CSum cps;
            if (live) {
                const unsigned long long* e0 = wp + tlm * ent + q;
                for (int p0 = l; p0 < parts; p0 += 8 * L) {
                    float bm[8], bs[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int p = p0 + i * L;
                        const unsigned long long v =
                            p < parts ? __hip_atomic_load(e0 + p * entries, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT)
                                      : 0xFF800000ull;  // (-inf, 0)
                        bm[i] = __uint_as_float(static_cast<unsigned>(v));
                        bs[i] = __uint_as_float(static_cast<unsigned>(v >> 32));
                    }
                    float m2 = pm;
#pragma unroll
                    for (int i = 0; i < 8; ++i) m2 = max3f(m2, bm[i], m2);
                    const float c2 = base2_ref(m2);
                    const float r = exp2_hw(base2_ref(pm) - c2);
                    cps.s *= r;
                    cps.e *= r;
#pragma unroll
                    for (int i = 0; i < 8; ++i) cps.add(bs[i] * exp2_hw(base2_ref(bm[i]) - c2));
                    pm = m2;
                }
            }
            lds_m[t] = pm;
            lds_s[t] = cps.total();
            __syncthreads();
            const int g0 = t - l;  // the entry's first lane
            float m = -kInf;
            for (int i = 0; i < L; ++i) m = max3f(m, lds_m[g0 + i], m);
            const float cm = base2_ref(m);
            CSum cs;
            for (int i = 0; i < L; ++i) cs.add(lds_s[g0 + i] * exp2_hw(base2_ref(lds_m[g0 + i]) - cm));
            const float sum = cs.total();
            const bool slow = live && needs_natural_units(m, sum);
            const int64_t qo = live ? qcv / cvs : 0;
            const int64_t qi = qcv - qo * cvs;
            float s2 = 0.0f;
            if (slow) {
                const char* p = x + (qo * n * inner + qi * K + k) * EB;
                for (int64_t j = l; j < n; j += L)
                    s2 += exp2_hw((load_scalar<D>(p + j * jstride) - m) * kLog2e);
            }
            __syncthreads();  // every lane has read the partials
            lds_s[t] = s2;
            __syncthreads();
            if (live && l == 0) {
                float r;
                if (slow) {
                    float t2 = 0.0f;
                    for (int i = 0; i < L; ++i) t2 += lds_s[g0 + i];
                    r = __builtin_fmaf(log2_hw(t2), kLn2, m);
                } else {
                    r = finish(m, cm, sum);
                }
                out[qo * inner + qi * K + k] = r;
            }
            __syncthreads();
        }
    };

    // Merge the rw lanes of each column through LDS: entry q = col * K + k of
    // this tile collects the pairs (jr, col, k) for jr < rw. Narrow tiles have
    // few entries and many steps each (gw = 1: 256 steps), so where rw >= 32,
    // L lanes share an entry (the largest power of two with L * L <= rw and
    // L * entries <= 256): each merges every L-th step, and the entry's first
    // lane merges their L partials, about 2 sqrt(rw) steps in a row instead of
    // rw. Measured as library copies (medians of six alternating blocks), over
    // the first axis: bf16 [1000000, 8] 33.0 -> 17.8 us, fp32 [1000000, 4]
    // 33.0 -> 17.9, fp32 [1000000, 8] 23.7 -> 17.2, fp32 [262144, 16] 17.7 ->
    // 14.9, fp32 [16777216, 16] 160.4 -> 157.5. Wider tiles (rw <= 16, L = 1) merge each
    // entry in one lane, as the extra barriers cost more than they save there.
#pragma unroll
    for (int k = 0; k < K; ++k) {
        lds_m[t * K + k] = active ? a[k].m : -kInf;
        lds_s[t * K + k] = active ? acc_sum(a[k]) : 0.0f;
    }
    __syncthreads();
    const int ent = gw * K;
    auto merge_steps = [&](int q, int r0, int dr, float& m, float& s) {
        const int c = q / K;
        const int k = q - c * K;
        m = -kInf;
        for (int r = r0; r < rw; r += dr) m = max3f(m, lds_m[(r * gw + c) * K + k], m);
        const float cm = base2_ref(m);
        CSum cs;
        for (int r = r0; r < rw; r += dr) {
            const int i = (r * gw + c) * K + k;
            cs.add(lds_s[i] * exp2_hw(base2_ref(lds_m[i]) - cm));
        }
        s = cs.total();
    };
    auto entry_out = [&](int q, float m, float s) {
        const int c = q / K;
        const int k = q - c * K;
        const float cm = base2_ref(m);
        const int64_t qcv = (tile0 + tl) * gw + c;
        if (qcv >= ncv) return;
        if constexpr (SPLIT) {
            // Part-major (consecutive lanes write consecutive pairs), one
            // agent-scope 8-byte store per pair: coherent across the XCDs'
            // L2s, so the merging workgroup reads it wherever it runs.
            const int64_t entries = static_cast<int64_t>(gridDim.x / parts) * gw * K;
            const unsigned long long pair =
                (static_cast<unsigned long long>(__float_as_uint(s)) << 32) | __float_as_uint(m);
            __hip_atomic_store(reinterpret_cast<unsigned long long*>(ws_pairs) +
                                   (part * entries + tl * gw * K + q),
                               pair, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            const int64_t qo = qcv / cvs;
            const int64_t qi = qcv - qo * cvs;
            float r;
            if (needs_natural_units(m, s)) {  // maximum beyond +-2^30: all of j again
                const char* p = x + (qo * n * inner + qi * K + k) * EB;
                float s2 = 0.0f;
                for (int64_t j = 0; j < n; ++j)
                    s2 += exp2_hw((load_scalar<D>(p + j * jstride) - m) * kLog2e);
                r = __builtin_fmaf(log2_hw(s2), kLn2, m);
            } else {
                r = finish(m, cm, s);
            }
            out[qo * inner + qi * K + k] = r;
        }
    };
    int L = 1;
    if (rw >= 32)
        while (L < 64 && 2 * L * ent <= 256 && 4 * L * L <= rw) L *= 2;
    if (L > 1) {
        const int q = t / L;
        const int l = t - q * L;
        float pm = -kInf, ps = 0.0f;
        if (q < ent) merge_steps(q, l, L, pm, ps);
        __syncthreads();  // every lane has read the step pairs
        lds_m[t] = pm;
        lds_s[t] = ps;
        __syncthreads();
        if (q < ent && l == 0) {
            float m = -kInf;
            for (int i = 0; i < L; ++i) m = max3f(m, lds_m[t + i], m);
            const float cm = base2_ref(m);
            CSum cs;
            for (int i = 0; i < L; ++i) cs.add(lds_s[t + i] * exp2_hw(base2_ref(lds_m[t + i]) - cm));
            entry_out(q, m, cs.total());
        }
    } else {
        for (int q = t; q < ent; q += 256) {
            float m, s;
            merge_steps(q, 0, 1, m, s);
            entry_out(q, m, s);
        }
    }

    if constexpr (SPLIT) {
        // Count this workgroup in once every lane's pair stores have
        // completed; the last of the tile's parts to arrive merges them. In
        // the gfx942/gfx950 memory model, atomic loads and stores at agent
        // scope are issued with the sc1 bit and performed at the point of
        // coherence of all the device's L2s, and atomic read-modify-writes
        // at agent scope are coherent across them: s_waitcnt vmcnt(0) has
        // the pairs there before the counter add issues, and the merging
        // part's loads issue after its add has returned.
        __shared__ int is_last;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __syncthreads();
        if (t == 0) {
            const unsigned prev = __hip_atomic_fetch_add(counters + tl * kCounterWords, 1u,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            is_last = prev == static_cast<unsigned>(parts - 1);
        }
        __syncthreads();
        if (!is_last) return;
        merge_parts(tl);
        if (t == 0)
            __hip_atomic_store(counters + tl * kCounterWords, 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------------------
// The backward pass over the middle axis,
//
//     grad_x[(o*n + j)*inner + i] = grad_out[o*inner + i]
//                                   * exp(x[(o*n + j)*inner + i] - lse[o*inner + i]),
//
// the gradient of lse_forward_dim's output with respect to x: along j, each
// column's softmax scaled by that column's incoming gradient (the backward
// support the paper lists for its kernels, Table 3, for the torch.logsumexp
// drop-in of the abstract and section 6, whose dim may be any axis). The
// same tiles as lse_cols: a lane owns K adjacent columns (one 16-byte group,
// x and grad_x 16-byte aligned and inner a multiple of K) or one column,
// reads their lse and grad_out once, and walks its part's j with one load
// and one store per step; nothing is merged, so the parts are independent.
// Per element: subtract, scale by log2 e, v_exp_f32, multiply, as the
// row-wise backward pass. Loads past the part's end reload its last row (in
// bounds) and their stores are skipped; lanes past the last column store
// nothing.
template <DType D>
__device__ __forceinline__ u32x4 pack_out(const float* o) {
    if constexpr (D == DType::F32) {
        return u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                     __float_as_uint(o[3])};
    } else {
        typedef float f2 __attribute__((ext_vector_type(2)));
        unsigned p[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if constexpr (D == DType::F16) {
                p[k] = __builtin_bit_cast(unsigned,
                                          __builtin_convertvector(f2{o[2 * k], o[2 * k + 1]}, half2_t));
            } else {
                typedef __bf16 b2 __attribute__((ext_vector_type(2)));
                p[k] = __builtin_bit_cast(unsigned,
                                          __builtin_convertvector(f2{o[2 * k], o[2 * k + 1]}, b2));
            }
        }
        return u32x4{p[0], p[1], p[2], p[3]};
    }
}

template <DType D>
__device__ __forceinline__ void store_elem(char* p, float v) {
    if constexpr (D == DType::F32) {
        __builtin_nontemporal_store(v, reinterpret_cast<float*>(p));
    } else if constexpr (D == DType::BF16) {
        __builtin_nontemporal_store(__builtin_bit_cast(unsigned short, static_cast<__bf16>(v)),
                                    reinterpret_cast<unsigned short*>(p));
    } else {
        __builtin_nontemporal_store(__builtin_bit_cast(unsigned short, static_cast<_Float16>(v)),
                                    reinterpret_cast<unsigned short*>(p));
    }
}

template <DType D, bool VEC, int U>
__global__ __launch_bounds__(256) void lse_grad_cols(const char* __restrict__ x, int64_t n,
                                                     int64_t inner, int64_t ncv, int gw,
                                                     int64_t tile0, int parts,
                                                     const float* __restrict__ lse,
                                                     const float* __restrict__ gout,
                                                     char* __restrict__ gx, int xcd_runs) {
    constexpr int K = VEC ? Elem<D>::kPerVec : 1;
    constexpr int EB = Elem<D>::kBytes;
    const int t = threadIdx.x;
    const int rw = 256 / gw;
    const int col = t % gw;
    const int jr = t / gw;
    unsigned wgi = blockIdx.x;  // as in lse_cols: XCD runs where tiles share lines
    if (xcd_runs) {
        const unsigned b = blockIdx.x, q = gridDim.x / 8, r = gridDim.x % 8, xcd = b % 8;
        wgi = xcd * q + (xcd < r ? xcd : r) + b / 8;
    }
    const unsigned tlu = wgi / static_cast<unsigned>(parts);
    const int part = static_cast<int>(wgi - tlu * static_cast<unsigned>(parts));
    const int64_t cvs = VEC ? inner / K : inner;
    const int64_t cv_raw = (tile0 + static_cast<int64_t>(tlu)) * gw + col;
    const bool live = jr < rw && cv_raw < ncv;
    const int64_t cv = cv_raw < ncv ? cv_raw : ncv - 1;
    int64_t o, iv;
    if (ncv <= 0xFFFFFFFFll) {
        const unsigned c = static_cast<unsigned>(cv), cs = static_cast<unsigned>(cvs);
        const unsigned oo = c / cs;
        o = oo;
        iv = c - oo * cs;
    } else {
        o = cv / cvs;
        iv = cv - o * cvs;
    }
    const int64_t off0 = o * n * inner + iv * K;  // element (o, 0, iv*K)
    const char* xb = x + off0 * EB;
    char* gb = gx + off0 * EB;
    const int64_t jstride = inner * EB;
    float L[K], G[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        L[k] = lse[o * inner + iv * K + k];
        G[k] = gout[o * inner + iv * K + k];
    }
    // this part's j range, as in lse_cols (32-bit: rn * (part + 1) < parts^2
    // <= 2^32 for the at most 65536 parts the planner gives a tile)
    const unsigned nu = static_cast<unsigned>(n), pu = static_cast<unsigned>(parts);
    const unsigned qn = nu / pu, rn = nu - qn * pu;
    const unsigned partu = static_cast<unsigned>(part);
    const int64_t pj0 = qn * partu + rn * partu / pu;
    const int64_t pj1 = qn * (partu + 1) + rn * (partu + 1) / pu;
    if (pj1 <= pj0) return;  // uniform: the part is empty
    const int64_t steps = (pj1 - pj0 + rw - 1) / rw;
    const int64_t nb = (steps + U - 1) / U;

    struct Batch {
        u32x4 w[VEC ? U : 1];
        float e[VEC ? 1 : U];
    };
    auto load = [&](Batch& bt, int64_t kb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = pj0 + jr + (kb * U + u) * rw;
            const char* p = xb + (j < pj1 ? j : pj1 - 1) * jstride;
            if constexpr (VEC)
                bt.w[u] = load_vec(reinterpret_cast<const u32x4*>(p));
            else
                bt.e[u] = load_scalar<D>(p);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto process = [&](const Batch& bt, int64_t kb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = pj0 + jr + (kb * U + u) * rw;
            char* q = gb + j * jstride;
            if constexpr (VEC) {
                float f[K], r[K];
                decode<D>(bt.w[u], f);
#pragma unroll
                for (int k = 0; k < K; ++k) r[k] = G[k] * exp2_hw((f[k] - L[k]) * kLog2e);
                if (live && j < pj1)
                    __builtin_nontemporal_store(pack_out<D>(r), reinterpret_cast<u32x4*>(q));
            } else {
                const float r = G[0] * exp2_hw((bt.e[u] - L[0]) * kLog2e);
                if (live && j < pj1) store_elem<D>(q, r);
            }
        }
    };
    // two batches in flight: the next is loaded before one is computed and stored
    Batch ba, bb;
    load(ba, 0);
    for (int64_t kb = 0; kb < nb; kb += 2) {
        if (kb + 1 < nb) load(bb, kb + 1);
        process(ba, kb);
        if (kb + 1 < nb) {
            if (kb + 2 < nb) load(ba, kb + 2);
            process(bb, kb + 1);
        }
    }
}

// ---------------------------------------------------------------------------
// The same backward pass with lanes that own memory instead of columns. For
// an inner width that is not a multiple of the vector (or a base that is not
// 16-byte aligned) the column tiles above read and write 2- or 4-byte pieces
// whose rows start at every phase of the 128-byte lines, and neighbouring
// tiles write the two halves of a line at different times. Here a workgroup
// takes 4096 consecutive elements of the flat array as 256 * U 16-byte
// vectors (x and grad_x share their phase mod 16; the head and tail elements
// outside whole vectors go one by one), or as single elements where the
// phases differ, and reads and writes them like a copy. It first stages the
// lse and grad_out of its 4096 elements in LDS, slot d for element F + d:
// each slot finds its column i and slice o (exact 32-bit divisions) and
// reads o * inner + i, so consecutive lanes read consecutive addresses
// except where a row wraps. Each lane then takes its K pairs from LDS with
// aligned reads. That is 8 bytes per element read from the caches (lse and
// grad_out, outer * inner * 8 bytes in all, are read again for every j),
// against the column kernel's one read per column; the arithmetic per element
// is the column kernel's, so the results are the same bits. Timed as library
// copies (medians of six alternating blocks, over the first axis, against
// the column kernel and a copy kernel moving the same bytes): fp32 [65536,
// 4097] 1316 -> 364 us (copy 349), fp32 [2048, 30001] 223 -> 85 (81), fp32
// [8, 25000001] 1211 -> 430 (299), bf16 [65536, 4097] 675 -> 280 (172), bf16
// [512, 50257] 48.5 -> 28.0 (18.2), bf16 [1000000, 7] 14.3 -> 11.7 (6.4); on
// aligned widths fp32 [65536, 4096] 417 -> 359 (350), fp32 [16777216, 16]
// 357 -> 341 (348) and fp32 [2048, 30000] 100 -> 85 (79), but fp32 [16,
// 4000000] (32 MB of lse and grad_out, read 16 times) 98 -> 135 and 16-bit
// types, whose elements carry half the bytes, bf16 [512, 128256] 49 -> 69,
// bf16 [65536, 4096] 235 -> 274. Without the staging (K lookups per lane,
// each wave instruction spanning K * 256 bytes) the flat kernel took 491, 113,
// 376 and 41 us on fp32 [65536, 4097], fp32 [2048, 30001], bf16 [65536, 4097]
// and bf16 [512, 50257].

// Exact floor(a / d) for a, d < 2^32, from m = floor((2^64 - 1) / d) + 1: the
// high 64 bits of m * a (Lemire, Kaser and Kurz, "Faster Remainder by Direct
// Computation", 2019). d = 1 would need m = 2^64; callers pass m = 0 for it.
__device__ __forceinline__ unsigned fastdiv(unsigned a, uint64_t m) {
    return m ? static_cast<unsigned>(__umul64hi(m, static_cast<uint64_t>(a))) : a;
}

template <DType D, bool VEC, int U>
__global__ __launch_bounds__(256) void lse_grad_flat(const char* __restrict__ x,
                                                     char* __restrict__ gx,
                                                     const float* __restrict__ lse,
                                                     const float* __restrict__ gout, int64_t n,
                                                     int64_t inner, int64_t total, int64_t head,
                                                     int64_t nvec, uint64_t m_inner,
                                                     uint64_t m_n) {
    constexpr int K = VEC ? Elem<D>::kPerVec : 1;
    constexpr int EB = Elem<D>::kBytes;
    constexpr int CH = 256 * U * K;  // elements per workgroup
    __shared__ float sl[CH];
    __shared__ float sg[CH];
    const int t = threadIdx.x;
    const int64_t v0 = static_cast<int64_t>(blockIdx.x) * (256 * U);

    // One element, located with 64-bit divisions: the head and tail.
    auto one = [&](int64_t f) {
        const int64_t q = f / inner;
        const int64_t i = f - q * inner;
        const int64_t g = (q / n) * inner + i;
        const float v = load_scalar<D>(x + f * EB);
        store_elem<D>(gx + f * EB, gout[g] * exp2_hw((v - lse[g]) * kLog2e));
    };
    if constexpr (VEC) {
        const int64_t tail0 = head + nvec * K;
        if (blockIdx.x == 0 && t < head + (total - tail0))
            one(t < head ? t : tail0 + (t - head));
    }
    if (v0 >= nvec) return;  // uniform: no whole vectors here

    // x's loads go first, ahead of the 64-bit divisions below (measured as
    // library copies against the other order: fp32 [65536, 4096] over its
    // first axis 357 -> 349 us, fp32 [65536, 4097] 362 -> 353, bf16 [65536,
    // 4097] 275 -> 266; bf16 [512, 50257] 27.4 -> 28.2).
    u32x4 w[VEC ? U : 1];
    float e[VEC ? 1 : U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + u * 256 + t;
        const int64_t vv = v < nvec ? v : nvec - 1;  // past the end: reload the last vector
        const char* p = x + (head + vv * K) * EB;
        if constexpr (VEC)
            w[u] = load_vec(reinterpret_cast<const u32x4*>(p));
        else
            e[u] = load_scalar<D>(p);
    }

    // (o, j, i) of the workgroup's first element, once per workgroup (64-bit
    // divisions), then the lookup index o * inner + i of each slot d, element
    // F + d. Where inner > CH the slots wrap at most once: to column 0 of the
    // next row of the same slice (inner back), or, from the slice's last row,
    // of the next slice (no jump). Else slot m * 256 + t steps its column and
    // row by 256 elements at a time from one exact 32-bit division, and the
    // slice is a second division unless the array has one slice. For 16-bit
    // elements the slots' arithmetic is a large share of the work: dividing
    // each slot by inner and n took bf16 [65536, 4097] over its first axis
    // 279 us against 241, bf16 [512, 50257] 28.6 against 25.0, f16 [16384,
    // 4097] 69.6 against 60.6, f16 [8192, 2049] 18.8 against 17.6 (library
    // copies; fp32 within 1 %).
    const int64_t F = head + v0 * K;
    const int64_t qF = F / inner;
    const int64_t iF = F - qF * inner;
    const int64_t oF = qF / n;
    const unsigned jF = static_cast<unsigned>(qF - oF * n);

    // Stage lse and grad_out of the chunk's elements in LDS, slot d for
    // element F + d: consecutive lanes take consecutive slots, so each load
    // instruction reads a contiguous run (broken only where a row wraps).
    const int64_t left = total - F;
    constexpr int M = CH / 256;
    int64_t gs[M];
    if (inner > CH) {
        const int64_t gF = oF * inner + iF;
        const bool last_row = jF + 1 == static_cast<unsigned>(n);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int d = m * 256 + t;
            const bool wrap = iF + d >= inner;
            gs[m] = d < left ? gF + d - (wrap && !last_row ? inner : 0) : 0;
        }
    } else {
        const unsigned in32 = static_cast<unsigned>(inner);
        const unsigned a0 = static_cast<unsigned>(iF) + static_cast<unsigned>(t);
        unsigned q = fastdiv(a0, m_inner);  // rows past F's row
        unsigned i = a0 - q * in32;         // column
        const unsigned q256 = fastdiv(256u, m_inner);
        const unsigned r256 = 256u - q256 * in32;
        const bool one_slice = total == n * inner;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            if (m > 0) {
                i += r256;
                q += q256;
                const bool c = i >= in32;
                i = c ? i - in32 : i;
                q = c ? q + 1 : q;
            }
            const unsigned b = one_slice ? 0u : fastdiv(jF + q, m_n);  // slices past F's
            const int d = m * 256 + t;
            gs[m] = d < left ? (oF + b) * inner + i : 0;
        }
    }
    float ls[M], os[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        ls[m] = lse[gs[m]];
        os[m] = gout[gs[m]];
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        sl[m * 256 + t] = ls[m];
        sg[m * 256 + t] = os[m];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + u * 256 + t;
        if (v >= nvec) continue;
        const int d0 = (u * 256 + t) * K;
        char* q = gx + (head + v * K) * EB;
        if constexpr (VEC) {
            float f[K], r[K];
            decode<D>(w[u], f);
#pragma unroll
            for (int k = 0; k < K; ++k) r[k] = sg[d0 + k] * exp2_hw((f[k] - sl[d0 + k]) * kLog2e);
            __builtin_nontemporal_store(pack_out<D>(r), reinterpret_cast<u32x4*>(q));
        } else {
            store_elem<D>(q, sg[d0] * exp2_hw((e[u] - sl[d0]) * kLog2e));
        }
    }
}

namespace {

// Steps of j per batch: 4 16-byte loads per lane on the vector path; on the
// one-column path, whose 2- and 4-byte loads keep few bytes in flight, 8 for
// 16-bit elements (4 for fp32) when j is not split and twice that when it is
// (a split launch has about one or two workgroups per CU). Measured as
// library copies, medians of six alternating blocks, over the first axis:
// unsplit, 16-bit at 8 against 4: bf16 [512, 50257] 20.7 -> 15.4 us, [2048,
// 50257] 71.7 -> 49.4 (fp32 moved by -18 to +5 % at 8, the vector path by +1
// to +6 %); split, 16 and 8 against 8 and 4: bf16 [65536, 4097] 315 -> 259,
// fp32 [65536, 4097] 378 -> 334, fp32 [4096, 4097] 28.8 -> 25.5, bf16
// [1000000, 7] 17.1 -> 15.7, bf16 [256, 1001] (one batch per lane) 7.3 -> 7.6.
template <DType D, bool VEC>
hipError_t launch_cols_d(const DimArgs& a) {
    constexpr int U = VEC || Elem<D>::kBytes == 4 ? 4 : 8;
    constexpr int US = VEC ? 4 : 2 * U;  // split launches
    if (a.parts == 1)
        hipLaunchKernelGGL((lse_cols<D, VEC, U, false>), dim3(a.grid), dim3(256), 0, a.stream, a.x,
                           a.n, a.inner, a.ncv, a.gw, a.tile0, a.out, 1, a.ws_pairs, a.counters,
                           a.xcd_runs ? 1 : 0);
    else
        hipLaunchKernelGGL((lse_cols<D, VEC, US, true>), dim3(a.grid), dim3(256), 0, a.stream, a.x,
                           a.n, a.inner, a.ncv, a.gw, a.tile0, a.out, a.parts, a.ws_pairs,
                           a.counters, a.xcd_runs ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

template <DType D, bool VEC>
hipError_t launch_grad_cols_d(const DimGradArgs& a) {
    hipLaunchKernelGGL((lse_grad_cols<D, VEC, 4>), dim3(a.grid), dim3(256), 0, a.stream, a.x, a.n,
                       a.inner, a.ncv, a.gw, a.tile0, a.parts, a.lse, a.grad_out, a.grad_x,
                       a.xcd_runs ? 1 : 0);
    return hipGetLastError();
}

template <DType D, bool VEC>
hipError_t launch_grad_flat_d(const DimFlatArgs& a) {
    constexpr int U = 16 / (VEC ? Elem<D>::kPerVec : 1);  // 4096 elements per workgroup
    const int64_t grid = a.nvec > 0 ? (a.nvec + 256 * U - 1) / (256 * U) : 1;
    if (grid > INT32_MAX) return hipErrorInvalidValue;  // 2^43 elements: beyond any device
    hipLaunchKernelGGL((lse_grad_flat<D, VEC, U>), dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                       a.stream, a.x, a.grad_x, a.lse, a.grad_out, a.n, a.inner, a.total, a.head,
                       a.nvec, a.m_inner, a.m_n);
    return hipGetLastError();
}

hipError_t launch_grad_flat(const DimFlatArgs& a) {
    if (a.total <= 0) return hipSuccess;
    switch (a.dtype) {
        case LSE_DTYPE_F32:
            return a.vec ? launch_grad_flat_d<DType::F32, true>(a)
                         : launch_grad_flat_d<DType::F32, false>(a);
        case LSE_DTYPE_BF16:
            return a.vec ? launch_grad_flat_d<DType::BF16, true>(a)
                         : launch_grad_flat_d<DType::BF16, false>(a);
        case LSE_DTYPE_F16:
            return a.vec ? launch_grad_flat_d<DType::F16, true>(a)
                         : launch_grad_flat_d<DType::F16, false>(a);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_grad_cols(const DimGradArgs& a) {
    if (a.grid <= 0) return hipSuccess;
    switch (a.dtype) {
        case LSE_DTYPE_F32:
            return a.vector_cols ? launch_grad_cols_d<DType::F32, true>(a)
                                 : launch_grad_cols_d<DType::F32, false>(a);
        case LSE_DTYPE_BF16:
            return a.vector_cols ? launch_grad_cols_d<DType::BF16, true>(a)
                                 : launch_grad_cols_d<DType::BF16, false>(a);
        case LSE_DTYPE_F16:
            return a.vector_cols ? launch_grad_cols_d<DType::F16, true>(a)
                                 : launch_grad_cols_d<DType::F16, false>(a);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_cols(const DimArgs& a) {
    if (a.grid <= 0) return hipSuccess;
    switch (a.dtype) {
        case LSE_DTYPE_F32:
            return a.vector_cols ? launch_cols_d<DType::F32, true>(a)
                                 : launch_cols_d<DType::F32, false>(a);
        case LSE_DTYPE_BF16:
            return a.vector_cols ? launch_cols_d<DType::BF16, true>(a)
                                 : launch_cols_d<DType::BF16, false>(a);
        case LSE_DTYPE_F16:
            return a.vector_cols ? launch_cols_d<DType::F16, true>(a)
                                 : launch_cols_d<DType::F16, false>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace lse
