// lse_backward.hip - the backward pass of the row-wise log-sum-exp for gfx950:
//
//     grad_x[r, j] = grad_out[r] * exp(x[r, j] - lse[r]),
//
// the gradient of lse[r] = LSE(x[r, :]) with respect to x (the row's softmax,
// scaled by the incoming gradient). The paper "Speeding up Log-Sum-Exp: Kernel
// Fusion at the Memory Wall, Integer Arithmetic at the Compute Wall" lists
// backward support among its kernels' properties (Table 3); this is that
// step for the fused forward in lse_kernels.hip. With targets (TOK), the same
// pass is the backward of the token log-probability x[r, t] - lse[r]:
//
//     grad_x[r, j] = grad_logp[r] * ([j == t] - exp(x[r, j] - lse[r])),
//
// computed as (-g) * exp(x - lse), minus (-g) at the target column; a target
// outside [0, cols) makes the row's lse NaN, so the whole row is NaN.
// It is a second streaming pass
// over x that writes as many bytes as it reads, so it is bound by HBM
// bandwidth like the forward pass: 16-byte loads and stores, one per-row
// scalar pair (lse, grad_out), and per element one subtract, one multiply,
// one v_exp_f32 and one multiply.
//
// Work split (planned on the host, lse_api.cpp): the row's units (16-byte
// vectors when every row of x and of grad_x starts 16-byte aligned; also,
// with a per-row head of fewer than K elements peeled off (PEEL), when the
// rows are misaligned alike in x and grad_x, as contiguous rows of an odd
// width are; single elements otherwise) are cut into workgroup items. A long row gives several
// workgroups a contiguous chunk each (R == 1; the row's lse and grad_out are
// uniform and read through the scalar unit); short rows are packed R per
// workgroup, whose lanes walk the R x W units of the block (the row index
// from an exact float reciprocal). All loads and stores of x and grad_x are
// raw buffer operations: a lane past the end gets an offset beyond the
// buffer's range, where loads return zero without touching memory and stores
// are dropped, so every batch issues the same instructions and the hardware
// wait counts stay exact.
#include "lse_device.h"
#include "lse_launch.h"

namespace lse {

namespace {

constexpr unsigned kRsrcWord3 = 0x00020000u;  // raw buffer resource, gfx9 data format
constexpr int kOffFar = 0x7FFFFFF0;            // an offset past any buffer's range

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                             static_cast<int>(bytes), kRsrcWord3);
}

// One unit's grad: g * 2^((x - L) * log2 e) per element, packed back into the
// element type (bf16 rounds to nearest even from fp32). TOK: element tk of the
// unit (if 0 <= tk < K) is the target column and also gets -g.
template <DType D, bool TOK>
__device__ __forceinline__ u32x4 grad_vec(u32x4 w, float lse, float g, int tk) {
    float f[Elem<D>::kPerVec];
    decode<D>(w, f);
    float o[Elem<D>::kPerVec];
#pragma unroll
    for (int k = 0; k < Elem<D>::kPerVec; ++k) {
        o[k] = g * exp2_hw((f[k] - lse) * kLog2e);
        if (TOK && k == tk) o[k] -= g;
    }
    u32x4 r;
    if constexpr (D == DType::F32) {
        r = u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                  __float_as_uint(o[3])};
    } else if constexpr (D == DType::F16) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        unsigned p[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            p[k] = __builtin_bit_cast(unsigned,
                                      __builtin_convertvector(f2{o[2 * k], o[2 * k + 1]}, half2_t));
        r = u32x4{p[0], p[1], p[2], p[3]};
    } else {
        typedef float f2 __attribute__((ext_vector_type(2)));
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        unsigned p[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            p[k] = __builtin_bit_cast(unsigned, __builtin_convertvector(f2{o[2 * k], o[2 * k + 1]}, b2));
        r = u32x4{p[0], p[1], p[2], p[3]};
    }
    return r;
}

template <DType D>
__device__ __forceinline__ float grad_scalar(float x, float lse, float g) {
    return g * exp2_hw((x - lse) * kLog2e);
}

// fp32 to the bits of a 16-bit element, rounded to nearest even.
template <DType D>
__device__ __forceinline__ unsigned short float_to_half_bits(float v) {
    if constexpr (D == DType::BF16)
        return __builtin_bit_cast(unsigned short, static_cast<__bf16>(v));
    else
        return __builtin_bit_cast(unsigned short, static_cast<_Float16>(v));
}

template <DType D>
__device__ __forceinline__ void store_scalar(char* p, float v) {
    if constexpr (D == DType::F32) {
        *reinterpret_cast<float*>(p) = v;
    } else {
        *reinterpret_cast<unsigned short*>(p) = float_to_half_bits<D>(v);
    }
}

}  // namespace

// VEC: units are 16-byte vectors (K elements); otherwise single elements.
// PEEL (VEC only): row r's units start h(r) < K elements into the row, at its
// first 16-byte boundary; x and grad_x have the same phase, so one h(r)
// serves both. Every row then has the same nunits = (cols - K + 1) / K units
// and cols - nunits * K elements outside them (its head and its tail).
// ONE_ROW: the workgroup takes one chunk of one row (rows_per_wg == 1), so
// the row's lse and grad_out are uniform; otherwise every unit loads its own
// row's pair. Each instance issues the same loads in every batch.
template <DType D, int BLOCK, int U, bool VEC, bool PEEL, bool ONE_ROW, bool TOK>
__global__ __launch_bounds__(BLOCK) void lse_grad(const char* __restrict__ x, int64_t rows,
                                                  int64_t cols, int64_t xs_bytes,
                                                  const float* __restrict__ lse,
                                                  const float* __restrict__ gout,
                                                  const int64_t* __restrict__ targets,
                                                  char* __restrict__ gx, int64_t gs_bytes,
                                                  int64_t rows_per_wg, int64_t chunks_per_row,
                                                  int64_t chunk_units) {
    constexpr int EB = Elem<D>::kBytes;
    constexpr int K = VEC ? Elem<D>::kPerVec : 1;
    constexpr int UB = VEC ? 16 : EB;  // bytes per unit
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int64_t nunits = PEEL ? (cols - (K - 1)) / K : cols / K;
    // elements of each row outside its units: the tail (and with PEEL the head)
    const int rest = VEC ? static_cast<int>(cols - nunits * K) : 0;

    // PEEL: the head h(r) of row r from the phase of its start mod 16, which
    // is (x + r * xs) mod 16 = (x mod 16 + (r mod 16) * (xs mod 16)) mod 16.
    const unsigned xphase = static_cast<unsigned>(reinterpret_cast<uintptr_t>(x)) & 15u;
    const unsigned sphase = static_cast<unsigned>(xs_bytes) & 15u;
    auto head_of = [&](int64_t row) -> int {
        if constexpr (!PEEL) {
            return 0;
        } else {
            const unsigned ph = (xphase + (static_cast<unsigned>(row) & 15u) * sphase) & 15u;
            return static_cast<int>(((16u - ph) & 15u) / EB);
        }
    };

    // This workgroup's block: rows [r0, r0 + nr), units [u0, u0 + W) of each.
    int64_t r0, u0, W;
    int nr;
    if constexpr (ONE_ROW) {
        r0 = b / chunks_per_row;
        const int64_t chunk = b - r0 * chunks_per_row;
        u0 = chunk * chunk_units;
        W = nunits - u0 < chunk_units ? nunits - u0 : chunk_units;
        nr = 1;
    } else {
        r0 = b * rows_per_wg;
        nr = static_cast<int>(rows - r0 < rows_per_wg ? rows - r0 : rows_per_wg);
        u0 = 0;
        W = nunits;
    }
    const int n = static_cast<int>(nr * W);  // the planner keeps this below 2^22
    // The block's bytes as one buffer each for x and grad_x (offsets are
    // relative to the block's first unit, or with PEEL and several rows to
    // its first row's start; the planner keeps them below 2^31).
    const int h0 = ONE_ROW ? head_of(r0) : 0;
    const char* xb = x + r0 * xs_bytes + h0 * EB + u0 * UB;
    char* gb = gx + r0 * gs_bytes + h0 * EB + u0 * UB;
    const int64_t last_bytes = (PEEL && !ONE_ROW) ? cols * EB : W * UB;
    const int64_t xspan = (nr - 1) * xs_bytes + last_bytes;
    const int64_t gspan = (nr - 1) * gs_bytes + last_bytes;
    const auto xr = make_rsrc(xb, xspan);
    const auto gr = make_rsrc(gb, gspan);
    const float inv_w = 1.0f / static_cast<float>(W);

    // A row's (lse, g, target): TOK negates g and makes lse NaN for a target
    // outside [0, cols).
    auto row_terms = [&](int64_t row, float& l, float& g, int64_t& tt) {
        l = lse[row];
        g = gout[row];
        tt = -1;
        if constexpr (TOK) {
            tt = targets[row];
            if (tt < 0 || tt >= cols) l = __builtin_nanf("");
            g = -g;
        }
    };
    // The target's place in a unit whose first column is c0: 0..K-1, else -1.
    auto unit_target = [&](int64_t tt, int64_t c0) {
        const int64_t d = tt - c0;
        return d >= 0 && d < K ? static_cast<int>(d) : -1;
    };

    // uniform per-row scalars in the one-row case
    float l0 = 0.0f, g0 = 0.0f;
    int64_t t0 = -1;
    if (ONE_ROW && n > 0) row_terms(r0, l0, g0, t0);

    // Item j of the block: its row (local), byte offsets, and the column of
    // its unit's first element.
    auto offsets = [&](int j, int& rl, int& xo, int& go, int64_t& c0) {
        const bool in = j < n;
        rl = 0;
        if constexpr (!ONE_ROW) {
            // exact for j < 2^22: (j + 0.5) / W stays 0.5 / W away from integers
            rl = static_cast<int>((static_cast<float>(j) + 0.5f) * inv_w);
            rl = rl < nr ? rl : nr - 1;
        }
        const int u = j - rl * static_cast<int>(W);
        const int h = ONE_ROW ? 0 : head_of(r0 + rl);  // ONE_ROW: in the base already
        xo = in ? static_cast<int>(rl * xs_bytes) + h * EB + u * UB : kOffFar;
        go = in ? static_cast<int>(rl * gs_bytes) + h * EB + u * UB : kOffFar;
        c0 = (ONE_ROW ? h0 : h) + (u0 + u) * static_cast<int64_t>(K);
    };

    struct Batch {
        u32x4 w[VEC ? U : 1];
        float e[VEC ? 1 : U];
        float l[U], g[U];
        int go[U];
        int tk[TOK ? U : 1];
    };
    auto load_batch = [&](Batch& t, int j0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int rl, xo, go;
            int64_t c0;
            offsets(j0 + u * BLOCK, rl, xo, go, c0);
            t.go[u] = go;
            if constexpr (VEC) {
                t.w[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xo, 0, 2));
            } else if constexpr (D == DType::F32) {
                t.e[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, xo, 0, 2));
            } else {
                t.e[u] = half_to_float<D>(__builtin_amdgcn_raw_buffer_load_b16(xr, xo, 0, 2));
            }
            int64_t tt = t0;
            if constexpr (!ONE_ROW) {
                row_terms(r0 + rl, t.l[u], t.g[u], tt);
            } else {
                t.l[u] = l0;
                t.g[u] = g0;
            }
            if constexpr (TOK) t.tk[u] = unit_target(tt, c0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto store_batch = [&](const Batch& t) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (VEC) {
                const u32x4 r = grad_vec<D, TOK>(t.w[u], t.l[u], t.g[u], TOK ? t.tk[u] : -1);
                typedef unsigned v4u __attribute__((ext_vector_type(4)));
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, r), gr, t.go[u], 0, 2);
            } else {
                float v = grad_scalar<D>(t.e[u], t.l[u], t.g[u]);
                if (TOK && t.tk[u] == 0) v -= t.g[u];
                if constexpr (D == DType::F32)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), gr, t.go[u], 0, 2);
                else
                    __builtin_amdgcn_raw_buffer_store_b16(float_to_half_bits<D>(v), gr, t.go[u], 0,
                                                          2);
            }
        }
    };

    // Software-pipelined: the next batch's loads are issued before this
    // batch is computed and stored.
    const int per_batch = U * BLOCK;
    const int nb = (n + per_batch - 1) / per_batch;
    if (nb > 0) {
        Batch ta, tb;
        load_batch(ta, tid);
        int k = 0;
        for (; k + 2 <= nb - 1; k += 2) {
            load_batch(tb, (k + 1) * per_batch + tid);
            store_batch(ta);
            load_batch(ta, (k + 2) * per_batch + tid);
            store_batch(tb);
        }
        if (k + 1 <= nb - 1) {
            load_batch(tb, (k + 1) * per_batch + tid);
            store_batch(ta);
            store_batch(tb);
        } else {
            store_batch(ta);
        }
    }

    // The elements of each row outside its units (vector units only): item e
    // < h(r) is head column e, the others tail column nunits * K + e. In the
    // one-row case the row's first chunk takes the head and its last chunk the
    // tail; otherwise the block takes every row's.
    if constexpr (VEC) {
        const bool first = !ONE_ROW || u0 == 0;
        const bool last = !ONE_ROW || u0 + W == nunits;
        if (rest > 0 && (first || last)) {
            for (int i = tid; i < nr * rest; i += BLOCK) {
                const int rl = i / rest;
                const int e = i - rl * rest;
                const int64_t row = r0 + rl;
                const int h = head_of(row);
                if (e < h ? !first : !last) continue;
                const int64_t col = e < h ? e : nunits * K + e;
                const float xv = load_scalar<D>(x + row * xs_bytes + col * EB);
                float l, g;
                int64_t tt;
                row_terms(row, l, g, tt);
                float v = grad_scalar<D>(xv, l, g);
                if (TOK && col == tt) v -= g;
                store_scalar<D>(gx + row * gs_bytes + col * EB, v);
            }
        }
    }
}

namespace {

template <DType D, bool VEC, bool PEEL, bool ONE_ROW, bool TOK>
hipError_t launch_grad_k(const GradArgs& a) {
    constexpr int BLOCK = 256, U = 4;
    hipLaunchKernelGGL((lse_grad<D, BLOCK, U, VEC, PEEL, ONE_ROW, TOK>), dim3(a.grid), dim3(BLOCK), 0,
                       a.stream, a.x, a.rows, a.cols, a.xs_bytes, a.lse, a.grad_out, a.targets,
                       a.grad_x, a.gs_bytes, a.rows_per_wg, a.chunks_per_row, a.chunk_units);
    return hipGetLastError();
}

template <DType D, bool VEC, bool PEEL, bool TOK>
hipError_t launch_grad_t(const GradArgs& a) {
    return a.rows_per_wg == 1 ? launch_grad_k<D, VEC, PEEL, true, TOK>(a)
                              : launch_grad_k<D, VEC, PEEL, false, TOK>(a);
}

template <DType D, bool VEC, bool PEEL>
hipError_t launch_grad_p(const GradArgs& a) {
    return a.targets != nullptr ? launch_grad_t<D, VEC, PEEL, true>(a)
                                : launch_grad_t<D, VEC, PEEL, false>(a);
}

template <DType D>
hipError_t launch_grad_d(const GradArgs& a) {
    if (!a.vector_units) return launch_grad_p<D, false, false>(a);
    return a.peel ? launch_grad_p<D, true, true>(a) : launch_grad_p<D, true, false>(a);
}

}  // namespace

hipError_t launch_grad(const GradArgs& a) {
    if (a.grid <= 0) return hipSuccess;
    switch (a.dtype) {
        case LSE_DTYPE_F32: return launch_grad_d<DType::F32>(a);
        case LSE_DTYPE_BF16: return launch_grad_d<DType::BF16>(a);
        case LSE_DTYPE_F16: return launch_grad_d<DType::F16>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace lse
