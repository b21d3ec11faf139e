// lse_device.h - device-side building blocks of the row-wise log-sum-exp
// kernels for gfx950 (CDNA4, wave64).
//
// The accumulator. The paper "Speeding up Log-Sum-Exp: Kernel Fusion at the
// Memory Wall, Integer Arithmetic at the Compute Wall" computes LSE in one
// pass by folding elements with the associative, commutative pairwise LSE,
// each thread keeping a register accumulator (§3.1): a running maximum and a
// sum of exponentials, the online form its §2.2 describes. Here a lane keeps
//
//     m  a reference: the largest element folded so far, or (fold_lazy_vecs) a
//        value at most 32*ln2 below it (natural units, exact),
//     c  = fl(clamp(m, -2^30, 2^30) * log2(e)), the base-2 reference,
//     s  = sum over folded x of 2^(x*log2(e) - c),
//
// so the value it represents is ln2 * (c + log2 s). The exponentials run on
// the hardware exp2 (v_exp_f32): each term costs one fused multiply-add
// x*log2(e) - c and one v_exp_f32. A new maximum rescales s by 2^(c_old -
// c_new) <= 1. The pairwise merge of (m1, c1, s1) and (m2, c2, s2) is
// (max m, max c, s1*2^(c1 - C) + s2*2^(c2 - C)); the kernels apply it once
// per batch of elements, across lanes and across workgroups.
//
// Why the clamp: c = fl(m*log2e) misses m*log2e by up to half an ulp, and a
// term x = m contributes 2^(m*log2e - c). For |m| <= 2^30, m*log2e < 2^31,
// so that residual is at most 2^6 and every term is at most 2^64: no sum can
// overflow. Clamping m to +-2^30 before taking c keeps c finite for every m,
// including +-inf, so no inf - inf or 0 * inf arises in the recursion. Rows
// whose maximum lies beyond +-2^30 are recomputed by a natural-units pass,
// sum 2^((x - m)*log2e), which has no such limit.
//
// Special values: a NaN element makes its own term NaN, so s becomes NaN and
// stays NaN whatever the max does; +inf gives s = +inf with m = +inf; a row
// of -inf (or no elements) keeps s = 0 and m = -inf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lse {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 0x1.715476p+0f;  // log2(e) rounded to fp32
constexpr float kLn2 = 0x1.62e430p-1f;    // ln(2) rounded to fp32
constexpr float kClamp = 0x1p30f;         // |m| beyond this takes the slow pass
constexpr float kInf = __builtin_inff();
// s_waitcnt immediate for gfx9: vmcnt = 0, expcnt and lgkmcnt left at their
// maxima (not waited on).
constexpr int kWaitVmcnt0 = 0x0F70;

enum class DType : int { F32 = 0, BF16 = 1, F16 = 2 };

template <DType D> struct Elem;
template <> struct Elem<DType::F32> {
    static constexpr int kBytes = 4;
    static constexpr int kPerVec = 4;            // elements in one 16-byte load
    static constexpr unsigned kNegInfWord = 0xFF800000u;
};
template <> struct Elem<DType::BF16> {
    static constexpr int kBytes = 2;
    static constexpr int kPerVec = 8;
    static constexpr unsigned kNegInfWord = 0xFF80FF80u;  // two bf16 -inf
};
template <> struct Elem<DType::F16> {
    static constexpr int kBytes = 2;
    static constexpr int kPerVec = 8;
    static constexpr unsigned kNegInfWord = 0xFC00FC00u;  // two fp16 -inf
};

// ---- arithmetic primitives -------------------------------------------------

// max of three floats in one v_max3_f32. Written as asm so that the compiler
// does not wrap each input in a canonicalising max (IEEE maxNum lowering);
// NaN handling does not rely on the max (see the header comment).
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// c(m): the base-2 reference of a running maximum; finite for every m. It
// must be the rounded product fl(m * log2 e) wherever it is used: merges
// rely on two references of the same m being equal, so that 2^(c1 - C) is
// exactly 1, and the finish recovers the rounding by an fma. A product the
// compiler fused into a following subtraction (fp-contract) would leave the
// rounding residual, up to half an ulp of c, in the exponent instead; the
// pragma keeps this multiply a multiply.
__device__ __forceinline__ float base2_ref(float m) {
#pragma clang fp contract(off)
    return __builtin_amdgcn_fmed3f(m, -kClamp, kClamp) * kLog2e;
}

__device__ __forceinline__ bool is_nan(float v) {
    return (__float_as_uint(v) & 0x7FFFFFFFu) > 0x7F800000u;
}

// ---- element decoding ------------------------------------------------------

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// One 16-bit element (its bits in the low half of `bits`) to fp32, exactly:
// bf16's 16 bits become the high half of an fp32 word; fp16 converts with
// v_cvt_f32_f16 (every fp16 value, subnormals included, is an fp32 value).
template <DType D>
__device__ __forceinline__ float half_to_float(unsigned bits) {
    if constexpr (D == DType::BF16)
        return __uint_as_float(bits << 16);
    else
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(bits)));
}

// The 16-bit element in the high (hi) or low half of a 32-bit word, as fp32.
template <DType D>
__device__ __forceinline__ float word_half_to_float(unsigned word, bool hi) {
    if constexpr (D == DType::BF16)
        return __uint_as_float(hi ? (word & 0xFFFF0000u) : (word << 16));
    else
        return half_to_float<D>(hi ? word >> 16 : word & 0xFFFFu);
}

// One 16-byte word vector to fp32 values, in memory order. bf16 is exact: its
// 16 bits become the high half of an fp32 word; fp16 is exact by conversion.
template <DType D>
__device__ __forceinline__ void decode(const u32x4 w, float* f) {
    if constexpr (D == DType::F32) {
        f[0] = __uint_as_float(w.x);
        f[1] = __uint_as_float(w.y);
        f[2] = __uint_as_float(w.z);
        f[3] = __uint_as_float(w.w);
    } else if constexpr (D == DType::F16) {
        const unsigned ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const half2_t h = __builtin_bit_cast(half2_t, ws[k]);
            f[2 * k] = static_cast<float>(h.x);
            f[2 * k + 1] = static_cast<float>(h.y);
        }
    } else {
        f[0] = __uint_as_float(w.x << 16);
        f[1] = __uint_as_float(w.x & 0xFFFF0000u);
        f[2] = __uint_as_float(w.y << 16);
        f[3] = __uint_as_float(w.y & 0xFFFF0000u);
        f[4] = __uint_as_float(w.z << 16);
        f[5] = __uint_as_float(w.z & 0xFFFF0000u);
        f[6] = __uint_as_float(w.w << 16);
        f[7] = __uint_as_float(w.w & 0xFFFF0000u);
    }
}

template <DType D>
__device__ __forceinline__ float load_scalar(const char* p) {
    if constexpr (D == DType::F32) {
        return __builtin_nontemporal_load(reinterpret_cast<const float*>(p));
    } else {
        unsigned short h = __builtin_nontemporal_load(reinterpret_cast<const unsigned short*>(p));
        return half_to_float<D>(h);
    }
}

__device__ __forceinline__ u32x4 load_vec(const u32x4* p) {
    return __builtin_nontemporal_load(p);
}

template <DType D>
__device__ __forceinline__ u32x4 neg_inf_vec() {
    const unsigned w = Elem<D>::kNegInfWord;
    return u32x4{w, w, w, w};
}

// ---- the accumulator -------------------------------------------------------

struct Acc {
    float m;  // running max
    float c;  // base2_ref(m)
    float s;  // sum of 2^(x*log2e - c) ...
    float e;  // ... plus this compensation term (rounding errors of the sum)
};

__device__ __forceinline__ Acc acc_empty() { return Acc{-kInf, base2_ref(-kInf), 0.0f, 0.0f}; }

// The lane's sum, compensation included. Once s is +inf or NaN (a +inf or NaN
// element, or a maximum beyond 2^126), TwoSum's inf - inf has made e NaN:
// s alone is then the answer.
__device__ __forceinline__ float acc_sum(const Acc& a) {
    return (__float_as_uint(a.s) & 0x7FFFFFFFu) >= 0x7F800000u ? a.s : a.s + a.e;
}

// A compensated running sum for the merges that add partial sums one after
// another (across wavefronts, across the lanes or parts of a column): each
// add's rounding error (TwoSum) goes to e, so terms that are each smaller
// than half an ulp of the total still count. Without it, one partial near 1
// followed by 63 partials of 5.7e-8 lost 1.7e-6 of the sum.
struct CSum {
    float s = 0.0f;
    float e = 0.0f;
    __device__ __forceinline__ void add(float t) {
        const float sum = s + t;
        const float bp = sum - s;
        e += (s - (sum - bp)) + (t - bp);
        s = sum;
    }
    // the total; +inf or NaN as they stand (their TwoSum error is NaN)
    __device__ __forceinline__ float total() const {
        return (__float_as_uint(s) & 0x7FFFFFFFu) >= 0x7F800000u ? s : s + e;
    }
};

// Maximum of the N values v[0..N) by a chain of v_max3_f32, each taking two
// new values: (N - 1) / 2 instructions, rounded up.
template <int N>
__device__ __forceinline__ float max_chain(const float* v) {
    float r = v[0];
    int j = 1;
#pragma unroll
    for (; j + 1 < N; j += 2) r = max3f(r, v[j], v[j + 1]);
    if (j < N) r = max3f(r, v[j], v[j]);
    return r;
}

// Maximum of m0 and f[0..N): three independent chains of odd length (no
// wasted max3 operand when N + 1 splits evenly) joined by one more max3.
template <int N>
__device__ __forceinline__ float max_of(float m0, const float* f) {
    constexpr int V = N + 1;
    float v[V];
    v[0] = m0;
#pragma unroll
    for (int j = 0; j < N; ++j) v[j + 1] = f[j];
    if constexpr (V <= 7) {
        return max_chain<V>(v);
    } else {
        constexpr int A = (V / 3) | 1;
        constexpr int B = ((V - A) / 2) | 1;
        return max3f(max_chain<A>(v), max_chain<B>(v + A), max_chain<V - A - B>(v + A + B));
    }
}

// Pairwise (tree) sum of 2^(f[j]*log2e - c), j < N.
template <int N>
__device__ __forceinline__ float sum_exp_of(const float* f, float c) {
    if constexpr (N == 1) {
        return exp2_hw(__builtin_fmaf(f[0], kLog2e, -c));
    } else {
        constexpr int H = N / 2;
        return sum_exp_of<H>(f, c) + sum_exp_of<N - H>(f + H, c);
    }
}

// Fold N values into the accumulator: one max, one rescale, N exponentials
// summed as a tree, and one compensated add of that batch sum. The add is
// Knuth's TwoSum, whose rounding error goes to `e`: without it, a long row
// of near-constant batch sums (each smaller than the running sum's ulp
// allows to add exactly) drifts by up to 1e-4 relative over 10^5 batches.
template <int N>
__device__ __forceinline__ void fold(Acc& a, const float* f) {
    const float m = max_of<N>(a.m, f);
    const float c = base2_ref(m);
    const float t = sum_exp_of<N>(f, c);
    const float r = exp2_hw(a.c - c);  // rescale of the old sum, <= 1
    const float s = a.s * r;
    const float sum = s + t;
    const float bp = sum - s;
    const float err = (s - (sum - bp)) + (t - bp);
    a.e = __builtin_fmaf(a.e, r, err);
    a.s = sum;
    a.m = m;
    a.c = c;
}

// Sum of v[0..N) as the same tree sum_exp_of<N> builds (halves of N / 2 and
// N - N / 2, recursively).
template <int N>
__device__ __forceinline__ float tree_sum(const float* v) {
    if constexpr (N == 1) {
        return v[0];
    } else {
        constexpr int H = N / 2;
        return tree_sum<H>(v) + tree_sum<N - H>(v + H);
    }
}

// Fold a batch of U 16-byte vectors of type D (N = U * K values) lazily. The
// batch's terms are first taken against the lane's current reference c, with
// no maximum computed. That sum is kept when it is
// at most 2^32 and the reference is a finite maximum within +-2^30; otherwise
// (a new maximum more than 32*ln2 above the reference, an infinity, a NaN, no
// finite maximum yet, or the clamp in use) the batch is folded again by fold<N>,
// which moves the reference to the batch maximum. So the reference stays within
// 32*ln2 of the lane's running maximum: no term exceeds 2^38, no sum of fewer
// than 2^31 terms overflows, and the lane's largest element contributed a term
// of at least 2^-6, so terms that underflow are negligible. The value the lane
// represents, m + ln2*(log2 s - (m*log2e - c)), does not need m to be the
// maximum, only the reference that c and s were formed with. A lane whose
// reference is not a finite value within +-2^30 (its first batch, above all)
// goes to fold<N> directly: its lazy sum would be thrown away. Where each lane
// folds only one or two batches per row, that halves the exponentials.
//
// The lazy test reads only the accumulator, so it is taken before any vector
// is decoded: each vector's exponentials start as soon as that vector's load
// has returned, and the batch's arithmetic overlaps the arrival of its later
// loads (at a row's end only the last vector's terms remain after the last
// load). With U and K powers of two, the per-vector sums joined by
// tree_sum<U> are the tree of sum_exp_of<N> over the decoded batch.
template <DType D, int U>
__device__ __forceinline__ void fold_lazy_vecs(Acc& a, const u32x4 (&w)[U]) {
    constexpr int K = Elem<D>::kPerVec;
    static_assert((U & (U - 1)) == 0 && (K & (K - 1)) == 0, "the two trees agree for powers of two");
    if (__builtin_fabsf(a.m) <= kClamp) {
        float tv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float f[K];
            decode<D>(w[u], f);
            tv[u] = sum_exp_of<K>(f, a.c);
        }
        const float t = tree_sum<U>(tv);
        if (t <= 0x1p32f) {
            const float s = a.s;
            const float sum = s + t;
            const float bp = sum - s;
            a.e += (s - (sum - bp)) + (t - bp);
            a.s = sum;
            return;
        }
    }
    // The empty asm makes these words opaque, so that the decodes here are
    // not merged with the lazy path's and hoisted above its test (which
    // would wait for every load of the batch before the first exponential).
    float f[U * K];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        u32x4 v = w[u];
        asm volatile("" : "+v"(v));
        decode<D>(v, &f[u * K]);
    }
    fold<U * K>(a, f);
}

// The lazy fold of N decoded values f whose terms against the accumulator's
// reference, sum_exp_of<N>(f, a.c), the caller has already summed into t:
// for accumulators that fold many small batches (one per column and step in
// the non-last-axis kernel), where the terms are computed as their loads
// return and a second branch per fold would cost more than the exponentials
// it saves on an accumulator's first batch. t is kept under the lazy rule of
// fold_lazy_vecs; otherwise the batch is folded again by fold<N>.
template <int N>
__device__ __forceinline__ void fold_lazy_terms(Acc& a, const float* f, float t) {
    if (t <= 0x1p32f && __builtin_fabsf(a.m) <= kClamp) {
        const float s = a.s;
        const float sum = s + t;
        const float bp = sum - s;
        a.e += (s - (sum - bp)) + (t - bp);
        a.s = sum;
    } else {
        fold<N>(a, f);
    }
}

// True when |m| is finite and beyond 2^30: one unsigned range test on the bits.
__device__ __forceinline__ bool beyond_clamp(float m) {
    return (__float_as_uint(m) & 0x7FFFFFFFu) - 0x4E800001u < 0x7F800000u - 0x4E800001u;
}

// True when a reduced row must be recomputed in natural units: its maximum is
// finite but beyond +-2^30 (and no NaN made the answer NaN already).
__device__ __forceinline__ bool needs_natural_units(float m, float s) {
    return !is_nan(s) && __builtin_fabsf(m) > kClamp && __builtin_fabsf(m) != kInf;
}

// The finished value ln(sum exp) = m + ln2 * (log2 s - (m*log2e - c)) of a
// reduced (m, c, s) with |m| <= 2^30 or m = +-inf: NaN if s is NaN, +inf if
// m = +inf, -inf if m = -inf (s = 0: no element above -inf).
//
// The lazy reference can trail the maximum by up to 32*ln2, so s can reach
// 2^38 and log2 s 38, where one ulp of fp32 is 4e-6: taken whole, log2 s
// would put that much absolute error on a result near zero. So s is split
// exactly as mant * 2^k (mant in [0.5, 1)): m + k*ln2 is one fused
// multiply-add, and the hardware log2 sees only mant, whose log2 lies in
// [-1, 0). The error is then a few ulps of max(|result|, 1).
__device__ __forceinline__ float finish(float m, float c, float s) {
    if (is_nan(s)) return __builtin_nanf("");
    if (m == kInf) return kInf;
    if (m == -kInf) return -kInf;
    const float e = __builtin_fmaf(m, kLog2e, -c);  // exact residual of c = fl(m*log2e)
    const int k = __builtin_amdgcn_frexp_expf(s);
    const float mant = __builtin_amdgcn_frexp_mantf(s);
    const float hi = __builtin_fmaf(static_cast<float>(k), kLn2, m);
    return __builtin_fmaf(log2_hw(mant) - e, kLn2, hi);
}

// ---- cross-lane reductions (wave64) ---------------------------------------
//
// DPP row patterns combine lanes within a row of 16: quad_perm [1,0,3,2]
// pairs lanes i^1, [2,3,0,1] pairs i^2, row_half_mirror pairs i and 7-i in
// each half-row, row_mirror pairs i and 15-i. Applied in that order they give
// every lane of a group of 2, 4, 8 or 16 the group total (the pairs are
// symmetric, and a+b == b+a exactly, so all lanes agree bit for bit).
// ds_swizzle's xor-16 pattern joins two rows within 32 lanes. For the whole
// wavefront, row_bcast15 (row r's lane 15 into row r+1, rows 1 and 3) and
// row_bcast31 (lane 31 into rows 2 and 3) carry the row totals into lane 63,
// which readlane makes uniform: all DPP, no LDS-unit latency.

constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror
constexpr int kDppBcast15 = 0x142;     // row_bcast:15
constexpr int kDppBcast31 = 0x143;     // row_bcast:31
constexpr int kSwizzleXor16 = 0x401F;  // bit mode: and 0x1f, or 0, xor 0x10

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}

// DPP move restricted to the rows in ROW_MASK; other rows keep `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_rows(float old, float v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}

__device__ __forceinline__ float swizzle_xor16(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), kSwizzleXor16));
}

__device__ __forceinline__ float readlane(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

struct OpMax {
    __device__ __forceinline__ float operator()(float a, float b) const { return max3f(a, b, b); }
    static constexpr float kIdentity = -__builtin_inff();
};
struct OpSum {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
    static constexpr float kIdentity = 0.0f;
};

// A DPP move with no old value (every lane reads an in-bounds lane for the
// quad and mirror patterns), so that the compiler can fold it into the
// consuming add as a DPP operand.
template <int CTRL>
__device__ __forceinline__ float dpp_free(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Every lane of each aligned group of G lanes (G a power of two <= 64) gets
// the group's reduction. All lanes of a group must be active.
template <int G, typename Op>
__device__ __forceinline__ float group_reduce(float v, Op op) {
    if constexpr (G >= 2) v = op(v, dpp_free<kDppXor1>(v));
    if constexpr (G >= 4) v = op(v, dpp_free<kDppXor2>(v));
    if constexpr (G >= 8) v = op(v, dpp_free<kDppHalfMirror>(v));
    if constexpr (G >= 16) v = op(v, dpp_free<kDppMirror>(v));
    if constexpr (G == 32) v = op(v, swizzle_xor16(v));
    if constexpr (G == 64) {
        // rows 1, 3 += row 0, 2 (via lane 15, 47); rows 2, 3 += lane 31
        v = op(v, dpp_rows<kDppBcast15, 0xA>(Op::kIdentity, v));
        v = op(v, dpp_rows<kDppBcast31, 0xC>(Op::kIdentity, v));
        v = readlane(v, 63);
    }
    return v;
}

// Workgroup-wide reduction; the result is uniform. `scratch` holds one float
// per wavefront. Contains barriers: every thread of the block must call it.
// Used only off the hot path (the natural-units pass).
template <int BLOCK, typename Op>
__device__ __forceinline__ float block_reduce(float v, Op op, float* scratch) {
    constexpr int NW = BLOCK / 64;
    v = group_reduce<64>(v, op);
    if constexpr (NW == 1) {
        return v;
    } else {
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) scratch[wave] = v;
        __syncthreads();
        float r = scratch[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) r = op(r, scratch[w]);
        __syncthreads();
        return r;
    }
}

// The block's merged accumulator, uniform in every thread.
struct Merged {
    float m, c, s;
};

// A compensated sum over each aligned group of G lanes (G a power of two, at
// most 16): every lane of a group ends with the group's sum `s` and the
// accumulated rounding error `e` of its adds (TwoSum at every step, as CSum
// keeps for sequential adds). The patterns pair lanes symmetrically and TwoSum
// is exact, so every lane of a group holds the same bits.
template <int G>
__device__ __forceinline__ void group_csum(float& s, float& e) {
    auto step = [&](float vs, float ve) {
        const float sum = s + vs;
        const float bp = sum - s;
        const float err = (s - (sum - bp)) + (vs - bp);
        e = (e + ve) + err;
        s = sum;
    };
    if constexpr (G >= 2) step(dpp_free<kDppXor1>(s), dpp_free<kDppXor1>(e));
    if constexpr (G >= 4) step(dpp_free<kDppXor2>(s), dpp_free<kDppXor2>(e));
    if constexpr (G >= 8) step(dpp_free<kDppHalfMirror>(s), dpp_free<kDppHalfMirror>(e));
    if constexpr (G >= 16) step(dpp_free<kDppMirror>(s), dpp_free<kDppMirror>(e));
}

// Merge every lane's (m, c, s) into the workgroup's: each wavefront takes its
// lanes' max and then the sum of their sums rescaled to it (DPP, no LDS);
// lane 0 posts the wavefront's (max, sum) to `pairs` (2 floats per
// wavefront); after one barrier lanes 0..NW-1 of every wavefront each take
// one wavefront's pair and merge them with a DPP tree (maximum, then a
// compensated sum), lane 0's result broadcast to the whole wavefront, so the
// result is uniform and the same on every run. A tree of log2(NW) steps
// instead of NW sequential merges shortens the end of each workgroup, which
// lies on the launch's critical path: measured with per-wavefront timestamps
// on workload 2, from the last wavefront's final fold to the store took 0.73
// us with the sequential merge and 0.61 us with the tree (launch 21.60 ->
// 21.42 us). Every thread of the block must call it; `pairs` must not be
// rewritten before all threads have returned (a barrier separates two calls).
template <int BLOCK>
__device__ __forceinline__ Merged block_merge(float m, float c, float s, float* pairs) {
    constexpr int NW = BLOCK / 64;
    static_assert(NW <= 16, "the cross-wave tree spans one DPP row of 16 lanes");
    const float wm = group_reduce<64>(m, OpMax{});
    const float wc = base2_ref(wm);
    const float ws = group_reduce<64>(s * exp2_hw(c - wc), OpSum{});
    if constexpr (NW == 1) {
        return Merged{wm, wc, ws};
    } else {
        const int wave = threadIdx.x >> 6;
        const int l = threadIdx.x & 63;
        if (l == 0) {
            pairs[2 * wave] = wm;
            pairs[2 * wave + 1] = ws;
        }
        __syncthreads();
        // lanes past NW hold the empty pair (-inf, 0), which adds exactly 0
        const float pm = l < NW ? pairs[2 * l] : -kInf;
        const float ps = l < NW ? pairs[2 * l + 1] : 0.0f;
        const float bm = readlane(group_reduce<NW>(pm, OpMax{}), 0);
        const float bc = base2_ref(bm);
        float ts = ps * exp2_hw(base2_ref(pm) - bc);
        float te = 0.0f;
        group_csum<NW>(ts, te);
        CSum bs;
        bs.s = readlane(ts, 0);
        bs.e = readlane(te, 0);
        return Merged{bm, bc, bs.total()};
    }
}

}  // namespace lse
