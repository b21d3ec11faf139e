// Control kernels: the measuring sticks for the LSE kernels.
//
// It reads a contiguous byte range exactly once, with the load instruction and
// software pipeline of the streaming LSE schedule: 16-byte non-temporal loads,
// batches of 4 per lane, the next batch in flight while one is consumed. It
// keeps only the XOR of the 32-bit words of each chunk. Timed on the same
// buffers, launch geometry and stream as an LSE launch, it shows how fast this
// device streams those bytes when nothing else is done with them. The paper's
// introduction (section 1, its motivation) sets torch's LSE against a plain
// sum over the same tensor; this is that comparison with the sum replaced by
// the cheapest full read.
//
// Measurement infrastructure only: it is built into its own library
// (libread_control.so), and nothing on the LSE path calls it.
//
//   int lse_control_read(const void* x, int64_t bytes, int64_t chunks, int block,
//                        unsigned* out, hipStream_t stream)
//
// x: device pointer, 16-byte aligned; bytes: a multiple of 16. The range's nvec
// 16-byte vectors are cut into `chunks` pieces: with q = nvec / chunks and
// r = nvec % chunks, chunk g holds q + (g < r) vectors starting at
// g*q + min(g, r) (no division on the device); one workgroup of `block` threads (64,
// 128, 256, 512 or 1024) reads each chunk and writes the XOR of its 32-bit
// words to out[g] (device, `chunks` words). Returns 0 on success, 1 for an
// invalid argument (checked before any HIP call), 2 if the launch fails.
// Asynchronous on `stream`; allocates nothing.
//
//   int lse_control_copy(const void* src, void* dst, int64_t bytes, int64_t chunks,
//                        int block, hipStream_t stream)
//
// The measuring stick for the backward passes, which read x and write grad_x
// of the same size: src[0:bytes] copied to dst with the same chunks, loads and
// pipeline, non-temporal 16-byte stores. src and dst 16-byte aligned and not
// overlapping; the same return codes.
//
//   int lse_control_rows(const void* x, int64_t bytes, int64_t grid, int store,
//                        unsigned* out, hipStream_t stream)
//
// The measuring stick for many 64-byte rows (16 fp32), read with the register-
// rows schedule's pattern: `grid` workgroups of 256 threads, 4 lanes per row,
// 4 KiB per wavefront per iteration, grid-stride over iterations. bytes: a
// multiple of 4096. store != 0 writes the XOR of each row's 16 words to
// out[row] (bytes / 64 words), staged in LDS and stored 64 iterations at a
// time as the LSE kernel writes its results: the read + write control. store == 0
// writes one word per wavefront (out: grid * 4 words): the read-only control
// with the same geometry.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBatch = 4;  // 16-byte loads per lane per batch

__device__ __forceinline__ unsigned xor4(u32x4 v) { return (v.x ^ v.y) ^ (v.z ^ v.w); }

template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void read_chunks(const u32x4* __restrict__ x, int64_t q,
                                                     int64_t r, unsigned* __restrict__ out) {
    __shared__ unsigned wave_x[BLOCK / 64];
    const int tid = threadIdx.x;
    const int64_t g = blockIdx.x;
    const int64_t v0 = g * q + (g < r ? g : r);
    const int64_t n = q + (g < r ? 1 : 0);
    const u32x4* p = x + v0 + tid;
    constexpr int64_t kStep = static_cast<int64_t>(kBatch) * BLOCK;
    const int64_t nfull = n / kStep;

    unsigned acc = 0;
    u32x4 a[kBatch], b[kBatch];
    auto load = [&](u32x4* r, int64_t k) {
        // The batch's addresses take an opaque zero computed from acc, so its
        // loads issue after the batch held in the same registers has been
        // consumed, as written. Without it the compiler hoists them above
        // that consumption and then copies the registers back, which waits
        // for every load in flight at the end of each iteration.
        unsigned z;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z) : "v"(acc));
        const u32x4* q = p + k * kStep + z;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) r[u] = __builtin_nontemporal_load(q + u * BLOCK);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto consume = [&](const u32x4* r) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) acc ^= xor4(r[u]);
    };
    if (nfull > 0) {
        load(a, 0);
        int64_t k = 0;
        for (; k + 2 < nfull; k += 2) {
            load(b, k + 1);
            consume(a);
            load(a, k + 2);
            consume(b);
        }
        if (k + 1 < nfull) {
            load(b, k + 1);
            consume(a);
            consume(b);
        } else {
            consume(a);
        }
    }
    // the last n - nfull*kStep < kStep vectors, each lane's in bounds only
    for (int64_t i = nfull * kStep + tid; i < n; i += BLOCK)
        acc ^= xor4(__builtin_nontemporal_load(x + v0 + i));

    // XOR across the wavefront, then across the wavefronts through LDS
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    if ((tid & 63) == 0) wave_x[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
        unsigned r = 0;
#pragma unroll
        for (int w = 0; w < BLOCK / 64; ++w) r ^= wave_x[w];
        out[g] = r;
    }
}

// The copy control: the same chunks, each vector loaded and stored back to
// dst at the same offset with 16-byte non-temporal loads and stores, the
// next batch's loads issued before a batch is stored.
template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void copy_chunks(const u32x4* __restrict__ src,
                                                     u32x4* __restrict__ dst, int64_t q,
                                                     int64_t r) {
    const int tid = threadIdx.x;
    const int64_t g = blockIdx.x;
    const int64_t v0 = g * q + (g < r ? g : r);
    const int64_t n = q + (g < r ? 1 : 0);
    constexpr int64_t kStep = static_cast<int64_t>(kBatch) * BLOCK;
    const int64_t nfull = n / kStep;
    const u32x4* p = src + v0 + tid;
    u32x4* d = dst + v0 + tid;

    u32x4 a[kBatch], b[kBatch];
    auto load = [&](u32x4* w, int64_t k) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) w[u] = __builtin_nontemporal_load(p + k * kStep + u * BLOCK);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto store = [&](const u32x4* w, int64_t k) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) __builtin_nontemporal_store(w[u], d + k * kStep + u * BLOCK);
        __builtin_amdgcn_sched_barrier(0);
    };
    if (nfull > 0) {
        load(a, 0);
        int64_t k = 0;
        for (; k + 2 < nfull; k += 2) {
            load(b, k + 1);
            store(a, k);
            load(a, k + 2);
            store(b, k + 1);
        }
        if (k + 1 < nfull) {
            load(b, k + 1);
            store(a, k);
            store(b, k + 1);
        } else {
            store(a, k);
        }
    }
    for (int64_t i = nfull * kStep + tid; i < n; i += BLOCK)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + v0 + i), dst + v0 + i);
}

// The row control: the memory pattern of the register-rows LSE schedule on
// 64-byte rows (4 lanes per row, 16 rows per wavefront per round, 4 rounds:
// 4 KiB per wavefront per iteration, iterations wave, wave + nwaves, ... with
// the next iteration's loads in flight while one is consumed). Each row's 16
// words are XORed into one word. With STORE, the words go out as the LSE
// kernel writes its results: each wavefront stages 64 iterations' words (64
// per iteration, row it*64 + l in slot l) in LDS and then stores them with
// non-temporal 256-byte stores, lane l storing row it*64 + l; without, each
// wavefront writes the XOR of all its rows to out[wave] once at the end.
// Workgroups of 256 threads.
constexpr int kRowsFlush = 64;  // iterations staged per wavefront between stores

template <bool STORE>
__global__ __launch_bounds__(256) void rows64_chunks(const u32x4* __restrict__ x, int64_t iters,
                                                      unsigned* __restrict__ out) {
    __shared__ unsigned stage[4][STORE ? kRowsFlush * 64 : 1];
    const int lane = threadIdx.x & 63;
    unsigned* st = stage[threadIdx.x >> 6];
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
    const int64_t last = iters - 1;
    unsigned acc = 0;
    int slot = 0;
    int64_t first_it = wave;
    auto flush = [&]() {
        __builtin_amdgcn_wave_barrier();
        for (int j = 0; j < slot; ++j)
            __builtin_nontemporal_store(st[j * 64 + lane],
                                        out + (first_it + static_cast<int64_t>(j) * nwaves) * 64 + lane);
        __builtin_amdgcn_wave_barrier();
        slot = 0;
    };
    auto load = [&](u32x4* r, int64_t it) {
        // an opaque zero computed from acc keeps these loads after the
        // consumption of the registers they overwrite (as in read_chunks)
        unsigned z;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z) : "v"(acc));
        const u32x4* q = x + it * 256 + lane + z;  // round k: vectors it*256 + k*64 + lane
#pragma unroll
        for (int k = 0; k < 4; ++k) r[k] = __builtin_nontemporal_load(q + k * 64);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto consume = [&](const u32x4* r, int64_t it) {
        unsigned v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] = xor4(r[k]);
            v[k] ^= __shfl_xor(v[k], 1, 64);
            v[k] ^= __shfl_xor(v[k], 2, 64);
            acc ^= v[k];
        }
        if constexpr (STORE) {
            // lane 4j of round k holds row k*16 + j of the iteration
            if (slot == 0) first_it = it;
            if ((lane & 3) == 0) {
#pragma unroll
                for (int k = 0; k < 4; ++k) st[slot * 64 + k * 16 + (lane >> 2)] = v[k];
            }
            if (++slot == kRowsFlush) flush();
        }
    };
    if (wave <= last) {
        u32x4 a[4], b[4];
        int64_t it = wave;
        load(a, it);
        while (true) {
            int64_t next = it + nwaves;
            load(b, next < last ? next : last);
            consume(a, it);
            it = next;
            if (it > last) break;
            next = it + nwaves;
            load(a, next < last ? next : last);
            consume(b, it);
            it = next;
            if (it > last) break;
        }
        if (STORE && slot > 0) flush();
    }
    if constexpr (!STORE) {
        // every lane of a row's group holds the same words: XOR across groups
#pragma unroll
        for (int off = 4; off < 64; off <<= 1) acc ^= __shfl_xor(acc, off, 64);
        if (lane == 0) out[wave] = acc;
    }
}

template <int BLOCK>
int launch(const void* x, int64_t nvec, int64_t chunks, unsigned* out, hipStream_t stream) {
    hipLaunchKernelGGL(read_chunks<BLOCK>, dim3(static_cast<unsigned>(chunks)), dim3(BLOCK), 0,
                       stream, static_cast<const u32x4*>(x), nvec / chunks, nvec % chunks, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

template <int BLOCK>
int launch_copy(const void* src, void* dst, int64_t nvec, int64_t chunks, hipStream_t stream) {
    hipLaunchKernelGGL(copy_chunks<BLOCK>, dim3(static_cast<unsigned>(chunks)), dim3(BLOCK), 0,
                       stream, static_cast<const u32x4*>(src), static_cast<u32x4*>(dst),
                       nvec / chunks, nvec % chunks);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // namespace

extern "C" int lse_control_read(const void* x, int64_t bytes, int64_t chunks, int block,
                                unsigned* out, hipStream_t stream) {
    if (bytes < 0 || bytes % 16 != 0 || chunks < 1 || chunks > 0x7FFFFFFF) return 1;
    if (x == nullptr || out == nullptr || reinterpret_cast<uintptr_t>(x) % 16 != 0) return 1;
    if (reinterpret_cast<uintptr_t>(out) % 4 != 0) return 1;
    const int64_t nvec = bytes / 16;
    switch (block) {
        case 64: return launch<64>(x, nvec, chunks, out, stream);
        case 128: return launch<128>(x, nvec, chunks, out, stream);
        case 256: return launch<256>(x, nvec, chunks, out, stream);
        case 512: return launch<512>(x, nvec, chunks, out, stream);
        case 1024: return launch<1024>(x, nvec, chunks, out, stream);
        default: return 1;
    }
}

extern "C" int lse_control_copy(const void* src, void* dst, int64_t bytes, int64_t chunks,
                                int block, hipStream_t stream) {
    if (bytes < 0 || bytes % 16 != 0 || chunks < 1 || chunks > 0x7FFFFFFF) return 1;
    if (src == nullptr || dst == nullptr) return 1;
    if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
        return 1;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    if (s0 < d0 + static_cast<uintptr_t>(bytes) && d0 < s0 + static_cast<uintptr_t>(bytes))
        return 1;  // overlapping ranges
    const int64_t nvec = bytes / 16;
    switch (block) {
        case 64: return launch_copy<64>(src, dst, nvec, chunks, stream);
        case 128: return launch_copy<128>(src, dst, nvec, chunks, stream);
        case 256: return launch_copy<256>(src, dst, nvec, chunks, stream);
        case 512: return launch_copy<512>(src, dst, nvec, chunks, stream);
        case 1024: return launch_copy<1024>(src, dst, nvec, chunks, stream);
        default: return 1;
    }
}

extern "C" int lse_control_rows(const void* x, int64_t bytes, int64_t grid, int store,
                                unsigned* out, hipStream_t stream) {
    if (bytes < 0 || bytes % 4096 != 0 || grid < 1 || grid > 0x7FFFFFFF) return 1;
    if (x == nullptr || out == nullptr || reinterpret_cast<uintptr_t>(x) % 16 != 0) return 1;
    if (reinterpret_cast<uintptr_t>(out) % 4 != 0) return 1;
    const int64_t iters = bytes / 4096;
    if (store)
        hipLaunchKernelGGL(rows64_chunks<true>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                           stream, static_cast<const u32x4*>(x), iters, out);
    else
        hipLaunchKernelGGL(rows64_chunks<false>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                           stream, static_cast<const u32x4*>(x), iters, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
