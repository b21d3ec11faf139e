// lse_noalloc.hip - lse_forward_noalloc: the row-wise LSE of lse_forward for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc), with no handle.
//
// The only device memory these calls use beyond the caller's input and output
// is the split-row schedule's workspace: partial (max, sum) pairs and arrival
// counters. Here it is `scratch`, a file-scope device array of fixed size that
// every GPU the library runs on holds until the process ends. Its device
// address is looked up once per device (hipGetSymbolAddress, with the device
// current) and kept; kernels are given that address, never the array's name,
// which in host code is only a host-side stand-in.
//
// Every call on one GPU shares that GPU's scratch, which keeps the last call's
// contents. The pairs and arrival counters must be zero when a launch starts:
// they are cleared once per device by a small fill kernel on the first call's
// stream (again on later calls while the clearing launch was only captured
// into a graph), and every split launch leaves what it used zero. Calls that overlap on one
// GPU (two streams, two threads, two graphs replayed at once) race on the
// scratch and give wrong results; serialise them.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "lse.h"
#include "lse_launch.h"

namespace {

// Capacity: LSE_SPLIT_MAX_ROWS rows of LSE_SPLIT_MAX_PARTS (max, sum) pairs
// (512 KiB), then LSE_SPLIT_MAX_ROWS counters, each in its own 256 bytes
// (256 KiB): 768 KiB per GPU, the same as a handle's split-row workspace.
constexpr int64_t kPairs = int64_t{LSE_SPLIT_MAX_ROWS} * LSE_SPLIT_MAX_PARTS;
constexpr int64_t kPairBytes = kPairs * 8;
constexpr int64_t kCounterWordsAll = int64_t{LSE_SPLIT_MAX_ROWS} * lse::kCounterWords;
constexpr int64_t kScratchBytes = kPairBytes + kCounterWordsAll * 4;
static_assert(kScratchBytes == 768 * 1024, "scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    bool ready = false;     // address and CU count known
    bool cleared = false;   // pairs and counters zeroed by a launch that ran (not only captured)
    unsigned char* ptr = nullptr;  // this device's copy of `scratch`
    int n_cu = 0;
};

std::mutex g_mutex;
DeviceScratch g_dev[kMaxDevices];

__global__ void zero_words(unsigned* __restrict__ p, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = 0u;
}

// Look up this device's scratch (the current device must be `device`) and
// check that it is a gfx950; once per device.
lse_status_t set_up(int device, DeviceScratch& d) {
    if (d.ready) return LSE_OK;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return LSE_ERR_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return LSE_ERR_NO_DEVICE;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
        (void)hipGetLastError();
        return LSE_ERR_HIP;
    }
    d.ptr = static_cast<unsigned char*>(ptr);
    d.n_cu = prop.multiProcessorCount;
    d.ready = true;
    return LSE_OK;
}

}  // namespace

namespace lse {

// Set up the scratch of the current device `device` and clear it on
// `stream` if no launch has cleared it yet. Called by lse_create (with
// the null stream, which it then synchronises) and by the entry point.
lse_status_t noalloc_prepare(int device, hipStream_t stream, unsigned char** ptr, int* n_cu) {
    if (device < 0 || device >= kMaxDevices) return LSE_ERR_NO_DEVICE;
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceScratch& d = g_dev[device];
    lse_status_t st = set_up(device, d);
    if (st != LSE_OK) return st;
    if (!d.cleared) {
        hipLaunchKernelGGL(zero_words, dim3(64), dim3(256), 0, stream,
                           reinterpret_cast<unsigned*>(d.ptr), kScratchBytes / 4);
        if (hipGetLastError() != hipSuccess) return LSE_ERR_HIP;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
            (void)hipGetLastError();
            cs = hipStreamCaptureStatusActive;  // unknown: clear again next time
        }
        d.cleared = cs == hipStreamCaptureStatusNone;
    }
    if (ptr) *ptr = d.ptr;
    if (n_cu) *n_cu = d.n_cu;
    return LSE_OK;
}

}  // namespace lse

extern "C" lse_status_t lse_forward_noalloc(const void* x, lse_dtype_t dtype, int64_t rows,
                                            int64_t cols, int64_t row_stride, float* out,
                                            hipStream_t stream) {
    lse_status_t st = lse::check_forward(x, dtype, rows, cols, row_stride, out);
    if (st != LSE_OK || rows == 0) return st;
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) return LSE_ERR_NO_DEVICE;
    unsigned char* ptr = nullptr;
    int n_cu = 0;
    st = lse::noalloc_prepare(device, stream, &ptr, &n_cu);
    if (st != LSE_OK) return st;
    lse::ForwardContext c{};
    c.device = device;
    c.n_cu = n_cu;
    c.schedule = LSE_SCHED_AUTO;
    c.ws_pairs = reinterpret_cast<unsigned*>(ptr);
    c.counters = reinterpret_cast<unsigned*>(ptr + kPairBytes);
    c.pair_capacity = kPairs;
    c.counter_capacity = LSE_SPLIT_MAX_ROWS;
    return lse::run_forward(c, x, dtype, rows, cols, row_stride, out, nullptr, nullptr, stream);
}
