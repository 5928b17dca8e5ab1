// Statically allocated split-K scratch for w4a16_matmul_noalloc: callers that cannot
// allocate device memory (code under HIP graph capture, serving loops, harnesses that forbid
// hipMalloc) get the same kernels with their fp32 partial sums and arrival counters in a
// file-scope device array instead of the library's per-stream workspace.
//
// The array's name is a host-side stand-in in host code, not a device address: its device
// address is taken once per device with hipGetSymbolAddress, with that device current, and
// only that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "w4a16_internal.h"

namespace w4a16 {

namespace {

// Layout: arrival counters first (zero between calls), then the fp32 partials.
static __device__ __align__(256) uint8_t scratch[kScratchCounterBytes + kScratchPartialBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices];            // device address of `scratch` per device, or null

__global__ __launch_bounds__(256) void zero_words(uint32_t* __restrict__ p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

}  // namespace

int scratch_workspace(void* stream, float** partials, uint32_t** counters) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_addr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        // the counters must start at zero; every kernel returns the counters it takes to
        // zero, so they are cleared once per device, with a kernel (not a memset node, which
        // graph capture would record) ordered before the first product on this stream
        constexpr int n = (int)(kScratchCounterBytes / 4);
        hipLaunchKernelGGL(zero_words, dim3((n + 255) / 256), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                           static_cast<uint32_t*>(ptr), n);
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
        g_addr[dev] = ptr;
    }
    uint8_t* base = static_cast<uint8_t*>(g_addr[dev]);
    *counters = reinterpret_cast<uint32_t*>(base);
    *partials = reinterpret_cast<float*>(base + kScratchCounterBytes);
    return (int)hipSuccess;
}

}  // namespace w4a16
