// A plain read of a device buffer, the measured ceiling for the weight stream: "Triton
// Kernel Matches bitsandbytes: Why Both Lose to Math", section "Roofline First: Calculate
// the Ceiling Before Writing Code", takes the measured bandwidth of the same machine (not
// the datasheet figure) as the roofline's denominator. The loads have the decode kernel's
// width (16 bytes per lane) and cache policy (non-temporal), with nothing else to do.
#include <hip/hip_runtime.h>

#include "w4a16_internal.h"

namespace w4a16 {

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;          // 16-byte loads in flight per lane
constexpr int kReadChunk = kReadThreads * kReadUnroll * 16;   // bytes per work-group: 16 KiB
constexpr int kCpolNt = 2;

// Work-group b reads bytes [b * 16 KiB, (b + 1) * 16 KiB) of the buffer (the last one less):
// lane l loads 16 bytes at l * 16 + u * 4 KiB, u = 0..3, so every load instruction of a
// wavefront covers 1 KiB of consecutive bytes. The XOR of everything a lane read is stored
// only if it equals a value the data cannot be expected to produce, which keeps the loads
// without writing anything in practice.
__global__ __launch_bounds__(kReadThreads) void read_kernel(const uint8_t* __restrict__ buf, int64_t bytes,
                                                            uint32_t* __restrict__ sink) {
    const int64_t base = (int64_t)blockIdx.x * kReadChunk;
    const int64_t left = bytes - base;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(buf + base), 0, (int)(left < kReadChunk ? left : kReadChunk), 0x00020000);
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
        // loads past the range end return 0
        const uint4 v = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(threadIdx.x * 16 + u * kReadThreads * 16), 0, kCpolNt));
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

}  // namespace

int launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
    const int64_t blocks = (bytes + kReadChunk - 1) / kReadChunk;
    hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(kReadThreads), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<const uint8_t*>(buf), bytes, sink);
    return (int)hipGetLastError();
}

}  // namespace w4a16
