// The device unpack/dequant exposed on its own (w4a16_dequant), so that the codes and the
// fp16 weights the kernels work with can be compared bit for bit with the oracle.
//
// It uses the same helpers as the product kernels (w4a16_device.hpp): unpack_sub gives the
// exact fp16 (q - zero) of each code, dequant_frag its fp16 product with the scale, one
// rounding of the exact value ("Beating FP16 with 4-bit Weights: A Portable W4A16 GEMM in
// Triton", section "The design": dequant (w - zero) * scale in registers).
#include <hip/hip_runtime.h>

#include "w4a16_device.hpp"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {

// One thread per (packed row, 4-column quad).
__global__ __launch_bounds__(256) void dequant_kernel(const uint4* __restrict__ qw,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint16_t* __restrict__ zeros,
                                                      uint8_t* __restrict__ codes,
                                                      uint16_t* __restrict__ w, int N, int K,
                                                      int group_shift, int layout) {
    const int nq = N >> 2;
    const size_t total = (size_t)(K >> 3) * nq;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int i = (int)(idx / nq);                 // packed row
    const int n = (int)(idx % nq) * 4;             // first column
    const int grp = (i * 8) >> group_shift;
    const bool nat = layout == W4A16_LAYOUT_INTERLEAVED;   // fragments already in natural K order
    const uint4 wv = qw[idx];
    const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
    const uint2 sv = *reinterpret_cast<const uint2*>(scales + (size_t)grp * N + n);
    const uint2 zv = *reinterpret_cast<const uint2*>(zeros + (size_t)grp * N + n);
    const half2_t s01 = as_h2(sv.x), s23 = as_h2(sv.y);
    const half2_t z01 = as_h2(zv.x), z23 = as_h2(zv.y);
    const _Float16 sc[4] = {s01[0], s01[1], s23[0], s23[1]};
    const _Float16 zc[4] = {z01[0], z01[1], z23[0], z23[1]};
    const ZeroOffsets no_zero = zero_offsets((_Float16)0.0f);
    const UnpackConsts uc = unpack_consts();
    // element e of the four columns' fragments share one output row: one 4-byte (codes) or
    // 8-byte (weights) store per row
    if (codes) {
        half8_t q[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) q[t] = unpack_sub(words[t], no_zero, uc);       // q exactly
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t v = (uint32_t)(int)q[0][e] | ((uint32_t)(int)q[1][e] << 8) |
                               ((uint32_t)(int)q[2][e] << 16) | ((uint32_t)(int)q[3][e] << 24);
            *reinterpret_cast<uint32_t*>(codes + (size_t)(i * 8 + (nat ? e : frag_k(e))) * N + n) = v;
        }
    }
    if (w) {
        half8_t d[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) d[t] = dequant_frag(words[t], zero_offsets(zc[t]), sc[t], uc);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const half2_t lo = half2_t{d[0][e], d[1][e]}, hi = half2_t{d[2][e], d[3][e]};
            *reinterpret_cast<uint2*>(w + (size_t)(i * 8 + (nat ? e : frag_k(e))) * N + n) =
                make_uint2(as_u32(lo), as_u32(hi));
        }
    }
}

}  // namespace

int launch_dequant(const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                   uint8_t* codes, uint16_t* w, int N, int K, int group_shift, int layout, void* stream) {
    const size_t total = (size_t)(K >> 3) * (size_t)(N >> 2);
    const unsigned blocks = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL(dequant_kernel, dim3(blocks), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<const uint4*>(qweight), scales, zeros, codes, w, N, K, group_shift, layout);
    return (int)hipGetLastError();
}

}  // namespace w4a16
