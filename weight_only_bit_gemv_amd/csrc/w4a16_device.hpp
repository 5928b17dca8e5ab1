// Device helpers shared by every W4A16 kernel: nibble unpack, zero subtraction, fp16
// dequant and the matching activation permutation.
//
// A packed word holds 8 codes of one column for K = 8i .. 8i+7, nibble j at bit 4j
// ("Beating FP16 with 4-bit Weights: A Portable W4A16 GEMM in Triton", section "The
// design"). The unpack below builds fp16 numbers directly from the bits:
//   (w & 0x000F000F) | 0x64006400  ->  halves (1024 + q0, 1024 + q4)  (q in mantissa bits 0..3)
//   (w & 0x00F000F0) | 0x54005400  ->  halves (  64 + q1,   64 + q5)  (q in mantissa bits 4..7,
//                                      where one mantissa step of 2^6 is 1/16)
// and the same two masks on w >> 8 give (1024 + q2, 1024 + q6) and (64 + q3, 64 + q7).
// Subtracting (1024 + z) or (64 + z) in fp16 is exact for |z| <= 1024, so each lane holds
// q - z exactly, in the K order [0, 4, 1, 5, 2, 6, 3, 7]. A contraction over K may use any
// order as long as the activations use the same one: permute_x puts 8 consecutive fp16
// activations into that order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kMaskLo = 0x000F000Fu;
constexpr uint32_t kMaskHi = 0x00F000F0u;
constexpr uint32_t kBias1024 = 0x64006400u;   // fp16 1024.0 in both halves
constexpr uint32_t kBias64 = 0x54005400u;     // fp16 64.0 in both halves

// The two fp16 offsets subtracted from the biased codes of one column:
// lo = (1024 + z, 1024 + z), hi = (64 + z, 64 + z). Both sums are exact for |z| <= 1024.
struct ZeroOffsets {
    half2_t lo;
    half2_t hi;
};

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ __forceinline__ uint32_t as_u32(half2_t v) { return __builtin_bit_cast(uint32_t, v); }
// Bits of one fp16 value. Takes the value as a scalar: __builtin_bit_cast applied directly to
// a vector-element lvalue (v[e]) reads element 0 whatever e is, so never write that form.
__device__ __forceinline__ uint16_t f16_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }

__device__ __forceinline__ ZeroOffsets zero_offsets(_Float16 z) {
    ZeroOffsets o;
    const _Float16 a = (_Float16)1024.0f + z;
    const _Float16 b = (_Float16)64.0f + z;
    o.lo = half2_t{a, a};
    o.hi = half2_t{b, b};
    return o;
}

// The four unpack constants, held in VGPRs. gfx9 VOP3 instructions cannot take a 32-bit
// literal, so with the masks as literals the compiler would split every (w & m) | b into
// v_and_b32 + v_or_b32; with both in registers it emits one v_and_or_b32. The empty asm
// only hides the values from constant folding.
struct UnpackConsts {
    uint32_t mask_lo, mask_hi, bias1024, bias64;
};

__device__ __forceinline__ UnpackConsts unpack_consts() {
    UnpackConsts c{kMaskLo, kMaskHi, kBias1024, kBias64};
    asm volatile("" : "+v"(c.mask_lo), "+v"(c.mask_hi), "+v"(c.bias1024), "+v"(c.bias64));
    return c;
}

// q - z for the 8 codes of word w, exact fp16, K order [0, 4, 1, 5, 2, 6, 3, 7].
__device__ __forceinline__ half8_t unpack_sub(uint32_t w, ZeroOffsets zo, const UnpackConsts& c) {
    const uint32_t s = w >> 8;
    const half2_t d0 = as_h2((w & c.mask_lo) | c.bias1024) - zo.lo;   // q0, q4
    const half2_t d1 = as_h2((w & c.mask_hi) | c.bias64) - zo.hi;     // q1, q5
    const half2_t d2 = as_h2((s & c.mask_lo) | c.bias1024) - zo.lo;   // q2, q6
    const half2_t d3 = as_h2((s & c.mask_hi) | c.bias64) - zo.hi;     // q3, q7
    return half8_t{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
}

// fp16 dequant (q - z) * s: one rounding of the exact product.
__device__ __forceinline__ half8_t dequant_frag(uint32_t w, ZeroOffsets zo, _Float16 s,
                                                const UnpackConsts& c) {
    const half8_t d = unpack_sub(w, zo, c);
    const half8_t sv = half8_t{s, s, s, s, s, s, s, s};
    return d * sv;
}

// Position in natural K order (0..7) of element e of an unpacked fragment of a word packed
// in the linear layout (the interleaved layout's fragments are in natural order).
__device__ __forceinline__ constexpr int frag_k(int e) { return (e >> 1) + ((e & 1) << 2); }

// 8 consecutive fp16 activations (as 16 bytes) into the fragment K order.
__device__ __forceinline__ half8_t permute_x(uint4 v) {
    const half8_t h = __builtin_bit_cast(half8_t, v);
    return __builtin_shufflevector(h, h, 0, 4, 1, 5, 2, 6, 3, 7);
}

// The activation fragment matching an unpacked word. NAT: the words are packed in the
// interleaved layout (nibble p holds K offset (0, 2, 4, 6, 1, 3, 5, 7)[p]), whose unpack
// already yields natural K order, so the activations stay as they are.
template <bool NAT>
__device__ __forceinline__ half8_t x_frag(uint4 v) {
    if constexpr (NAT) return __builtin_bit_cast(half8_t, v);
    else return permute_x(v);
}

}  // namespace w4a16
