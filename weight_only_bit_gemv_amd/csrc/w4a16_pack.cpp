// Host quantiser / packer behind w4a16_pack and w4a16_unpack.
//
// "Beating FP16 with 4-bit Weights: A Portable W4A16 GEMM in Triton", section "The design":
// one scale and one zero-point per group of 128 rows (GPTQ/AWQ style) and eight 4-bit
// values packed into one int32 along the contraction dimension (packed row i, nibble j
// holds K index 8i + j). The quantiser is the asymmetric min/max one:
//   scale = fp16_rne((max - min) / 15)  (1.0 when that rounds to zero)
//   zero  = rne(-min / scale)           (stored as fp16, |zero| <= 1024)
//   q     = clamp(rne(w / scale) + zero, 0, 15)
// with every step an IEEE fp32 operation. Build with -ffp-contract=off and without
// fast-math so that no step is fused or reassociated.
//
// Symmetric mode (the +8 zero point of "Triton Kernel Matches bitsandbytes: Why Both Lose
// to Math", section "Three Kernel Versions and Two Bugs"):
//   scale = fp16_rne(max|w| / 7)        (1.0 when that rounds to zero)
//   zero  = 8
//   q     = clamp(rne(w / scale) + 8, 0, 15)
// Group sizes: any multiple of 8 rows here; the library accepts 32, 64, 128 and 256 (the
// GemLite README takes group sizes divisible by 32).
//
// Layouts: nibble j of a word holds K offset kNibbleK[layout][j] of its 8 K indices - j
// itself (linear), or (0, 2, 4, 6, 1, 3, 5, 7)[j] (interleaved, the pre-permuted order of
// "Beating FP16 with 4-bit Weights", section "What's next").
#include <cmath>
#include <cstdint>
#include <cstring>
#include <algorithm>
#include <thread>
#include <vector>

#include "w4a16_internal.h"

namespace w4a16 {

// fp32 -> fp16 bit pattern, round to nearest, ties to even (IEEE 754 binary16).
uint16_t f32_to_f16_rne(float f) {
    uint32_t x;
    std::memcpy(&x, &f, 4);
    const uint32_t sign = (x >> 16) & 0x8000u;
    const uint32_t ax = x & 0x7fffffffu;
    if (ax >= 0x7f800000u)                      // Inf or NaN
        return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? 0x0200u : 0u));
    if (ax >= 0x477ff000u)                      // >= 65520 rounds to infinity
        return (uint16_t)(sign | 0x7c00u);
    if (ax < 0x38800000u) {                     // below 2^-14: fp16 subnormal or zero
        const uint32_t e = ax >> 23;            // biased fp32 exponent
        if (e < 102) return (uint16_t)sign;     // below 2^-25 -> 0 (2^-25 itself ties to 0)
        const uint32_t m = (ax & 0x7fffffu) | 0x800000u;
        const uint32_t shift = 126 - e;         // value / 2^-24 = m >> shift (14..24)
        uint32_t q = m >> shift;
        const uint32_t rem = m & ((1u << shift) - 1u);
        const uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (q & 1u))) ++q;
        return (uint16_t)(sign | q);            // q == 0x400 is the smallest normal
    }
    const uint32_t e = (ax >> 23) - 127 + 15;
    const uint32_t m = ax & 0x7fffffu;
    uint32_t h = (e << 10) | (m >> 13);
    const uint32_t rem = m & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;   // carry may bump the exponent
    return (uint16_t)(sign | h);
}

// fp16 bit pattern -> fp32 (exact).
float f16_to_f32(uint16_t h) {
    const uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    const uint32_t e = (h >> 10) & 0x1fu;
    const uint32_t m = h & 0x3ffu;
    uint32_t bits;
    if (e == 0) {
        const float v = std::ldexp((float)m, -24);
        std::memcpy(&bits, &v, 4);
        bits |= sign;
    } else if (e == 31) {
        bits = sign | 0x7f800000u | (m << 13);
    } else {
        bits = sign | ((e - 15 + 127) << 23) | (m << 13);
    }
    float f;
    std::memcpy(&f, &bits, 4);
    return f;
}

namespace {

constexpr int kCols = 64;   // columns per work item of the packer's threads

// Quantise and pack columns [n0, n1) of every K-group. Returns W4A16_OK or an error.
int pack_columns(const float* W, int64_t K, int64_t N, int64_t g, bool symmetric, const int* nibble_k,
                 int64_t n0, int64_t n1, int32_t* qweight, uint16_t* scales, uint16_t* zeros) {
    const int64_t nc = n1 - n0;
    float mn[kCols], mx[kCols], s[kCols], z[kCols];
    uint8_t q[kCols * 8];
    for (int64_t grp = 0; grp < K / g; ++grp) {
        const float* Wg = W + grp * g * N;
        for (int64_t c = 0; c < nc; ++c) { mn[c] = Wg[n0 + c]; mx[c] = Wg[n0 + c]; }
        for (int64_t r = 1; r < g; ++r) {
            const float* row = Wg + r * N + n0;
            for (int64_t c = 0; c < nc; ++c) {
                mn[c] = std::min(mn[c], row[c]);
                mx[c] = std::max(mx[c], row[c]);
            }
        }
        for (int64_t c = 0; c < nc; ++c) {
            const float s32 = symmetric ? std::max(std::fabs(mn[c]), std::fabs(mx[c])) / 7.0f
                                        : (mx[c] - mn[c]) / 15.0f;
            uint16_t s16 = f32_to_f16_rne(s32);
            if ((s16 & 0x7c00u) == 0x7c00u) return W4A16_ERR_NONFINITE;
            if ((s16 & 0x7fffu) == 0) s16 = 0x3c00u;             // 1.0 for a zero scale
            s[c] = f16_to_f32(s16);
            z[c] = symmetric ? 8.0f : std::rint(-mn[c] / s[c]);
            if (std::fabs(z[c]) > 1024.0f) return W4A16_ERR_UNSUPPORTED;
            scales[grp * N + n0 + c] = s16;
            zeros[grp * N + n0 + c] = f32_to_f16_rne(z[c]);
        }
        for (int64_t i = 0; i < g / 8; ++i) {                    // packed rows of the group
            for (int j = 0; j < 8; ++j) {
                const float* row = Wg + (i * 8 + j) * N + n0;
                for (int64_t c = 0; c < nc; ++c) {
                    float v = std::rint(row[c] / s[c]) + z[c];
                    v = std::min(std::max(v, 0.0f), 15.0f);
                    q[c * 8 + j] = (uint8_t)v;
                }
            }
            int32_t* out = qweight + (grp * (g / 8) + i) * N + n0;
            for (int64_t c = 0; c < nc; ++c) {
                uint32_t w = 0;
                for (int j = 0; j < 8; ++j) w |= (uint32_t)q[c * 8 + nibble_k[j]] << (4 * j);
                out[c] = (int32_t)w;
            }
        }
    }
    return W4A16_OK;
}

}  // namespace

int pack_host(const float* W, int64_t K, int64_t N, int64_t g, bool symmetric, int layout,
              int32_t* qweight, uint16_t* scales, uint16_t* zeros) {
    // Reject non-finite input up front so that no output is written on that error.
    {
        const int64_t total = K * N;
        for (int64_t i = 0; i < total; ++i)
            if (!std::isfinite(W[i])) return W4A16_ERR_NONFINITE;
    }
    const int64_t chunks = (N + kCols - 1) / kCols;
    unsigned hw = std::thread::hardware_concurrency();
    if (hw == 0) hw = 1;
    const int64_t nthreads = std::min<int64_t>(std::min<int64_t>(hw, 64), chunks);
    std::vector<int> status(nthreads > 0 ? nthreads : 1, W4A16_OK);
    auto work = [&](int64_t t) {
        for (int64_t ch = t; ch < chunks; ch += nthreads) {
            const int64_t n0 = ch * kCols;
            const int64_t n1 = std::min<int64_t>(N, n0 + kCols);
            const int rc = pack_columns(W, K, N, g, symmetric, kNibbleK[layout], n0, n1, qweight, scales, zeros);
            if (rc != W4A16_OK) { status[t] = rc; return; }
        }
    };
    if (nthreads <= 1) {
        work(0);
    } else {
        std::vector<std::thread> pool;
        pool.reserve(nthreads);
        for (int64_t t = 0; t < nthreads; ++t) pool.emplace_back(work, t);
        for (auto& th : pool) th.join();
    }
    // Report the error of the lowest-numbered failing thread (deterministic choice).
    for (int rc : status)
        if (rc != W4A16_OK) return rc;
    return W4A16_OK;
}

void unpack_host(const int32_t* qweight, int64_t K, int64_t N, int layout, uint8_t* codes) {
    const int* nk = kNibbleK[layout];
    for (int64_t i = 0; i < K / 8; ++i)
        for (int64_t n = 0; n < N; ++n) {
            const uint32_t w = (uint32_t)qweight[i * N + n];
            for (int j = 0; j < 8; ++j) codes[(i * 8 + nk[j]) * N + n] = (uint8_t)((w >> (4 * j)) & 0xFu);
        }
}

}  // namespace w4a16
