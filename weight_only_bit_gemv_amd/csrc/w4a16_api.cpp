// C ABI of the W4A16 library: argument validation, the shape-based dispatcher, and the
// library-owned split-K workspace. Declarations and contracts are in include/w4a16.h.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <vector>
#include <utility>

#include "w4a16_internal.h"

namespace {

thread_local std::string g_detail;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_detail = buf;
    return code;
}

int ok() {
    g_detail.clear();
    return W4A16_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shape checks shared by the GPU entry points.
int check_gpu_shape(int64_t M, int64_t N, int64_t K, int64_t group_size) {
    if (M < 1 || N < 1 || K < 1) return fail(W4A16_ERR_INVALID_ARG, "M, N, K must be >= 1 (got %lld, %lld, %lld)",
                                            (long long)M, (long long)N, (long long)K);
    if (!w4a16::group_supported(group_size))
        return fail(W4A16_ERR_UNSUPPORTED, "group_size %lld not supported (32, 64, 128 or 256)",
                    (long long)group_size);
    if (K % group_size != 0 || K % 128 != 0)
        return fail(W4A16_ERR_UNSUPPORTED, "K=%lld must be a multiple of 128 and of group_size", (long long)K);
    if (N % 4 != 0) return fail(W4A16_ERR_UNSUPPORTED, "N=%lld is not a multiple of 4", (long long)N);
    const int64_t lim = INT32_MAX;
    if ((K / 8) * N > lim || M * K > lim || M * N > lim)
        return fail(W4A16_ERR_UNSUPPORTED, "problem too large for 32-bit indexing");
    return W4A16_OK;
}

// ---- dispatcher --------------------------------------------------------------------------

// Skinny-kernel plans. Autotuned per shape (the pages tune block sizes and split factors per
// shape and cache the winner: "Things I got wrong along the way" on the Triton W4A16 page):
// kTuned holds, for the projection shapes of the decode, MoE-expert and prefill workloads,
// the fastest plan of a sweep of cols x waves x kc x seg on MI355X (graph-timed launches
// after a clock warm-up, weights rotated over 600 MB), per M bucket (the decode-sweep and
// MoE shapes re-swept on the current kernel, 180-243 plans each; entries marked re-swept
// won an alternating A/B against the earlier plan), and for the projections of 34 other
// decoder shapes (K and N from 512 to 18944: narrow key/value projections, 4864- to
// 18944-wide feed-forward layers and their transposes; 72 plans each at 4-step segments, the
// earlier rule's plan timed beside them) and the summed N of the grouped launches of the
// benchmarks (gate+up of 4096 x 14336, experts' gate+up and down) and one GPU's share of
// the decode shapes split by columns over 8 GPUs: an entry covers M up to m_max and above the
// previous entry's m_max. Other shapes take a rule fitted to those sweeps, for M <= 16 (on
// those 34 shapes its plans are on average 3 % (K <= 4096) and 9 % (deeper K) slower than
// each shape's best, against 8 % and 25 % for the rule before it; fitted on half of the
// shapes, it is 2-5 % and 9-12 % slower on the other half):
//  * K <= 4096: one work-group covers K, at M = 1 with 16 wavefronts (K = 4096), 8 (K = 2048
//    to 4095) or 4 (shorter K), at larger M or N >= 16384 (256 or more 64-column strips) with
//    4; strips of 16 columns up to N = 4096, 32 up to 8192, 64 beyond;
//  * deeper K: 12 K-steps per wavefront and 8 wavefronts at M = 1, 16 K-steps and 4
//    wavefronts above, K split over work-groups; strips of 16 columns up to N = 1024, 32 up
//    to 4096, 64 beyond.
// Past M = 16, where no sweep of the rule was made, the earlier rule stays: 64-column strips
// for wide or deep matrices, 16 otherwise (32 past M = 32), 4 wavefronts, 32 K-steps per
// wavefront (fewer when K is short, so that one work-group covers K).
struct TunedPlan {
    int32_t K, N, m_max;
    int8_t cols, waves, kc, seg;
};

const TunedPlan kTuned[] = {
    //  K       N      m_max cols waves kc seg      time of the plan in the sweep
    {  768,   2048,  1, 16,  4,  8, 4},   // 2.93 us (re-swept: 2.98 us before)
    {  768,   2048,  4, 16,  4,  8, 4},   // 3.11 us
    {  768,   2048, 16, 16,  4,  8, 4},   // 3.41 us
    {  768,  16384,  1, 32,  8,  4, 4},   // 4.19 us (summed N of a grouped launch)
    {  768,  16384,  4, 32,  4,  8, 4},   // 4.43 us (summed N of a grouped launch)
    {  768,  16384, 16, 64,  4,  8, 4},   // 4.70 us (summed N of a grouped launch)
    {  896,   4864,  1, 32,  4,  8, 4},   // 3.47 us (earlier rule for other shapes: 3.48 us)
    {  896,   4864,  4, 32,  4,  8, 4},   // 3.72 us (earlier rule for other shapes: 3.72 us)
    {  896,   4864, 16, 32,  4,  8, 4},   // 3.94 us (earlier rule for other shapes: 3.94 us)
    { 1024,   4096,  1, 16,  4,  8, 4},   // 3.07 us (earlier rule for other shapes: 3.08 us)
    { 1024,   4096,  4, 16,  4,  8, 4},   // 3.40 us (earlier rule for other shapes: 3.40 us)
    { 1024,   4096, 16, 16,  4,  8, 4},   // 3.85 us (earlier rule for other shapes: 3.86 us)
    { 1408,   2048,  1, 16, 16,  4, 4},   // 3.32 us
    { 1408,   2048,  4, 16,  8,  8, 4},   // 3.74 us
    { 1408,   2048, 16, 16,  4, 12, 4},   // 4.20 us (re-swept: 4.32 us before)
    { 1408,   8192,  1, 32,  4, 12, 4},   // 4.09 us (summed N of a grouped launch)
    { 1408,   8192,  4, 32,  4, 12, 4},   // 4.39 us (summed N of a grouped launch)
    { 1408,   8192, 16, 32,  4, 12, 4},   // 4.72 us (summed N of a grouped launch)
    { 1408,  16384,  1, 64,  4, 12, 4},   // 5.07 us (summed N of a grouped launch)
    { 1408,  16384,  4, 64,  4, 12, 4},   // 5.47 us (summed N of a grouped launch)
    { 1408,  16384, 16, 64,  4, 12, 4},   // 5.67 us (summed N of a grouped launch)
    { 1536,   8960,  1, 64,  4, 12, 4},   // 4.63 us (earlier rule for other shapes: 4.63 us)
    { 1536,   8960,  4, 64,  4, 12, 4},   // 5.09 us (earlier rule for other shapes: 5.14 us)
    { 1536,   8960, 16, 64,  4, 12, 4},   // 5.47 us (earlier rule for other shapes: 5.48 us)
    { 2048,    512,  1, 16,  8,  8, 4},   // 3.47 us (earlier rule for other shapes: 3.74 us)
    { 2048,    512,  4, 16,  8,  8, 4},   // 3.91 us (earlier rule for other shapes: 4.04 us)
    { 2048,    512, 16, 16,  4, 16, 4},   // 4.76 us (earlier rule for other shapes: 4.76 us)
    { 2048,    768,  1, 16,  8,  8, 4},   // 3.08 us
    { 2048,    768,  4, 16,  8,  8, 4},   // 3.94 us (re-swept: 4.09 us before)
    { 2048,    768, 16, 16,  4, 24, 8},   // 4.80 us (re-swept: 4.90 us before)
    { 2048,   1408,  1, 16,  8,  8, 4},   // 3.41 us
    { 2048,   1408,  4, 16,  4, 16, 8},   // 3.92 us (re-swept: 4.07 us before)
    { 2048,   1408, 16, 16,  4, 24, 8},   // 4.88 us (re-swept: 4.93 us before)
    { 2048,   2048,  1, 16,  8,  8, 4},   // 3.57 us (earlier rule for other shapes: 3.86 us)
    { 2048,   2048,  4, 16,  8,  8, 4},   // 4.07 us (earlier rule for other shapes: 4.19 us)
    { 2048,   2048, 16, 16,  4, 16, 4},   // 4.88 us (earlier rule for other shapes: 4.88 us)
    { 2048,   8192,  1, 32, 16,  4, 4},   // 4.58 us (earlier rule for other shapes: 5.37 us)
    { 2048,   8192,  4, 32,  8,  8, 4},   // 5.02 us (earlier rule for other shapes: 5.76 us)
    { 2048,   8192, 16, 32,  8,  8, 4},   // 5.62 us (earlier rule for other shapes: 6.21 us)
    { 2048,  11264,  1, 64,  8,  8, 4},   // 5.44 us (summed N of a grouped launch)
    { 2048,  11264,  4, 64,  4, 16, 4},   // 5.91 us (summed N of a grouped launch)
    { 2048,  11264, 16, 64,  4, 16, 4},   // 6.48 us (summed N of a grouped launch)
    { 2048,  12288,  1, 64,  8,  8, 4},   // 5.61 us (summed N of a grouped launch)
    { 2048,  12288,  4, 64,  4, 16, 4},   // 6.06 us (summed N of a grouped launch)
    { 2048,  12288, 16, 64,  4, 16, 4},   // 6.80 us (summed N of a grouped launch)
    { 2560,  10240,  1, 64,  4, 20, 4},   // 6.10 us (earlier rule for other shapes: 6.10 us)
    { 2560,  10240,  4, 64,  4, 20, 4},   // 6.45 us (earlier rule for other shapes: 6.45 us)
    { 2560,  10240, 16, 64,  4, 20, 4},   // 7.46 us (earlier rule for other shapes: 7.46 us)
    { 3072,   3072,  1, 16, 16,  8, 4},   // 4.23 us (earlier rule for other shapes: 5.47 us)
    { 3072,   3072,  4, 16,  8, 12, 4},   // 4.79 us (earlier rule for other shapes: 5.74 us)
    { 3072,   3072, 16, 16,  4, 24, 4},   // 6.03 us (earlier rule for other shapes: 6.56 us)
    { 3072,   8192,  1, 32,  8, 12, 4},   // 5.51 us (earlier rule for other shapes: 5.81 us)
    { 3072,   8192,  4, 32,  8, 12, 4},   // 5.98 us (earlier rule for other shapes: 6.04 us)
    { 3072,   8192, 16, 32,  4, 24, 4},   // 6.82 us (earlier rule for other shapes: 6.82 us)
    { 3584,  18944,  1, 64,  4,  8, 4},   // 11.13 us (earlier rule for other shapes: 11.74 us)
    { 3584,  18944,  4, 64,  4,  8, 4},   // 11.54 us (earlier rule for other shapes: 12.34 us)
    { 3584,  18944, 16, 64,  4,  8, 4},   // 13.27 us (earlier rule for other shapes: 14.85 us)
    { 4096,    512,  1, 16, 16,  8, 4},   // 4.49 us (earlier rule for other shapes: 5.23 us)
    { 4096,    512,  4, 16,  4,  8, 4},   // 5.03 us (earlier rule for other shapes: 5.54 us)
    { 4096,    512, 16, 16,  4,  8, 4},   // 5.57 us (earlier rule for other shapes: 6.88 us)
    { 4096,   1024,  1, 16, 16,  8, 4},   // 4.57 us (earlier rule for other shapes: 5.28 us)
    { 4096,   1024,  4, 16,  8, 16, 4},   // 5.35 us (earlier rule for other shapes: 5.57 us)
    { 4096,   1024, 16, 32,  4,  8, 4},   // 6.00 us (earlier rule for other shapes: 6.90 us)
    { 4096,   1792,  1, 16, 16,  8, 4},   // 4.65 us (one GPU's column share of 8)
    { 4096,   1792,  4, 16,  8, 16, 4},   // 5.43 us (one GPU's column share of 8)
    { 4096,   1792, 16, 32,  4,  8, 4},   // 6.33 us (one GPU's column share of 8)
    { 4096,   2048,  1, 16, 16,  8, 4},   // 4.71 us (earlier rule for other shapes: 5.42 us)
    { 4096,   2048,  4, 16,  8, 16, 4},   // 5.43 us (earlier rule for other shapes: 5.73 us)
    { 4096,   2048, 16, 32,  4, 12, 4},   // 6.54 us (earlier rule for other shapes: 6.97 us)
    { 4096,   3072,  1, 16, 16,  8, 4},   // 4.78 us (earlier rule for other shapes: 6.40 us)
    { 4096,   3072,  4, 16,  8, 16, 4},   // 5.53 us (earlier rule for other shapes: 6.63 us)
    { 4096,   3072, 16, 32,  4,  8, 4},   // 6.98 us (earlier rule for other shapes: 7.74 us)
    { 4096,   4096,  1, 16, 16,  8, 4},   // 4.88 us
    { 4096,   4096,  2, 16, 16,  8, 4},   // 5.18 us
    { 4096,   4096,  4, 16,  8, 16, 4},   // 5.72 us
    { 4096,   4096,  8, 16,  4, 32, 4},   // 6.00 us (re-swept: 6.13 us before)
    { 4096,   4096, 16, 16,  4, 32, 4},   // 7.22 us
    { 4096,   4096, 32, 64,  4,  8, 2},   // 9.71 us (4 splits)
    { 4096,   4096, 64, 32,  4, 48, 4},   // 11.79 us
    { 4096,   6144,  1, 32, 16,  8, 4},   // 6.23 us (earlier rule for other shapes: 7.36 us)
    { 4096,   6144,  4, 32,  4, 32, 4},   // 6.88 us (earlier rule for other shapes: 8.25 us)
    { 4096,   6144, 16, 32,  4, 32, 4},   // 8.13 us (earlier rule for other shapes: 11.59 us)
    { 4096,   8192,  1, 32, 16,  8, 4},   // 6.43 us (earlier rule for other shapes: 7.71 us)
    { 4096,   8192,  4, 32,  4, 32, 4},   // 6.93 us (earlier rule for other shapes: 8.04 us)
    { 4096,   8192, 16, 32,  4, 32, 4},   // 8.03 us (earlier rule for other shapes: 9.01 us)
    { 4096,  11008,  1, 64, 16,  8, 4},   // 7.82 us (earlier rule for other shapes: 8.02 us)
    { 4096,  11008,  4, 64,  4, 32, 4},   // 8.38 us (earlier rule for other shapes: 8.40 us)
    { 4096,  11008, 16, 64,  4, 32, 4},   // 9.76 us (earlier rule for other shapes: 9.76 us)
    { 4096,  12288,  1, 64, 16,  8, 4},   // 8.28 us (q, k, v of 4096 x 4096 in one grouped launch)
    { 4096,  12288,  4, 64,  4, 32, 4},   // 8.60 us (summed N of a grouped launch)
    { 4096,  12288, 16, 64,  4, 32, 4},   // 10.20 us (summed N of a grouped launch)
    { 4096,  14336,  1, 64,  4, 32, 4},   // 9.01 us
    { 4096,  14336,  2, 64,  4, 32, 4},   // 9.13 us
    { 4096,  14336,  4, 64,  4, 32, 4},   // 9.30 us
    { 4096,  14336,  8, 64,  4, 32, 4},   // 9.69 us
    { 4096,  14336, 16, 64,  4, 32, 4},   // 10.35 us
    { 4096,  14336, 32, 64,  4, 32, 4},   // 14.79 us
    { 4096,  14336, 64, 64,  4, 48, 4},   // 23.98 us
    { 4096,  16032,  1, 64,  8, 32, 4},   // 8.88 us (one GPU's column share of 8)
    { 4096,  16032,  4, 64,  4, 32, 4},   // 9.05 us (one GPU's column share of 8)
    { 4096,  16032, 16, 64,  4, 32, 4},   // 9.99 us (one GPU's column share of 8)
    { 4096,  28672,  1, 64,  4, 32, 4},   // 14.44 us (summed N of a grouped launch)
    { 4096,  28672,  4, 64,  4, 32, 4},   // 15.23 us (summed N of a grouped launch)
    { 4096,  28672, 16, 64,  4, 32, 4},   // 18.40 us (summed N of a grouped launch)
    { 4096, 128256,  1, 64,  8, 28, 4},   // 47.1 us (re-swept: 47.6 us before)
    { 4864,    896,  1, 16,  8,  8, 4},   // 5.19 us (earlier rule for other shapes: 5.51 us)
    { 4864,    896,  4, 16,  8,  8, 4},   // 5.69 us (earlier rule for other shapes: 5.83 us)
    { 4864,    896, 16, 16,  4, 12, 4},   // 6.21 us (earlier rule for other shapes: 6.51 us)
    { 5120,   1024,  1, 16,  8,  8, 4},   // 5.17 us (earlier rule for other shapes: 6.75 us)
    { 5120,   1024,  4, 16,  8,  8, 4},   // 5.62 us (earlier rule for other shapes: 7.04 us)
    { 5120,   1024, 16, 16,  4, 12, 4},   // 6.32 us (earlier rule for other shapes: 8.48 us)
    { 5120,   5120,  1, 32, 16, 12, 4},   // 7.34 us (earlier rule for other shapes: 9.56 us)
    { 5120,   5120,  4, 32,  4, 12, 4},   // 7.82 us (earlier rule for other shapes: 10.45 us)
    { 5120,   5120, 16, 64,  4, 16, 4},   // 8.36 us (earlier rule for other shapes: 14.99 us)
    { 5120,  13824,  1, 64,  8, 24, 4},   // 10.53 us (earlier rule for other shapes: 12.27 us)
    { 5120,  13824,  4, 64,  4, 48, 4},   // 10.74 us (earlier rule for other shapes: 12.71 us)
    { 5120,  13824, 16, 64,  4, 48, 4},   // 11.82 us (earlier rule for other shapes: 15.14 us)
    { 6144,   4096,  1, 16, 16, 12, 4},   // 6.23 us (earlier rule for other shapes: 7.86 us)
    { 6144,   4096,  4, 16,  8, 24, 4},   // 7.17 us (earlier rule for other shapes: 8.53 us)
    { 6144,   4096, 16, 64,  4, 12, 4},   // 8.22 us (earlier rule for other shapes: 11.22 us)
    { 7168,   1024,  1, 16,  8,  8, 4},   // 5.49 us (earlier rule for other shapes: 6.00 us)
    { 7168,   1024,  4, 16,  8,  8, 4},   // 5.82 us (earlier rule for other shapes: 6.15 us)
    { 7168,   1024, 16, 16,  4, 16, 4},   // 6.79 us (earlier rule for other shapes: 6.79 us)
    { 8192,   1024,  1, 16,  8,  8, 4},   // 5.76 us (earlier rule for other shapes: 8.87 us)
    { 8192,   1024,  4, 16,  8,  8, 4},   // 6.19 us (earlier rule for other shapes: 9.32 us)
    { 8192,   1024, 16, 16,  4, 16, 4},   // 7.07 us (earlier rule for other shapes: 10.10 us)
    { 8192,   2048,  1, 16,  8,  8, 4},   // 6.27 us (earlier rule for other shapes: 9.04 us)
    { 8192,   2048,  4, 16,  8,  8, 4},   // 6.79 us (earlier rule for other shapes: 9.46 us)
    { 8192,   2048, 16, 32,  8,  8, 4},   // 7.99 us (earlier rule for other shapes: 10.27 us)
    { 8192,   3072,  1, 16, 16, 16, 4},   // 7.18 us (earlier rule for other shapes: 7.77 us)
    { 8192,   3072,  4, 64,  4, 16, 4},   // 8.06 us (earlier rule for other shapes: 8.21 us)
    { 8192,   3072, 16, 64,  4, 16, 4},   // 8.35 us (earlier rule for other shapes: 9.51 us)
    { 8192,   4096,  1, 16, 16, 16, 4},   // 7.45 us (earlier rule for other shapes: 9.27 us)
    { 8192,   4096,  4, 32,  8,  8, 4},   // 8.46 us (earlier rule for other shapes: 9.79 us)
    { 8192,   4096, 16, 64,  4, 16, 4},   // 8.90 us (earlier rule for other shapes: 10.65 us)
    { 8192,   8192,  1, 32, 16, 16, 4},   // 10.61 us
    { 8192,   8192, 16, 32,  4, 64, 4},   // 13.64 us
    { 8192,   8192, 32, 64,  4, 32, 4},   // 20.16 us
    { 8192,   8192, 64, 64,  4, 32, 4},   // 33.84 us
    { 8192,  28672,  1, 64,  4, 64, 4},   // 26.94 us
    { 8192,  28672, 16, 64,  4, 64, 4},   // 33.76 us
    { 8192,  28672, 32, 64,  4, 64, 4},   // 48.56 us
    { 8192,  28672, 64, 64,  4, 64, 4},   // 80.77 us
    { 8960,   1536,  1, 16, 16,  8, 4},   // 6.40 us (earlier rule for other shapes: 6.97 us)
    { 8960,   1536,  4, 16,  8,  8, 4},   // 7.12 us (earlier rule for other shapes: 7.36 us)
    { 8960,   1536, 16, 32,  4, 16, 4},   // 7.90 us (earlier rule for other shapes: 8.88 us)
    {10240,   2560,  1, 32,  8, 12, 4},   // 7.73 us (earlier rule for other shapes: 8.33 us)
    {10240,   2560,  4, 32,  8, 12, 4},   // 8.25 us (earlier rule for other shapes: 8.71 us)
    {10240,   2560, 16, 64,  4, 16, 4},   // 9.34 us (earlier rule for other shapes: 10.66 us)
    {11008,   4096,  1, 64,  4, 24, 4},   // 9.11 us (earlier rule for other shapes: 9.75 us)
    {11008,   4096,  4, 64,  4, 24, 4},   // 9.59 us (earlier rule for other shapes: 10.16 us)
    {11008,   4096, 16, 64,  4, 24, 4},   // 10.03 us (earlier rule for other shapes: 10.99 us)
    {12288,   4096,  1, 64,  4, 24, 4},   // 9.48 us (earlier rule for other shapes: 10.20 us)
    {12288,   4096,  4, 64,  4, 24, 4},   // 9.89 us (earlier rule for other shapes: 10.66 us)
    {12288,   4096, 16, 64,  4, 24, 4},   // 10.38 us (earlier rule for other shapes: 12.86 us)
    {13824,   5120,  1, 64,  4, 12, 4},   // 12.10 us (earlier rule for other shapes: 12.59 us)
    {13824,   5120,  4, 64,  4, 48, 4},   // 12.51 us (earlier rule for other shapes: 13.26 us)
    {13824,   5120, 16, 64,  4, 12, 4},   // 14.26 us (earlier rule for other shapes: 15.39 us)
    {14336,    512,  1, 16, 16,  8, 4},   // 6.07 us (one GPU's column share of 8)
    {14336,    512,  4, 16,  8,  8, 4},   // 6.64 us (one GPU's column share of 8)
    {14336,    512, 16, 16,  4, 16, 4},   // 7.47 us (one GPU's column share of 8)
    {14336,   4096,  1, 64,  4, 28, 4},   // 10.56 us (4 splits of 112 K-steps)
    {14336,   4096,  2, 64,  4, 28, 4},   // 10.72 us
    {14336,   4096,  4, 64,  4, 28, 4},   // 11.04 us
    {14336,   4096,  8, 64,  4, 28, 4},   // 11.09 us
    {14336,   4096, 16, 64,  4, 28, 4},   // 11.65 us
    {14336,   4096, 32, 64,  4, 28, 4},   // 16.54 us
    {14336,   4096, 64, 64,  4, 28, 4},   // 26.29 us
    {16384,   1024,  1, 16, 16,  8, 4},   // 6.68 us (earlier rule for other shapes: 9.29 us)
    {16384,   1024,  4, 16,  8, 16, 4},   // 7.23 us (earlier rule for other shapes: 9.67 us)
    {16384,   1024, 16, 32,  4, 16, 4},   // 8.49 us (earlier rule for other shapes: 10.44 us)
    {18944,   3584,  1, 64, 16, 12, 4},   // 12.11 us (earlier rule for other shapes: 14.37 us)
    {18944,   3584,  4, 64,  4, 48, 4},   // 12.86 us (earlier rule for other shapes: 14.97 us)
    {18944,   3584, 16, 64,  4, 16, 4},   // 14.49 us (earlier rule for other shapes: 17.27 us)
    {28672,   8192,  1, 64,  8, 56, 4},   // 23.5 us (re-swept: 25.6 us before; 2 even splits of 448 K-steps)
    {28672,   8192, 16, 64,  8, 56, 4},   // 29.4 us at M = 16 (re-swept: 31.6 us before)
    {28672,   8192, 32, 64,  8, 64, 4},   // 53.76 us
    {28672,   8192, 64, 64,  4, 64, 4},   // 101.19 us
};

const TunedPlan* tuned_plan(int64_t M, int64_t N, int64_t K) {
    for (const TunedPlan& t : kTuned)
        if (t.K == K && t.N == N && M <= t.m_max) return &t;
    return nullptr;
}

}  // namespace

namespace w4a16 {

// Built configurations of the decode kernel (the instances in w4a16_skinny_lw{1,2,4}.hip);
// host logic only, shared by plan completion and the launcher.
bool skinny_config_supported(int row_tiles, int waves, int lw, int seg, int seg_group) {
    if (lw != 1 && lw != 2 && lw != 4) return false;
    if (seg != 1 && seg != 2 && seg != 4 && seg != 8) return false;
    // built (segment, K-steps of one group in it) pairs: every segment inside one group,
    // 4-step segments over 2 or 4 groups (64- and 32-row groups), 8-step over 2 groups
    if (!(seg_group == seg || (seg == 4 && (seg_group == 1 || seg_group == 2)) ||
          (seg == 2 && seg_group == 1) || (seg == 8 && seg_group == 4)))
        return false;
    if (seg == 8 && seg_group == 8) return false;
    if (waves != 4 && waves != 8 && waves != 16) return false;
    if (row_tiles < 1 || row_tiles > (lw == 4 ? 4 : 2)) return false;
    // built (row_tiles, waves) pairs: the LDS of the wave reduction, (waves - 1) * 16 *
    // row_tiles rows of 16 * lw floats, stays within 64 KiB, and register use stays low
    // enough for at least two work-groups' worth of waves per compute unit
    if (row_tiles >= 3 && waves != 4) return false;
    if (row_tiles == 2 && waves == 16) return false;
    return (waves - 1) * 16 * row_tiles * 16 * lw * 4 <= 64 * 1024;
}

}  // namespace w4a16

namespace {

int64_t roundup4(int64_t v) { return ceil_div(v, 4) * 4; }

void default_skinny_plan(int64_t M, int64_t N, int64_t K, int64_t group_steps, w4a16_plan_t* pl) {
    const TunedPlan* t = tuned_plan(M, N, K);
    const int64_t KS = K / w4a16::kKStep;
    if (t) {
        if (pl->cols == 0) pl->cols = t->cols;
        if (pl->waves == 0) pl->waves = t->waves;
        if (pl->kc == 0) pl->kc = t->kc;
    } else if (M <= 16 && KS <= 4 * 32) {
        // one work-group covers K; at M = 1 with about 8 K-steps per wavefront (short chains)
        if (pl->cols == 0) pl->cols = N <= 4096 ? 16 : N <= 8192 ? 32 : 64;
        if (pl->waves == 0) pl->waves = M > 1 || N >= 16384 ? 4 : KS >= 128 ? 16 : KS >= 64 ? 8 : 4;
        if (pl->kc == 0) pl->kc = (int32_t)std::max<int64_t>(4, roundup4(ceil_div(KS, pl->waves)));
    } else if (M <= 16) {
        // K is split over work-groups
        if (pl->cols == 0) pl->cols = N <= 1024 ? 16 : N <= 4096 ? 32 : 64;
        if (pl->waves == 0) pl->waves = M <= 1 ? 8 : 4;
        if (pl->kc == 0) pl->kc = M <= 1 ? 12 : 16;
    } else {
        if (pl->cols == 0) pl->cols = (N >= 8192 || K >= 8192) ? 64 : (M > 32 ? 32 : 16);
        if (pl->waves == 0) pl->waves = 4;
        if (pl->kc == 0)
            pl->kc = (int32_t)(KS <= 4 * 32 ? std::max<int64_t>(4, roundup4(ceil_div(KS, pl->waves))) : 32);
    }
    if (pl->seg == 0) {
        int32_t seg = t ? t->seg : 4;
        // 8-step segments are built for 128-row groups only
        if (pl->kc % seg != 0 || (seg == 8 && (KS % 8 != 0 || group_steps != 4)))
            seg = pl->kc % 4 == 0 ? 4 : pl->kc;
        pl->seg = seg;
    }
}

int64_t prefill_stages_per_split(int64_t stages, int64_t splits) { return 2 * ceil_div(stages, 2 * splits); }

// Split-K for the async tile (measured on MI355X over the prefill shapes, M = 128 .. 2048):
// when its output tiles number at most one per compute unit, about one work-group per
// compute unit (splits = 256 / tiles, rounded), each split at least kMinSplitStages stages
// long; and when every split is then still longer than kLongSplitStages stages, twice as
// many, so that two work-groups share each compute unit. More splits cost more than they
// gain: the last work-group of a tile sums all of the tile's fp32 partials alone.
constexpr int64_t kPrefillSplitTarget = 256;
constexpr int64_t kMinSplitStages = 16;
constexpr int64_t kLongSplitStages = 128;

// Rows of M per work-group of the async tile: the smallest of 32, 64 and 128 that holds M
// (a 128-row tile at M = 64 spends half its MFMAs on padding rows).
int async_rows(int64_t M) { return M <= 32 ? 32 : M <= 64 ? 64 : 128; }

// The 32- and 64-row work-groups (M <= 64) are lighter: they aim at 512 work-groups, each
// split at least kMinSplitStagesSmall stages long, rounded down to a power of two (a sweep
// of 1..32 splits on the six prefill shapes at M = 24..64 picked these counts or came within
// 3 % of them; uneven splits measured worse than their power-of-two neighbours).
constexpr int64_t kMinSplitStagesSmall = 12;

int64_t auto_prefill_splits(int64_t M, int64_t N, int64_t K) {
    const int bm = async_rows(M);
    const bool small = bm < 128;
    const int64_t target = small ? 2 * kPrefillSplitTarget : kPrefillSplitTarget;
    const int64_t tiles = ceil_div(M, bm) * ceil_div(N, 256);
    const int64_t stages = K / 64;
    if (tiles > target) return 1;
    int64_t s = std::max<int64_t>(1, (target + tiles / 2) / tiles);
    s = std::min(s, std::max<int64_t>(1, stages / (small ? kMinSplitStagesSmall : kMinSplitStages)));
    if (small)
        while (s & (s - 1)) s &= s - 1;                      // largest power of two <= s
    if (tiles * s <= target && stages / s > kLongSplitStages) s *= 2;
    return s;
}

// Split-K of the W4A8 product (stages of 128 K rows). With the 128-row work-group tile: the
// same rule as the async W4A16 tile in K rows (about 256 work-groups, at least 1024 rows per
// split, doubled while the splits stay longer than 8192). The 32- and 64-row tiles hold
// fewer registers (three work-groups per compute unit) and a stage costs them less, so they
// aim at 512 work-groups with at least 768 rows per split, rounded down to a power of two
// (a sweep of 1..32 splits over the six prefill shapes at M = 32 and 64: 1.7 % above the
// best count on average, against 5.6 % with the 128-row rule; counts that split the stages
// unevenly, such as 5 or 10, measured well above their power-of-two neighbours).
int64_t auto_w4a8_splits(int64_t M, int64_t N, int64_t K, int bm) {
    const bool small = bm < 128;
    const int64_t target = small ? 2 * kPrefillSplitTarget : kPrefillSplitTarget;
    const int64_t min_stages = small ? 6 : 8;
    const int64_t tiles = ceil_div(M, bm) * ceil_div(N, 256);
    const int64_t stages = K / 128;
    if (tiles > target) return 1;
    int64_t s = std::max<int64_t>(1, (target + tiles / 2) / tiles);
    s = std::min(s, std::max<int64_t>(1, stages / min_stages));
    if (small)
        while (s & (s - 1)) s &= s - 1;                      // largest power of two <= s
    if (tiles * s <= target && stages / s > 64) s *= 2;
    return s;
}

// Prefill tile choice (measured on MI355X): the async tile (direct-to-LDS loads, split-K
// when its tiles underfill the chip) whenever N % 8 == 0; otherwise the register tile once
// it has kRegisterTileMinGroups 128 x 256 work-groups, the 128 x 128 tile below that.
constexpr int64_t kRegisterTileMinGroups = 384;

int32_t auto_prefill_tile(int64_t M, int64_t N) {
    if (N % 8 == 0) return W4A16_TILE_ASYNC;
    return ceil_div(M, 128) * ceil_div(N, 256) >= kRegisterTileMinGroups ? W4A16_TILE_REGISTER_B : W4A16_TILE_LDS;
}

// Kernel choice (measured crossover on MI355X): with N % 8 == 0 (the async split-K prefill
// tile, whose 32- and 64-row work-groups serve small M): prefill from M = 24 for the largest
// matrices (>= kPrefillHugeKN elements: 8192x28672 at M = 24..32 41-44 us against 43-50 us
// streaming), from M = 64 for matrices of >= kPrefillLargeKN elements that are at least as
// wide as deep (8192^2 and 4096x14336 at M = 64: 25.3 / 22.3 us against 27.7 / 23.9), from
// M = 65 for the deeper ones (14336x4096 streams faster at M = 64: 26.2 against 29.5 us),
// from M = 129 otherwise (for small matrices the streaming kernel still wins at M = 128).
// Without it: prefill once its 128 x 128 output tiles number at least kPrefillMinTiles (half
// a tile per compute unit; with fewer it leaves the chip idle and streaming the weights once
// per 64 rows is faster), and always beyond M = 1024.
constexpr int64_t kPrefillMinM = 65;
constexpr int64_t kPrefillMinMWide = 64;
constexpr int64_t kPrefillMinMHuge = 24;
constexpr int64_t kPrefillLargeKN = int64_t(1) << 25;
constexpr int64_t kPrefillHugeKN = int64_t(1) << 27;
constexpr int64_t kPrefillMinTiles = 128;
constexpr int64_t kSkinnyMaxM = 1024;

int64_t auto_kernel(int64_t M, int64_t N, int64_t K) {
    if (N % 8 == 0) {
        if (M >= kPrefillMinMHuge && K * N >= kPrefillHugeKN) return W4A16_KERNEL_PREFILL;
        if (M >= kPrefillMinMWide && K * N >= kPrefillLargeKN && K <= N) return W4A16_KERNEL_PREFILL;
        if (M < kPrefillMinM) return W4A16_KERNEL_SKINNY;
        return (M > 128 || K * N >= kPrefillLargeKN) ? W4A16_KERNEL_PREFILL : W4A16_KERNEL_SKINNY;
    }
    if (M < kPrefillMinM) return W4A16_KERNEL_SKINNY;
    const int64_t tiles = ceil_div(M, w4a16::kPrefillBM) * ceil_div(N, w4a16::kPrefillBN);
    return (tiles >= kPrefillMinTiles || M > kSkinnyMaxM) ? W4A16_KERNEL_PREFILL : W4A16_KERNEL_SKINNY;
}

// Plans measured on the device at run time (w4a16_autotune) or installed by the caller
// (w4a16_set_plan), per (M, N, K, group size): they take precedence over kTuned and the rule
// for calls that leave the plan to the dispatcher.
struct ShapeKey {
    int64_t M, N, K, g;
    bool operator<(const ShapeKey& o) const {
        return M != o.M ? M < o.M : N != o.N ? N < o.N : K != o.K ? K < o.K : g < o.g;
    }
};
std::mutex g_tuned_mu;
std::map<ShapeKey, w4a16_plan_t> g_tuned;

bool plan_is_auto(const w4a16_plan_t& p) {
    return !p.kernel && !p.kc && !p.splits && !p.row_tiles && !p.tile && !p.waves && !p.cols && !p.seg;
}

bool plan_equal(const w4a16_plan_t& a, const w4a16_plan_t& b) {
    return a.kernel == b.kernel && a.kc == b.kc && a.splits == b.splits && a.row_tiles == b.row_tiles &&
           a.tile == b.tile && a.waves == b.waves && a.cols == b.cols && a.seg == b.seg;
}

bool lookup_tuned(int64_t M, int64_t N, int64_t K, int64_t g, w4a16_plan_t* out) {
    std::lock_guard<std::mutex> lock(g_tuned_mu);
    auto it = g_tuned.find(ShapeKey{M, N, K, g});
    if (it == g_tuned.end()) return false;
    *out = it->second;
    return true;
}

int complete_plan(int64_t M, int64_t N, int64_t K, int64_t group_size, w4a16_plan_t* pl, bool use_tuned = true) {
    // a plan measured or installed for this shape (stored complete and validated)
    if (use_tuned && plan_is_auto(*pl) && lookup_tuned(M, N, K, group_size, pl)) return W4A16_OK;
    const int64_t group_steps = group_size / w4a16::kKStep;
    if (pl->kernel == W4A16_KERNEL_AUTO) pl->kernel = (int32_t)auto_kernel(M, N, K);
    if (pl->kernel == W4A16_KERNEL_PREFILL) {
        if (pl->tile == 0) pl->tile = auto_prefill_tile(M, N);
        if (pl->tile != W4A16_TILE_LDS && pl->tile != W4A16_TILE_REGISTER_B && pl->tile != W4A16_TILE_ASYNC)
            return fail(W4A16_ERR_INVALID_ARG, "prefill tile %d is not built", pl->tile);
        if (pl->tile == W4A16_TILE_ASYNC && N % 8 != 0)
            return fail(W4A16_ERR_UNSUPPORTED, "the async prefill tile needs N %% 8 == 0 (N=%lld)", (long long)N);
        if (pl->kc || pl->row_tiles || pl->waves || pl->cols || pl->seg)
            return fail(W4A16_ERR_INVALID_ARG, "kc/row_tiles/waves/cols/seg apply to the skinny kernel only");
        if (pl->splits && pl->tile != W4A16_TILE_ASYNC)
            return fail(W4A16_ERR_INVALID_ARG, "prefill splits apply to the async tile only");
        if (pl->splits < 0) return fail(W4A16_ERR_INVALID_ARG, "splits must be >= 0");
        const int64_t stages = K / 64;
        if (pl->splits > stages / 2)
            return fail(W4A16_ERR_INVALID_ARG, "splits=%d leaves fewer than 2 stages of 64 K rows per split",
                        pl->splits);
        if (pl->tile == W4A16_TILE_ASYNC) {
            // its loads address a stage with 32-bit byte offsets: up to 32 N (weights) and
            // 128 K 2 (activations)
            if ((int64_t)32 * N > INT32_MAX || (int64_t)128 * K * 2 > INT32_MAX)
                return fail(W4A16_ERR_UNSUPPORTED, "N=%lld or K=%lld exceeds the async tile's 32-bit load offsets",
                            (long long)N, (long long)K);
            if (pl->splits == 0) pl->splits = (int32_t)auto_prefill_splits(M, N, K);
            // the kernel addresses a tile's split partials (128 KiB each) with 32-bit offsets
            if ((int64_t)pl->splits * w4a16::kPrefillTileFloats * 4 > INT32_MAX)
                return fail(W4A16_ERR_UNSUPPORTED, "splits=%d exceeds the async tile's 32-bit workspace offsets",
                            pl->splits);
            // settle on a split count whose stages per split (prefill_stages_per_split, even,
            // which keeps the last split at >= 2 stages) cover K with exactly that many splits
            for (;;) {
                const int64_t s2 = ceil_div(stages, prefill_stages_per_split(stages, pl->splits));
                if (s2 == pl->splits) break;
                pl->splits = (int32_t)s2;
            }
        } else {
            pl->splits = 1;
        }
        if (ceil_div(M, w4a16::kPrefillBM) > 65535) return fail(W4A16_ERR_UNSUPPORTED, "grid too large");
        return W4A16_OK;
    }
    if (pl->kernel != W4A16_KERNEL_SKINNY)
        return fail(W4A16_ERR_INVALID_ARG, "unknown kernel id %d", pl->kernel);
    default_skinny_plan(M, N, K, group_steps, pl);
    if (pl->cols != 16 && pl->cols != 32 && pl->cols != 64)
        return fail(W4A16_ERR_INVALID_ARG, "cols must be 16, 32 or 64 (got %d)", pl->cols);
    const int lw = pl->cols / 16;
    if (pl->row_tiles == 0) pl->row_tiles = (int32_t)std::min<int64_t>(lw == 4 ? 4 : 2, ceil_div(M, 16));
    if (pl->row_tiles < 1 || pl->row_tiles > 4)
        return fail(W4A16_ERR_INVALID_ARG, "row_tiles must be 1..4 (got %d)", pl->row_tiles);
    const int64_t KS = K / w4a16::kKStep;
    const int64_t n_strips = ceil_div(N, pl->cols);
    const int64_t row_blocks = ceil_div(M, 16 * (int64_t)pl->row_tiles);
    if (pl->kc < 1 || pl->kc == 3 || (pl->kc > 4 && pl->kc % 4 != 0))
        return fail(W4A16_ERR_INVALID_ARG, "kc must be 1, 2 or a multiple of 4 (got %d)", pl->kc);
    if (pl->seg == 8 && KS % 8 != 0)
        return fail(W4A16_ERR_INVALID_ARG, "seg=8 needs K %% 256 == 0 (K=%lld)", (long long)K);
    if (pl->kc % pl->seg != 0)
        return fail(W4A16_ERR_INVALID_ARG, "kc=%d is not a multiple of seg=%d", pl->kc, pl->seg);
    if (!w4a16::skinny_config_supported(pl->row_tiles, pl->waves, lw, pl->seg,
                                        (int)std::min<int64_t>(pl->seg, group_steps)))
        return fail(W4A16_ERR_INVALID_ARG, "waves=%d, row_tiles=%d, cols=%d, seg=%d with %lld-row groups is not built",
                    pl->waves, pl->row_tiles, pl->cols, pl->seg, (long long)group_size);
    const int64_t chunks = ceil_div(KS, pl->kc);
    const int64_t splits = ceil_div(chunks, pl->waves);
    if (pl->splits != 0 && pl->splits != splits)
        return fail(W4A16_ERR_INVALID_ARG, "splits=%d does not match kc=%d, waves=%d (needs %lld)",
                    pl->splits, pl->kc, pl->waves, (long long)splits);
    pl->splits = (int32_t)splits;
    if (n_strips * splits > INT32_MAX || row_blocks > 65535)
        return fail(W4A16_ERR_UNSUPPORTED, "grid too large");
    // The kernel addresses a wavefront's weights (kc K-steps of 16 N bytes), a row block's
    // activations (16 row_tiles rows of 2 K bytes) and the scales/zeros with 32-bit byte
    // offsets into buffer resources.
    if (16 * N * (pl->kc + 1) > INT32_MAX || 32 * (int64_t)pl->row_tiles * K > INT32_MAX ||
        (K / group_size) * N * 2 > INT32_MAX)
        return fail(W4A16_ERR_UNSUPPORTED, "shape too large for the skinny kernel's 32-bit offsets (kc=%d)", pl->kc);
    return W4A16_OK;
}

// ---- workspace ---------------------------------------------------------------------------

struct Workspace {
    float* partials = nullptr;
    uint64_t partial_bytes = 0;
    uint32_t* counters = nullptr;
    uint64_t n_counters = 0;
};

std::mutex g_ws_mu;
std::map<std::pair<int, void*>, Workspace> g_ws;
// Buffers of workspaces that have grown. A graph captured on the stream before the growth
// holds their addresses and may be replayed later, so they are never freed (they stay
// allocated until the process ends); growth at least doubles, which bounds what is kept
// to the size of the current workspace.
std::vector<void*> g_retired;

int get_workspace(void* stream, uint64_t bytes, uint64_t n_counters, Workspace* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(W4A16_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_ws_mu);
    Workspace& w = g_ws[{dev, stream}];
    if (w.partial_bytes < bytes || w.n_counters < n_counters) {
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
            return fail(W4A16_ERR_HIP, "split-K workspace of %llu bytes is not allocated for this stream and "
                        "cannot be allocated during graph capture: make one call of this shape on the "
                        "stream before capturing", (unsigned long long)bytes);
        const uint64_t nb = std::max<uint64_t>({bytes, 2 * w.partial_bytes, 1u << 20});
        const uint64_t nc = std::max<uint64_t>({n_counters, 2 * w.n_counters, 4096});
        Workspace g;
        e = hipMalloc(reinterpret_cast<void**>(&g.partials), nb);
        if (e != hipSuccess) return fail(W4A16_ERR_HIP, "hipMalloc workspace: %s", hipGetErrorString(e));
        e = hipMalloc(reinterpret_cast<void**>(&g.counters), nc * sizeof(uint32_t));
        if (e != hipSuccess) {
            (void)hipFree(g.partials);
            return fail(W4A16_ERR_HIP, "hipMalloc counters: %s", hipGetErrorString(e));
        }
        // zero once; every kernel that takes a counter returns it to zero
        e = hipMemsetAsync(g.counters, 0, nc * sizeof(uint32_t), s);
        if (e != hipSuccess) {
            (void)hipFree(g.partials);
            (void)hipFree(g.counters);
            return fail(W4A16_ERR_HIP, "hipMemsetAsync: %s", hipGetErrorString(e));
        }
        g.partial_bytes = nb;
        g.n_counters = nc;
        // launches already enqueued on the stream, and graphs captured on it, keep using
        // the old buffers: retire them instead of freeing them
        if (w.partials) g_retired.push_back(w.partials);
        if (w.counters) g_retired.push_back(w.counters);
        w = g;
    }
    *out = w;
    return W4A16_OK;
}

// Split-K buffers of one call: the library's per-(device, stream) workspace, or for
// w4a16_matmul_noalloc the static per-device scratch, whose size bounds the plans it takes
// (checked before any HIP call).
int call_workspace(bool noalloc, void* stream, uint64_t bytes, uint64_t n_counters, float** ws,
                   uint32_t** counters) {
    if (noalloc) {
        if (bytes > w4a16::kScratchPartialBytes || n_counters * 4 > w4a16::kScratchCounterBytes)
            return fail(W4A16_ERR_UNSUPPORTED,
                        "the plan needs %llu bytes of split-K partials and %llu counters; the static scratch "
                        "holds %llu bytes and %llu counters (force fewer splits)",
                        (unsigned long long)bytes, (unsigned long long)n_counters,
                        (unsigned long long)w4a16::kScratchPartialBytes,
                        (unsigned long long)(w4a16::kScratchCounterBytes / 4));
        const int e = w4a16::scratch_workspace(stream, ws, counters);
        if (e != (int)hipSuccess)
            return fail(W4A16_ERR_HIP, "static scratch: %s", hipGetErrorString((hipError_t)e));
        return W4A16_OK;
    }
    Workspace w;
    const int rc = get_workspace(stream, bytes, n_counters, &w);
    if (rc) return rc;
    *ws = w.partials;
    *counters = w.counters;
    return W4A16_OK;
}

// One launch of the decode kernel over 1..kMaxGroupMats matrices (validated, plan completed
// for M, the summed N and K): their column strips are numbered one after the other, so each
// work-group finds its matrix from its strip. A matrix whose x is null reads the call's x.
int launch_skinny_mats(const void* x, const w4a16_matrix_t* mats, int n_mats, int64_t M, int64_t K,
                       int64_t group_size, int layout, void* stream, const w4a16_plan_t& pl, bool noalloc) {
    w4a16::SkinnyParams p{};
    p.x = static_cast<const uint16_t*>(x);
    p.n_mats = n_mats;
    int64_t strips = 0;
    for (int i = 0; i < w4a16::kMaxGroupMats; ++i) {
        const w4a16_matrix_t& m = mats[std::min(i, n_mats - 1)];       // unused entries repeat the last
        p.mat[i].x = static_cast<const uint16_t*>(m.x ? m.x : x);
        p.rows[i] = (int)(m.M ? m.M : M);
        p.mat[i].qweight = reinterpret_cast<const uint32_t*>(m.qweight);
        p.mat[i].scales = static_cast<const uint16_t*>(m.scales);
        p.mat[i].zeros = static_cast<const uint16_t*>(m.zeros);
        p.mat[i].y = static_cast<uint16_t*>(m.y);
        p.mat[i].N = (int)m.N;
        p.mat[i].strip0 = p.strip0[i] = (int)strips;
        if (i < n_mats) strips += ceil_div(m.N, pl.cols);
    }
    p.M = (int)M;
    p.K = (int)K;
    p.kc = pl.kc;
    p.splits = pl.splits;
    p.n_strips = (int)strips;
    p.row_tiles = pl.row_tiles;
    p.row_blocks = (int)ceil_div(M, 16 * (int64_t)pl.row_tiles);
    p.waves = pl.waves;
    p.lw = pl.cols / 16;
    p.seg = pl.seg;
    p.gshift = w4a16::log2_exact(group_size / w4a16::kKStep);
    p.layout = layout;
    uint64_t ws_bytes = 0, n_counters = 0;
    w4a16::skinny_workspace(p, &ws_bytes, &n_counters);
    if (ws_bytes) {
        const int rc = call_workspace(noalloc, stream, ws_bytes, n_counters, &p.ws, &p.counters);
        if (rc) return rc;
    }
    const int e = w4a16::launch_skinny(p, stream);
    if (e != (int)hipSuccess)
        return fail(W4A16_ERR_HIP, "skinny kernel launch: %s", hipGetErrorString((hipError_t)e));
    return ok();
}

int matmul_impl(const void* x, const int32_t* qweight, const void* scales, const void* zeros,
                void* y, int64_t M, int64_t N, int64_t K, int64_t group_size, int layout, void* stream,
                const w4a16_plan_t* forced, bool noalloc = false) {
    if (!x || !qweight || !scales || !zeros || !y)
        return fail(W4A16_ERR_INVALID_ARG, "null pointer argument");
    if (!w4a16::layout_supported(layout)) return fail(W4A16_ERR_INVALID_ARG, "unknown layout %d", layout);
    int rc = check_gpu_shape(M, N, K, group_size);
    if (rc) return rc;
    if (!aligned16(x) || !aligned16(qweight) || !aligned16(scales) || !aligned16(zeros) || !aligned16(y))
        return fail(W4A16_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    w4a16_plan_t pl = forced ? *forced : w4a16_plan_t{};
    rc = complete_plan(M, N, K, group_size, &pl);
    if (rc) return rc;

    if (pl.kernel == W4A16_KERNEL_PREFILL) {
        w4a16::PrefillParams q{};
        q.x = static_cast<const uint16_t*>(x);
        q.qweight = reinterpret_cast<const uint32_t*>(qweight);
        q.scales = static_cast<const uint16_t*>(scales);
        q.zeros = static_cast<const uint16_t*>(zeros);
        q.y = static_cast<uint16_t*>(y);
        q.M = (int)M;
        q.N = (int)N;
        q.K = (int)K;
        q.tile = pl.tile;
        q.group_shift = w4a16::log2_exact(group_size);
        q.layout = layout;
        q.bm = pl.tile == W4A16_TILE_ASYNC ? async_rows(M) : 128;
        q.splits = std::max(1, pl.splits);
        q.stages_per_split = (int)prefill_stages_per_split(K / 64, q.splits);
        if (q.splits > 1) {
            const int64_t tiles = ceil_div(M, q.bm) * ceil_div(N, 256);
            rc = call_workspace(noalloc, stream, (uint64_t)tiles * q.splits * w4a16::kPrefillTileFloats * 4,
                                (uint64_t)tiles, &q.ws, &q.counters);
            if (rc) return rc;
        }
        const int e = w4a16::launch_prefill(q, stream);
        if (e != (int)hipSuccess)
            return fail(W4A16_ERR_HIP, "prefill kernel launch: %s", hipGetErrorString((hipError_t)e));
        return ok();
    }

    const w4a16_matrix_t one{qweight, scales, zeros, y, N, nullptr, 0};
    return launch_skinny_mats(x, &one, 1, M, K, group_size, layout, stream, pl, noalloc);
}

// ---- autotuning (w4a16_autotune) ------------------------------------------------------

// Weights are rotated over copies totalling this much memory (at least two, at most
// kTuneMaxCopies), so that each timed call reads its weights from HBM as in a model, where
// the layers' weights far exceed the 256 MB Infinity Cache.
constexpr uint64_t kTuneRotateBytes = 512ull << 20;
constexpr int kTuneMaxCopies = 512;
constexpr int kTuneFinalists = 5;

// Frees the workspace of a stream the library created and has synchronised (no enqueued
// launch or captured graph refers to it any more).
void release_workspace(void* stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return;
    std::lock_guard<std::mutex> lock(g_ws_mu);
    auto it = g_ws.find({dev, stream});
    if (it == g_ws.end()) return;
    (void)hipFree(it->second.partials);
    (void)hipFree(it->second.counters);
    g_ws.erase(it);
}

// Split-K workspace of one call under a completed plan (what matmul_impl requests).
void plan_workspace(int64_t M, int64_t N, const w4a16_plan_t& pl, uint64_t* bytes, uint64_t* counters) {
    *bytes = 0;
    *counters = 0;
    if (pl.kernel == W4A16_KERNEL_PREFILL) {
        if (pl.tile == W4A16_TILE_ASYNC && pl.splits > 1) {
            const int64_t tiles = ceil_div(M, async_rows(M)) * ceil_div(N, 256);
            *bytes = (uint64_t)tiles * pl.splits * w4a16::kPrefillTileFloats * 4;
            *counters = (uint64_t)tiles;
        }
        return;
    }
    w4a16::SkinnyParams p{};
    p.splits = pl.splits;
    p.row_tiles = pl.row_tiles;
    p.row_blocks = (int)ceil_div(M, 16 * (int64_t)pl.row_tiles);
    p.n_strips = (int)ceil_div(N, pl.cols);
    p.lw = pl.cols / 16;
    w4a16::skinny_workspace(p, bytes, counters);
}

// The plans w4a16_autotune times: the dispatcher's own (tuned or not), every built decode-kernel
// plan when M <= 128, and the prefill tiles (each split count the async tile settles on) when
// M >= 17.
std::vector<w4a16_plan_t> tune_candidates(int64_t M, int64_t N, int64_t K, int64_t g) {
    std::vector<w4a16_plan_t> out;
    auto add = [&](w4a16_plan_t p, bool use_tuned) {
        if (complete_plan(M, N, K, g, &p, use_tuned) != W4A16_OK) return;
        for (const w4a16_plan_t& q : out)
            if (plan_equal(q, p)) return;
        out.push_back(p);
    };
    add(w4a16_plan_t{}, false);
    add(w4a16_plan_t{}, true);
    if (M <= 128)
        for (int cols : {16, 32, 64})
            for (int waves : {4, 8, 16})
                for (int kc : {4, 8, 12, 16, 20, 24, 28, 32, 40, 48, 56, 64})
                    for (int seg : {2, 4, 8}) {
                        w4a16_plan_t p{};
                        p.kernel = W4A16_KERNEL_SKINNY;
                        p.cols = cols;
                        p.waves = waves;
                        p.kc = kc;
                        p.seg = seg;
                        add(p, false);
                    }
    if (M >= 17) {
        if (N % 8 == 0) {
            for (int splits : {1, 2, 3, 4, 6, 8, 12, 16}) {
                w4a16_plan_t p{};
                p.kernel = W4A16_KERNEL_PREFILL;
                p.tile = W4A16_TILE_ASYNC;
                p.splits = splits;
                add(p, false);
            }
        } else {
            for (int tile : {W4A16_TILE_LDS, W4A16_TILE_REGISTER_B}) {
                w4a16_plan_t p{};
                p.kernel = W4A16_KERNEL_PREFILL;
                p.tile = tile;
                add(p, false);
            }
        }
    }
    return out;
}

struct TuneCtx {
    const void* x;
    void* y;
    int64_t M, N, K, g;
    int layout;
    hipStream_t s;
    std::vector<const int32_t*> qw;   // rotation copies; the first is the caller's
    std::vector<const void*> sc, zr;
};

// Seconds per call of `pl`: a HIP graph of one call per rotation copy, captured on the tuning
// stream, replayed once to warm up and then `reps` times between two events, best of
// `trials`. Negative when the plan cannot be captured or run.
double time_plan(const TuneCtx& c, const w4a16_plan_t& pl, int reps, int trials) {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    if (hipStreamBeginCapture(c.s, hipStreamCaptureModeThreadLocal) != hipSuccess) return -1.0;
    int rc = W4A16_OK;
    for (size_t i = 0; i < c.qw.size() && rc == W4A16_OK; ++i)
        rc = matmul_impl(c.x, c.qw[i], c.sc[i], c.zr[i], c.y, c.M, c.N, c.K, c.g, c.layout, c.s, &pl);
    const hipError_t ec = hipStreamEndCapture(c.s, &graph);
    if (rc != W4A16_OK || ec != hipSuccess || !graph) {
        if (graph) (void)hipGraphDestroy(graph);
        return -1.0;
    }
    if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
        (void)hipGraphDestroy(graph);
        return -1.0;
    }
    hipEvent_t e0 = nullptr, e1 = nullptr;
    double best = -1.0;
    bool good = hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess &&
                hipGraphLaunch(exec, c.s) == hipSuccess;
    for (int t = 0; good && t < trials; ++t) {
        good = hipEventRecord(e0, c.s) == hipSuccess;
        for (int r = 0; good && r < reps; ++r) good = hipGraphLaunch(exec, c.s) == hipSuccess;
        float ms = 0.f;
        good = good && hipEventRecord(e1, c.s) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
               hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
        const double sec = ms * 1e-3 / ((double)reps * (double)c.qw.size());
        if (good && (best < 0.0 || sec < best)) best = sec;
    }
    (void)hipStreamSynchronize(c.s);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return good ? best : -1.0;
}

int autotune_impl(const void* x, const int32_t* qweight, const void* scales, const void* zeros, void* y,
                  int64_t M, int64_t N, int64_t K, int64_t g, int layout, void* stream, w4a16_plan_t* best_out,
                  double* best_sec) {
    if (!x || !qweight || !scales || !zeros || !y) return fail(W4A16_ERR_INVALID_ARG, "null pointer argument");
    if (!w4a16::layout_supported(layout)) return fail(W4A16_ERR_INVALID_ARG, "unknown layout %d", layout);
    int rc = check_gpu_shape(M, N, K, g);
    if (rc) return rc;
    if (!aligned16(x) || !aligned16(qweight) || !aligned16(scales) || !aligned16(zeros) || !aligned16(y))
        return fail(W4A16_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    hipStream_t cs = reinterpret_cast<hipStream_t>(stream);
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(cs, &cap) == hipSuccess && cap != hipStreamCaptureStatusNone)
        return fail(W4A16_ERR_INVALID_ARG, "w4a16_autotune cannot run under stream capture");
    const std::vector<w4a16_plan_t> cands = tune_candidates(M, N, K, g);
    if (cands.empty()) return fail(W4A16_ERR_UNSUPPORTED, "no plan runs this shape");
    uint64_t ws_bytes = 0, ws_counters = 0;
    for (const w4a16_plan_t& p : cands) {
        uint64_t b = 0, c = 0;
        plan_workspace(M, N, p, &b, &c);
        ws_bytes = std::max(ws_bytes, b);
        ws_counters = std::max(ws_counters, c);
    }

    hipError_t e = hipStreamSynchronize(cs);                 // the caller's inputs are ready
    if (e != hipSuccess) return fail(W4A16_ERR_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
    TuneCtx c{x, y, M, N, K, g, layout, nullptr, {}, {}, {}};
    e = hipStreamCreateWithFlags(&c.s, hipStreamNonBlocking);
    if (e != hipSuccess) return fail(W4A16_ERR_HIP, "hipStreamCreate: %s", hipGetErrorString(e));
    const uint64_t qb = (uint64_t)(K / 8) * N * 4, sb = (uint64_t)(K / g) * N * 2;
    const uint64_t qa = (qb + 255) & ~255ull, sa = (sb + 255) & ~255ull, per = qa + 2 * sa;
    const int copies = (int)std::min<uint64_t>(kTuneMaxCopies, std::max<uint64_t>(2, (kTuneRotateBytes + per - 1) / per));
    char* rot = nullptr;
    double t_best = -1.0;
    w4a16_plan_t p_best{};
    rc = W4A16_OK;
    e = hipMalloc(reinterpret_cast<void**>(&rot), per * (copies - 1));
    if (e != hipSuccess) rc = fail(W4A16_ERR_HIP, "hipMalloc of %d weight copies: %s", copies - 1, hipGetErrorString(e));
    c.qw.push_back(qweight);
    c.sc.push_back(scales);
    c.zr.push_back(zeros);
    for (int i = 0; rc == W4A16_OK && i < copies - 1; ++i) {
        char* b = rot + per * i;
        if (hipMemcpyAsync(b, qweight, qb, hipMemcpyDeviceToDevice, c.s) != hipSuccess ||
            hipMemcpyAsync(b + qa, scales, sb, hipMemcpyDeviceToDevice, c.s) != hipSuccess ||
            hipMemcpyAsync(b + qa + sa, zeros, sb, hipMemcpyDeviceToDevice, c.s) != hipSuccess)
            rc = fail(W4A16_ERR_HIP, "copying the weights for rotation failed");
        c.qw.push_back(reinterpret_cast<const int32_t*>(b));
        c.sc.push_back(b + qa);
        c.zr.push_back(b + qa + sa);
    }
    // the largest workspace any candidate needs, allocated once before any capture
    if (rc == W4A16_OK && ws_bytes) {
        Workspace w;
        rc = get_workspace(c.s, ws_bytes, ws_counters, &w);
    }
    if (rc == W4A16_OK && hipStreamSynchronize(c.s) != hipSuccess) rc = fail(W4A16_ERR_HIP, "tuning stream failed");
    if (rc == W4A16_OK) {
        // clock warm-up: about 0.1 s of the dispatcher's plan
        const double t0 = time_plan(c, cands[0], 1, 1);
        if (t0 > 0.0)
            (void)time_plan(c, cands[0], (int)std::min(200.0, std::max(1.0, 0.1 / (t0 * copies))), 1);
        std::vector<std::pair<double, size_t>> screen;
        for (size_t i = 0; i < cands.size(); ++i) {
            const double t = time_plan(c, cands[i], 2, 2);
            if (t > 0.0) screen.emplace_back(t, i);
        }
        std::sort(screen.begin(), screen.end());
        // finalists (and the dispatcher's plan) timed again, interleaved, best of both rounds
        std::vector<size_t> fin;
        for (size_t i = 0; i < screen.size() && (int)fin.size() < kTuneFinalists; ++i) fin.push_back(screen[i].second);
        if (std::find(fin.begin(), fin.end(), (size_t)0) == fin.end() && !screen.empty()) fin.push_back(0);
        std::vector<double> tf(fin.size(), -1.0);
        for (int round = 0; round < 2; ++round)
            for (size_t j = 0; j < fin.size(); ++j) {
                const double t = time_plan(c, cands[fin[j]], 3, 3);
                if (t > 0.0 && (tf[j] < 0.0 || t < tf[j])) tf[j] = t;
            }
        double t_default = -1.0;
        for (size_t j = 0; j < fin.size(); ++j) {
            if (fin[j] == 0) t_default = tf[j];
            if (tf[j] > 0.0 && (t_best < 0.0 || tf[j] < t_best)) {
                t_best = tf[j];
                p_best = cands[fin[j]];
            }
        }
        // the dispatcher's plan unless another is more than 1 % faster (timing noise)
        if (t_default > 0.0 && t_default <= 1.01 * t_best) {
            t_best = t_default;
            p_best = cands[0];
        }
        if (t_best < 0.0) rc = fail(W4A16_ERR_HIP, "no plan could be timed");
    }
    if (rc == W4A16_OK) {                                   // y = the product, with the winner
        rc = matmul_impl(x, qweight, scales, zeros, y, M, N, K, g, layout, c.s, &p_best);
        if (rc == W4A16_OK && hipStreamSynchronize(c.s) != hipSuccess) rc = fail(W4A16_ERR_HIP, "tuning stream failed");
    }
    (void)hipStreamSynchronize(c.s);
    if (rot) (void)hipFree(rot);
    release_workspace(c.s);
    (void)hipStreamDestroy(c.s);
    if (rc) return rc;
    {
        std::lock_guard<std::mutex> lock(g_tuned_mu);
        g_tuned[ShapeKey{M, N, K, g}] = p_best;
    }
    if (best_out) *best_out = p_best;
    if (best_sec) *best_sec = t_best;
    return ok();
}

}  // namespace

extern "C" {

int w4a16_pack_ex(const float* W, int64_t K, int64_t N, int64_t group_size, int symmetric,
                  int layout, int32_t* qweight, uint16_t* scales, uint16_t* zeros) {
    if (!W || !qweight || !scales || !zeros) return fail(W4A16_ERR_INVALID_ARG, "null pointer argument");
    if (K < 1 || N < 1) return fail(W4A16_ERR_INVALID_ARG, "K and N must be >= 1");
    if (symmetric != 0 && symmetric != 1) return fail(W4A16_ERR_INVALID_ARG, "symmetric must be 0 or 1");
    if (!w4a16::layout_supported(layout)) return fail(W4A16_ERR_INVALID_ARG, "unknown layout %d", layout);
    if (!w4a16::group_supported(group_size))
        return fail(W4A16_ERR_UNSUPPORTED, "group_size %lld not supported (32, 64, 128 or 256)",
                    (long long)group_size);
    if (K % group_size != 0)
        return fail(W4A16_ERR_UNSUPPORTED, "K=%lld is not a multiple of group_size", (long long)K);
    const int rc = w4a16::pack_host(W, K, N, group_size, symmetric == 1, layout, qweight, scales, zeros);
    if (rc == W4A16_ERR_NONFINITE) return fail(rc, "non-finite weight or fp16 scale overflow");
    if (rc == W4A16_ERR_UNSUPPORTED) return fail(rc, "zero point outside |zero| <= 1024");
    if (rc) return fail(rc, "pack failed");
    return ok();
}

int w4a16_pack(const float* W, int64_t K, int64_t N, int64_t group_size, int32_t* qweight,
               uint16_t* scales, uint16_t* zeros) {
    return w4a16_pack_ex(W, K, N, group_size, 0, W4A16_LAYOUT_LINEAR, qweight, scales, zeros);
}

int w4a16_unpack_ex(const int32_t* qweight, int64_t K, int64_t N, int layout, uint8_t* codes) {
    if (!qweight || !codes) return fail(W4A16_ERR_INVALID_ARG, "null pointer argument");
    if (K < 8 || N < 1 || K % 8 != 0) return fail(W4A16_ERR_INVALID_ARG, "K must be a positive multiple of 8, N >= 1");
    if (!w4a16::layout_supported(layout)) return fail(W4A16_ERR_INVALID_ARG, "unknown layout %d", layout);
    w4a16::unpack_host(qweight, K, N, layout, codes);
    return ok();
}

int w4a16_unpack(const int32_t* qweight, int64_t K, int64_t N, uint8_t* codes) {
    return w4a16_unpack_ex(qweight, K, N, W4A16_LAYOUT_LINEAR, codes);
}

int w4a16_matmul(const void* x, const int32_t* qweight, const void* scales, const void* zeros,
                 void* y, int64_t M, int64_t N, int64_t K, int64_t group_size, void* stream) {
    return matmul_impl(x, qweight, scales, zeros, y, M, N, K, group_size, W4A16_LAYOUT_LINEAR, stream, nullptr);
}

int w4a16_matmul_ex(const void* x, const int32_t* qweight, const void* scales, const void* zeros,
                    void* y, int64_t M, int64_t N, int64_t K, int64_t group_size, void* stream,
                    const w4a16_plan_t* plan) {
    if (!plan) return fail(W4A16_ERR_INVALID_ARG, "null plan");
    return matmul_impl(x, qweight, scales, zeros, y, M, N, K, group_size, W4A16_LAYOUT_LINEAR, stream, plan);
}

int w4a16_matmul_fmt(const void* x, const int32_t* qweight, const void* scales, const void* zeros,
                     void* y, int64_t M, int64_t N, int64_t K, int64_t group_size, int layout, void* stream,
                     const w4a16_plan_t* plan) {
    return matmul_impl(x, qweight, scales, zeros, y, M, N, K, group_size, layout, stream, plan);
}

int w4a16_matmul_grouped(const void* x, const w4a16_matrix_t* mats, int n_mats, int64_t M, int64_t K,
                         int64_t group_size, int layout, void* stream, const w4a16_plan_t* plan) {
    if (!x || !mats) return fail(W4A16_ERR_INVALID_ARG, "null pointer argument");
    if (n_mats < 1 || n_mats > w4a16::kMaxGroupMats)
        return fail(W4A16_ERR_INVALID_ARG, "n_mats=%d must lie in 1..%d", n_mats, w4a16::kMaxGroupMats);
    if (!w4a16::layout_supported(layout)) return fail(W4A16_ERR_INVALID_ARG, "unknown layout %d", layout);
    int64_t n_total = 0;
    for (int i = 0; i < n_mats; ++i) {
        const w4a16_matrix_t& m = mats[i];
        if (!m.qweight || !m.scales || !m.zeros || !m.y)
            return fail(W4A16_ERR_INVALID_ARG, "null pointer in matrix %d", i);
        int rc = check_gpu_shape(M, m.N, K, group_size);
        if (rc) return rc;
        if (!aligned16(m.qweight) || !aligned16(m.scales) || !aligned16(m.zeros) || !aligned16(m.y) ||
            !aligned16(m.x))
            return fail(W4A16_ERR_ALIGNMENT, "device pointers of matrix %d must be 16-byte aligned", i);
        if (m.M < 0 || m.M > M)
            return fail(W4A16_ERR_INVALID_ARG, "matrix %d: M=%lld must lie in 0..M (%lld; 0: M)", i, (long long)m.M,
                        (long long)M);
        n_total += m.N;
    }
    int rc = check_gpu_shape(M, n_total, K, group_size);
    if (rc) return rc;
    if (!aligned16(x)) return fail(W4A16_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    w4a16_plan_t pl = plan ? *plan : w4a16_plan_t{};
    if (plan_is_auto(pl)) (void)lookup_tuned(M, n_total, K, group_size, &pl);
    if (pl.kernel == W4A16_KERNEL_AUTO) pl.kernel = (int32_t)auto_kernel(M, n_total, K);
    if (pl.kernel == W4A16_KERNEL_PREFILL) {
        // the prefill tiles fill the chip per matrix: one launch each, each with its own plan
        // unless the caller forced one
        const bool forced = plan && plan->kernel == W4A16_KERNEL_PREFILL;
        for (int i = 0; i < n_mats; ++i) {                    // every plan is checked before any launch
            w4a16_plan_t pi = forced ? *plan : w4a16_plan_t{};
            rc = complete_plan(M, mats[i].N, K, group_size, &pi);
            if (rc) return rc;
        }
        for (int i = 0; i < n_mats; ++i) {
            rc = matmul_impl(mats[i].x ? mats[i].x : x, mats[i].qweight, mats[i].scales, mats[i].zeros, mats[i].y,
                             mats[i].M ? mats[i].M : M, mats[i].N, K, group_size, layout, stream,
                             forced ? plan : nullptr);
            if (rc) return rc;
        }
        return ok();
    }
    rc = complete_plan(M, n_total, K, group_size, &pl);
    if (rc) return rc;
    return launch_skinny_mats(x, mats, n_mats, M, K, group_size, layout, stream, pl, false);
}

int w4a16_matmul_noalloc(const void* x, const int32_t* qweight, const void* scales, const void* zeros,
                         void* y, int64_t M, int64_t N, int64_t K, int64_t group_size, int layout, void* stream,
                         const w4a16_plan_t* plan) {
    return matmul_impl(x, qweight, scales, zeros, y, M, N, K, group_size, layout, stream, plan, true);
}

int w4a16_plan(int64_t M, int64_t N, int64_t K, int64_t group_size, w4a16_plan_t* plan) {
    if (!plan) return fail(W4A16_ERR_INVALID_ARG, "null plan");
    int rc = check_gpu_shape(M, N, K, group_size);
    if (rc) return rc;
    w4a16_plan_t pl = *plan;
    rc = complete_plan(M, N, K, group_size, &pl);
    if (rc) return rc;
    *plan = pl;
    return ok();
}

int w4a16_dequant_fmt(const int32_t* qweight, const void* scales, const void* zeros, uint8_t* codes,
                      void* w, int64_t N, int64_t K, int64_t group_size, int layout, void* stream) {
    if (!qweight || !scales || !zeros) return fail(W4A16_ERR_INVALID_ARG, "null pointer argument");
    if (!w4a16::layout_supported(layout)) return fail(W4A16_ERR_INVALID_ARG, "unknown layout %d", layout);
    if (!codes && !w) return fail(W4A16_ERR_INVALID_ARG, "codes and w are both NULL");
    int rc = check_gpu_shape(1, N, K, group_size);
    if (rc) return rc;
    if (!aligned16(qweight) || !aligned16(scales) || !aligned16(zeros) || (w && !aligned16(w)))
        return fail(W4A16_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    if (codes && reinterpret_cast<uintptr_t>(codes) % 4 != 0)
        return fail(W4A16_ERR_ALIGNMENT, "codes must be 4-byte aligned");
    const int e = w4a16::launch_dequant(reinterpret_cast<const uint32_t*>(qweight),
                                        static_cast<const uint16_t*>(scales),
                                        static_cast<const uint16_t*>(zeros), codes,
                                        static_cast<uint16_t*>(w), (int)N, (int)K,
                                        w4a16::log2_exact(group_size), layout, stream);
    if (e != (int)hipSuccess)
        return fail(W4A16_ERR_HIP, "dequant kernel launch: %s", hipGetErrorString((hipError_t)e));
    return ok();
}

int w4a16_dequant(const int32_t* qweight, const void* scales, const void* zeros, uint8_t* codes,
                  void* w, int64_t N, int64_t K, int64_t group_size, void* stream) {
    return w4a16_dequant_fmt(qweight, scales, zeros, codes, w, N, K, group_size, W4A16_LAYOUT_LINEAR, stream);
}

int w4a8_quantize_activations(const void* x, uint8_t* xq, float* sx, float* xsum, int64_t M, int64_t K,
                              void* stream) {
    if (!x || !xq || !sx || !xsum) return fail(W4A16_ERR_INVALID_ARG, "null pointer argument");
    if (M < 1 || K < 1) return fail(W4A16_ERR_INVALID_ARG, "M, K must be >= 1 (got %lld, %lld)", (long long)M,
                                    (long long)K);
    if (K % 128 != 0) return fail(W4A16_ERR_UNSUPPORTED, "K=%lld is not a multiple of 128", (long long)K);
    if (M > 65535 * 1024ll || M * K > INT32_MAX) return fail(W4A16_ERR_UNSUPPORTED, "problem too large");
    if (!aligned16(x) || !aligned16(xq) || !aligned16(xsum) || reinterpret_cast<uintptr_t>(sx) % 4 != 0)
        return fail(W4A16_ERR_ALIGNMENT, "x, xq and xsum must be 16-byte aligned, sx 4-byte aligned");
    const int e = w4a16::launch_w4a8_quantize(static_cast<const uint16_t*>(x), xq, sx, xsum, (int)M, (int)K, stream);
    if (e != (int)hipSuccess)
        return fail(W4A16_ERR_HIP, "activation quantiser launch: %s", hipGetErrorString((hipError_t)e));
    return ok();
}

int w4a8_matmul_ex(const uint8_t* xq, const float* sx, const float* xsum, const int32_t* qweight, const void* scales,
                   const void* zeros, void* y, int64_t M, int64_t N, int64_t K, int64_t group_size, int layout,
                   int splits, void* stream) {
    if (!xq || !sx || !xsum || !qweight || !scales || !zeros || !y)
        return fail(W4A16_ERR_INVALID_ARG, "null pointer argument");
    if (!w4a16::layout_supported(layout)) return fail(W4A16_ERR_INVALID_ARG, "unknown layout %d", layout);
    int rc = check_gpu_shape(M, N, K, group_size);
    if (rc) return rc;
    if (group_size != 128 && group_size != 256)
        return fail(W4A16_ERR_UNSUPPORTED, "W4A8 takes groups of 128 or 256 rows (got %lld)", (long long)group_size);
    if (N % 8 != 0) return fail(W4A16_ERR_UNSUPPORTED, "W4A8 needs N %% 8 == 0 (N=%lld)", (long long)N);
    // a wavefront addresses 16 packed rows of the weights (64 N bytes) with 32-bit offsets
    if (64 * N > INT32_MAX)
        return fail(W4A16_ERR_UNSUPPORTED, "N=%lld exceeds the W4A8 kernel's 32-bit weight offsets", (long long)N);
    if (ceil_div(M, 128) > 65535) return fail(W4A16_ERR_UNSUPPORTED, "grid too large");
    if (!aligned16(xq) || !aligned16(xsum) || !aligned16(qweight) || !aligned16(scales) || !aligned16(zeros) ||
        !aligned16(y) || reinterpret_cast<uintptr_t>(sx) % 4 != 0)
        return fail(W4A16_ERR_ALIGNMENT, "device pointers must be 16-byte aligned (sx 4-byte)");
    w4a16::W4A8Params p{};
    p.xq = xq;
    p.sx = sx;
    p.xsum = xsum;
    p.Ms = (int)(ceil_div(M, 4) * 4);
    p.qweight = reinterpret_cast<const uint32_t*>(qweight);
    p.scales = static_cast<const uint16_t*>(scales);
    p.zeros = static_cast<const uint16_t*>(zeros);
    p.y = static_cast<uint16_t*>(y);
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.group_shift = w4a16::log2_exact(group_size);
    p.layout = layout;
    p.bm = M <= 32 ? 32 : M <= 64 ? 64 : 128;                  // the smallest row tile that holds M
    const int64_t stages = K / 128;
    if (splits < 0 || splits > stages)
        return fail(W4A16_ERR_INVALID_ARG, "splits=%d must lie in 0..K/128 (%lld)", splits, (long long)stages);
    int64_t S = splits ? splits : auto_w4a8_splits(M, N, K, p.bm);
    const int64_t per = ceil_div(stages, S);
    S = ceil_div(stages, per);                                 // every split non-empty
    if (S * w4a16::kPrefillTileFloats * 4 > INT32_MAX)         // partials addressed with 32-bit offsets
        return fail(W4A16_ERR_UNSUPPORTED, "%lld splits exceed the W4A8 kernel's 32-bit workspace offsets",
                    (long long)S);
    p.splits = (int)S;
    p.stages_per_split = (int)per;
    if (S > 1) {
        const int64_t tiles = ceil_div(M, p.bm) * ceil_div(N, 256);
        Workspace w;
        rc = get_workspace(stream, (uint64_t)tiles * S * w4a16::kPrefillTileFloats * 4, (uint64_t)tiles, &w);
        if (rc) return rc;
        p.ws = w.partials;
        p.counters = w.counters;
    }
    const int e = w4a16::launch_w4a8(p, stream);
    if (e != (int)hipSuccess) return fail(W4A16_ERR_HIP, "W4A8 kernel launch: %s", hipGetErrorString((hipError_t)e));
    return ok();
}

int w4a8_matmul(const uint8_t* xq, const float* sx, const float* xsum, const int32_t* qweight, const void* scales,
                const void* zeros, void* y, int64_t M, int64_t N, int64_t K, int64_t group_size, int layout,
                void* stream) {
    return w4a8_matmul_ex(xq, sx, xsum, qweight, scales, zeros, y, M, N, K, group_size, layout, 0, stream);
}

int w4a16_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink) return fail(W4A16_ERR_INVALID_ARG, "null pointer argument");
    if (bytes < 16 || bytes % 16 != 0)
        return fail(W4A16_ERR_INVALID_ARG, "bytes=%lld must be a positive multiple of 16", (long long)bytes);
    if (bytes / (16 * 1024) >= INT32_MAX) return fail(W4A16_ERR_UNSUPPORTED, "buffer too large");
    if (!aligned16(buf) || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
        return fail(W4A16_ERR_ALIGNMENT, "buf must be 16-byte aligned, sink 4-byte aligned");
    const int e = w4a16::launch_read_probe(buf, bytes, sink, stream);
    if (e != (int)hipSuccess) return fail(W4A16_ERR_HIP, "read probe launch: %s", hipGetErrorString((hipError_t)e));
    return ok();
}

int w4a16_autotune(const void* x, const int32_t* qweight, const void* scales, const void* zeros, void* y,
                   int64_t M, int64_t N, int64_t K, int64_t group_size, int layout, void* stream,
                   w4a16_plan_t* best, double* seconds) {
    return autotune_impl(x, qweight, scales, zeros, y, M, N, K, group_size, layout, stream, best, seconds);
}

int w4a16_set_plan(int64_t M, int64_t N, int64_t K, int64_t group_size, const w4a16_plan_t* plan) {
    int rc = check_gpu_shape(M, N, K, group_size);
    if (rc) return rc;
    if (!plan) {
        std::lock_guard<std::mutex> lock(g_tuned_mu);
        g_tuned.erase(ShapeKey{M, N, K, group_size});
        return ok();
    }
    w4a16_plan_t pl = *plan;
    if (plan_is_auto(pl)) return fail(W4A16_ERR_INVALID_ARG, "the plan names no kernel");
    rc = complete_plan(M, N, K, group_size, &pl, false);
    if (rc) return rc;
    std::lock_guard<std::mutex> lock(g_tuned_mu);
    g_tuned[ShapeKey{M, N, K, group_size}] = pl;
    return ok();
}

int w4a16_clear_plans(void) {
    std::lock_guard<std::mutex> lock(g_tuned_mu);
    g_tuned.clear();
    return ok();
}

const char* w4a16_strerror(int code) {
    switch (code) {
        case W4A16_OK: return "success";
        case W4A16_ERR_INVALID_ARG: return "invalid argument";
        case W4A16_ERR_UNSUPPORTED: return "unsupported shape or parameter";
        case W4A16_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
        case W4A16_ERR_NONFINITE: return "non-finite value";
        case W4A16_ERR_HIP: return "HIP runtime error";
        default: return "unknown error code";
    }
}

const char* w4a16_last_error_detail(void) { return g_detail.c_str(); }

int w4a16_version(void) { return 100; }

}  // extern "C"
