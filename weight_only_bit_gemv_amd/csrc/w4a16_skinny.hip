// Decode / skinny-M W4A16 kernel for gfx950: a single pass over the packed weight stream.
//
// What it computes: y = x . dequant(Wq) ("Beating FP16 with 4-bit Weights: A Portable W4A16
// GEMM in Triton", section "The design"), with the split-K decode strategy of the same page
// (extra parallelism along K when M is small: sections "The design" and "Things I got
// wrong along the way") but with a deterministic fixed-order reduction instead of fp32
// atomics.
//
// Mapping (one work-group = W wavefronts = one 64-column strip x one K range):
//  * lane l reads one 16-byte word quad per K-step: packed row 4*ks + l/16, columns
//    strip*64 + 4*(l%16) .. +3. A wavefront's load is 4 rows x 256 contiguous bytes; every
//    packed int32 of qweight is read exactly once per 16-row block of M.
//  * each of the lane's 4 words is the B operand of one v_mfma_f32_16x16x32_f16: a lane of
//    that MFMA holds 8 K values of one column, which is exactly one packed word. Four MFMA
//    tiles cover columns {4j + t}; their outputs land back on the lane that owns the column.
//  * the words are unpacked to exact fp16 (q - zero) values; x (rows padded to 16) is the A
//    operand in the same K order; products accumulate in fp32 per 128-row group and the
//    group's fp32 partial is multiplied by the column's scale once:
//    sum_k x_k (q_k - z) s = s * sum_k x_k (q_k - z) over a group, which keeps every
//    product exact.
//  * the W wavefronts of a work-group stream consecutive K ranges and are summed in LDS in
//    wave order; with more than one work-group along K (splits > 1) each writes its fp32
//    partial to the workspace, and the last to arrive (arrival counter) sums the splits in
//    index order 0..splits-1 and writes y. Results are bitwise reproducible.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "w4a16_device.hpp"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {

constexpr int kGS = kGroup / kKStep;    // K-steps per scale/zero group (4)
// s_waitcnt immediate for vmcnt(0) with expcnt/lgkmcnt left at their maxima (gfx9 encoding).
constexpr int kWaitVmcnt0 = 0 | (0x7 << 4) | (0xf << 8);

// One segment: U consecutive K-steps (U * 32 rows) of one wavefront, all inside one
// 128-row group: U word quads per lane, the matching activations, one scale/zero quad.
// The loads only issue memory requests: nothing in load() reads the returned registers,
// so a wavefront can keep a prefetched segment in flight while it works on the current one
// (the activation permutation happens in accumulate(), at first use).
template <int MT, int U>
struct Segment {
    uint4 wv[U];
    uint4 xv[U][MT];
    uint2 sv, zv;

    __device__ __forceinline__ void load(const uint4* __restrict__ wbase, const uint16_t* const* xrow,
                                         const SkinnyParams& p, int ks, size_t nq, int nl) {
        const int grp = ks / kGS;
#pragma unroll
        for (int u = 0; u < U; ++u) wv[u] = wbase[(size_t)(ks + u) * 4 * nq];
        sv = *reinterpret_cast<const uint2*>(p.scales + (size_t)grp * p.N + nl);
        zv = *reinterpret_cast<const uint2*>(p.zeros + (size_t)grp * p.N + nl);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                xv[u][mt] = *reinterpret_cast<const uint4*>(xrow[mt] + (size_t)(ks + u) * kKStep);
    }

    // acc += scale * sum over the segment of x * (q - zero), per column, in fp32.
    __device__ __forceinline__ void accumulate(floatx4 (&acc)[MT][4], const UnpackConsts& uc) const {
        const half2_t z01 = as_h2(zv.x), z23 = as_h2(zv.y);
        const ZeroOffsets zo[4] = {zero_offsets(z01[0]), zero_offsets(z01[1]),
                                   zero_offsets(z23[0]), zero_offsets(z23[1])};
        floatx4 part[MT][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t words[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
            half8_t xa[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) xa[mt] = permute_x(xv[u][mt]);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const half8_t b = unpack_sub(words[t], zo[t], uc);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    part[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        xa[mt], b, u == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : part[mt][t], 0, 0, 0);
            }
        }
        const half2_t s01 = as_h2(sv.x), s23 = as_h2(sv.y);
        const float sc[4] = {(float)s01[0], (float)s01[1], (float)s23[0], (float)s23[1]};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[mt][t] += sc[t] * part[mt][t];
    }
};

// MT: 16-row MFMA tiles of M per work-group. U: K-steps per segment, min(kc, 4); the
// dispatcher keeps kc in {1, 2} or a multiple of 4, so every segment is exactly U K-steps
// inside one 128-row group and the loop below needs no predicates. W: wavefronts per
// work-group. Dynamic LDS: (W - 1) * rows * 64 floats, rows = min(16 * MT, M - row0).
template <int MT, int U, int W>
__global__ __launch_bounds__(64 * W) void skinny_kernel(SkinnyParams p) {
    static_assert(U == 1 || U == 2 || U == kGS, "segment must divide a group");
    extern __shared__ float red[];                  // [W - 1][rows][64]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lg = lane >> 4;            // which of the 4 packed rows of a K-step
    const int lc = lane & 15;            // column quad within the strip / A-operand row
    const int strip = blockIdx.x % p.n_strips;
    const int split = blockIdx.x / p.n_strips;
    const int row0 = blockIdx.y * 16 * MT;
    const int rows = min(16 * MT, p.M - row0);          // valid output rows of this work-group
    const int n = strip * kStripN + lc * 4;
    const bool col_ok = n < p.N;
    const int nl = col_ok ? n : 0;       // loads stay in bounds; results of such lanes are dropped
    const int KS = p.K / kKStep;
    const int chunk = split * W + wave;
    const int k0 = min(chunk * p.kc, KS);
    const int k1 = min(k0 + p.kc, KS);
    const size_t nq = (size_t)(p.N >> 2);                 // 16-byte word quads per packed row
    const uint4* __restrict__ wbase = reinterpret_cast<const uint4*>(p.qweight) + lg * nq + (nl >> 2);
    // A-operand rows beyond M only feed output rows beyond M, which are never stored, so
    // their loads are clamped to row M-1 instead of being predicated.
    const uint16_t* xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        xrow[mt] = p.x + (size_t)min(row0 + mt * 16 + lc, p.M - 1) * p.K + lg * 8;
    const UnpackConsts uc = unpack_consts();

    floatx4 acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mt][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Software pipeline over segments, unrolled twice so that the two buffers alternate
    // roles without register copies: the loads of segment i+1 are issued before segment i
    // is unpacked and multiplied, so every wavefront keeps two segments in flight.
    Segment<MT, U> sa, sb;
    if (k0 < k1) sa.load(wbase, xrow, p, k0, nq, nl);
    for (int ks = k0; ks < k1; ks += 2 * U) {
        const bool has_b = ks + U < k1;
        if (has_b) sb.load(wbase, xrow, p, ks + U, nq, nl);
        sa.accumulate(acc, uc);
        if (ks + 2 * U < k1) sa.load(wbase, xrow, p, ks + 2 * U, nq, nl);
        if (has_b) sb.accumulate(acc, uc);
    }

    // ---- sum the W wavefronts of the work-group in wave order (LDS) ----
    if (W > 1) {
        if (wave > 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rl = mt * 16 + lg * 4 + r;
                    if (rl < rows)
                        *reinterpret_cast<float4*>(&red[((wave - 1) * rows + rl) * kStripN + lc * 4]) =
                            make_float4(acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]);
                }
        }
        __syncthreads();
        if (wave != 0) return;
    }

    float4 out[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rl = mt * 16 + lg * 4 + r;
            float4 v = make_float4(acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]);
            if (rl < rows) {
                for (int w = 0; w < W - 1; ++w) {
                    const float4 o = *reinterpret_cast<const float4*>(&red[(w * rows + rl) * kStripN + lc * 4]);
                    v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
                }
            }
            out[mt][r] = v;
        }

    auto store_y = [&](int rl, float4 v) {
        const half2_t a = half2_t{(_Float16)v.x, (_Float16)v.y};
        const half2_t b = half2_t{(_Float16)v.z, (_Float16)v.w};
        *reinterpret_cast<uint2*>(p.y + (size_t)(row0 + rl) * p.N + n) = make_uint2(as_u32(a), as_u32(b));
    };

    if (p.splits == 1) {
        if (!col_ok) return;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rl = mt * 16 + lg * 4 + r;
                if (rl < rows) store_y(rl, out[mt][r]);
            }
        return;
    }

    // ---- split-K: publish this work-group's partial, the last arrival reduces ----
    // On gfx950 an agent-scope fence writes back and invalidates the whole L2, which costs
    // far more than this kernel's work when every work-group issues one. The partials are
    // therefore written and read with agent-scope atomic stores/loads, which go to the
    // coherent level and bypass stale cache lines, and ordering needs only a wait for this
    // wavefront's memory operations: partial stores complete before the arrival counter is
    // incremented, and the last arrival reads the partials only after its increment returns.
    const size_t counter = (size_t)blockIdx.y * p.n_strips + strip;
    const size_t slab = (size_t)16 * MT * kStripN;                        // floats per partial
    float* __restrict__ base = p.ws + (counter * p.splits) * slab;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rl = mt * 16 + lg * 4 + r;
            if (rl < rows) {
                float* dst = base + split * slab + rl * kStripN + lc * 4;
                __hip_atomic_store(dst + 0, out[mt][r].x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(dst + 1, out[mt][r].y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(dst + 2, out[mt][r].z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(dst + 3, out[mt][r].w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);           // partial stores have completed
    uint32_t ticket = 0;
    if (lane == 0)
        ticket = __hip_atomic_fetch_add(&p.counters[counter], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ticket = __shfl(ticket, 0);
    if (ticket != (uint32_t)(p.splits - 1)) return;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);           // counter read before any partial load
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

    if (col_ok) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rl = mt * 16 + lg * 4 + r;
                if (rl < rows) {
                    const float* src = base + rl * kStripN + lc * 4;
                    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                    for (int s = 0; s < p.splits; ++s) {               // fixed order 0..splits-1
                        const float* q = src + s * slab;
                        v.x += __hip_atomic_load(q + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        v.y += __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        v.z += __hip_atomic_load(q + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        v.w += __hip_atomic_load(q + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    store_y(rl, v);
                }
            }
    }
    if (lane == 0)                                     // ready for the next call
        __hip_atomic_store(&p.counters[counter], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MT, int U, int W>
hipError_t launch_one(const SkinnyParams& p, hipStream_t s) {
    const dim3 grid((unsigned)(p.n_strips * p.splits), (unsigned)p.row_blocks);
    const int rows = std::min(16 * MT, p.M);
    const size_t lds = (size_t)(W - 1) * rows * kStripN * sizeof(float);
    hipLaunchKernelGGL((skinny_kernel<MT, U, W>), grid, dim3(64 * W), lds, s, p);
    return hipGetLastError();
}

}  // namespace

bool skinny_config_supported(int row_tiles, int waves) {
    if (row_tiles < 1 || row_tiles > 4) return false;
    if (waves != 4 && waves != 8 && waves != 16) return false;
    // LDS for the wave reduction: (waves - 1) * 16 * row_tiles rows of 256 bytes
    return (waves - 1) * 16 * row_tiles * kStripN * 4 <= 64 * 1024;
}

int launch_skinny(const SkinnyParams& p, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int u = p.kc >= kGS ? kGS : p.kc;
    if ((p.kc >= kGS && p.kc % kGS != 0) || u == 3 || u < 1 || !skinny_config_supported(p.row_tiles, p.waves))
        return (int)hipErrorInvalidValue;
#define W4A16_SKINNY_CASE(MT, U, W) \
    if (p.row_tiles == MT && u == U && p.waves == W) return (int)launch_one<MT, U, W>(p, s);
#define W4A16_SKINNY_U(MT, W) W4A16_SKINNY_CASE(MT, 1, W) W4A16_SKINNY_CASE(MT, 2, W) W4A16_SKINNY_CASE(MT, 4, W)
    W4A16_SKINNY_U(1, 4) W4A16_SKINNY_U(1, 8) W4A16_SKINNY_U(1, 16)
    W4A16_SKINNY_U(2, 4) W4A16_SKINNY_U(2, 8)
    W4A16_SKINNY_U(3, 4)
    W4A16_SKINNY_U(4, 4)
#undef W4A16_SKINNY_U
#undef W4A16_SKINNY_CASE
    return (int)hipErrorInvalidValue;
}

}  // namespace w4a16
