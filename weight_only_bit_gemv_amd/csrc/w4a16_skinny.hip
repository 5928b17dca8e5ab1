// Decode / skinny-M W4A16 kernel for gfx950: a single pass over the packed weight stream.
//
// What it computes: y = x . dequant(Wq) ("Beating FP16 with 4-bit Weights: A Portable W4A16
// GEMM in Triton", section "The design"), with the split-K decode strategy of the same page
// (extra parallelism along K when M is small, section "The design" and "Things I got
// wrong along the way") but with a deterministic fixed-order reduction instead of fp32
// atomics.
//
// Mapping (one work-group = 4 wavefronts = one 64-column strip x one K range):
//  * lane l reads one 16-byte word quad per K-step: packed row 4*ks + l/16, columns
//    strip*64 + 4*(l%16) .. +3. A wavefront's load is 4 rows x 256 contiguous bytes; every
//    packed int32 of qweight is read exactly once per 16-row block of M.
//  * each of the lane's 4 words is the B operand of one v_mfma_f32_16x16x32_f16: a lane of
//    that MFMA holds 8 K values of one column, which is exactly one packed word. Four MFMA
//    tiles cover columns {4j + t}; their outputs land back on the lane that owns the column.
//  * the words are unpacked to exact fp16 (q - zero) values; x (rows padded to 16 with
//    zeros) is the A operand in the same K order; products accumulate in fp32 per 128-row
//    group and the group's fp32 partial is multiplied by the column's scale once:
//    sum_k x_k (q_k - z) s = s * sum_k x_k (q_k - z) over a group, which keeps every
//    product exact.
//  * the 4 wavefronts of a work-group stream consecutive K ranges and are summed in LDS in
//    wave order; with more than one work-group along K (splits > 1) each writes its fp32
//    partial to the workspace, and the last to arrive (arrival counter) sums the splits in
//    index order 0..splits-1 and writes y. Results are bitwise reproducible.
#include <hip/hip_runtime.h>

#include "w4a16_device.hpp"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {

constexpr int kGS = kGroup / kKStep;    // K-steps per scale/zero group (4)

// MT: 16-row MFMA tiles of M per work-group. U: K-steps per segment, min(kc, 4); the
// dispatcher keeps kc in {1, 2} or a multiple of 4, so every segment is exactly U K-steps
// inside one 128-row group and the loop below needs no predicates.
template <int MT, int U>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyParams p) {
    static_assert(U == 1 || U == 2 || U == kGS, "segment must divide a group");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lg = lane >> 4;            // which of the 4 packed rows of a K-step
    const int lc = lane & 15;            // column quad within the strip / A-operand row
    const int strip = blockIdx.x % p.n_strips;
    const int split = blockIdx.x / p.n_strips;
    const int row0 = blockIdx.y * 16 * MT;
    const int n = strip * kStripN + lc * 4;
    const bool col_ok = n < p.N;
    const int nl = col_ok ? n : 0;       // loads stay in bounds; results of such lanes are dropped
    const int KS = p.K / kKStep;
    const int chunk = split * kSkinnyWaves + wave;
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

    for (int ks = k0; ks < k1; ks += U) {
        const int grp = ks / kGS;
        uint4 wv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) wv[u] = wbase[(size_t)(ks + u) * 4 * nq];
        const uint2 sv = *reinterpret_cast<const uint2*>(p.scales + (size_t)grp * p.N + nl);
        const uint2 zv = *reinterpret_cast<const uint2*>(p.zeros + (size_t)grp * p.N + nl);
        half8_t xa[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                xa[u][mt] = permute_x(*reinterpret_cast<const uint4*>(xrow[mt] + (size_t)(ks + u) * kKStep));

        const half2_t z01 = as_h2(zv.x), z23 = as_h2(zv.y);
        const ZeroOffsets zo[4] = {zero_offsets(z01[0]), zero_offsets(z01[1]),
                                   zero_offsets(z23[0]), zero_offsets(z23[1])};
        floatx4 part[MT][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t words[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const half8_t b = unpack_sub(words[t], zo[t], uc);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    part[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        xa[u][mt], b, u == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : part[mt][t], 0, 0, 0);
            }
        }
        const half2_t s01 = as_h2(sv.x), s23 = as_h2(sv.y);
        const float sc[4] = {(float)s01[0], (float)s01[1], (float)s23[0], (float)s23[1]};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[mt][t] += sc[t] * part[mt][t];
    }

    // ---- sum the 4 wavefronts of the work-group in wave order (LDS) ----
    __shared__ float red[kSkinnyWaves - 1][16 * MT][kStripN];
    if (wave > 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rl = mt * 16 + lg * 4 + r;
                if (row0 + rl < p.M)
                    *reinterpret_cast<float4*>(&red[wave - 1][rl][lc * 4]) =
                        make_float4(acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]);
            }
    }
    __syncthreads();
    if (wave != 0) return;

    float4 out[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rl = mt * 16 + lg * 4 + r;
            float4 v = make_float4(acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]);
            if (row0 + rl < p.M) {
#pragma unroll
                for (int w = 0; w < kSkinnyWaves - 1; ++w) {
                    const float4 o = *reinterpret_cast<const float4*>(&red[w][rl][lc * 4]);
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
                if (row0 + rl < p.M) store_y(rl, out[mt][r]);
            }
        return;
    }

    // ---- split-K: publish this work-group's partial, the last arrival reduces ----
    const size_t counter = (size_t)blockIdx.y * p.n_strips + strip;
    const size_t slab = (size_t)16 * MT * kStripN;                        // floats per partial
    float* __restrict__ base = p.ws + (counter * p.splits) * slab;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rl = mt * 16 + lg * 4 + r;
            if (row0 + rl < p.M)
                *reinterpret_cast<float4*>(base + split * slab + rl * kStripN + lc * 4) = out[mt][r];
        }
    __threadfence();                                   // partial visible device-wide
    uint32_t ticket = 0;
    if (lane == 0) ticket = atomicAdd(&p.counters[counter], 1u);
    ticket = __shfl(ticket, 0);
    if (ticket != (uint32_t)(p.splits - 1)) return;
    __threadfence();                                   // see every other split's partial

    if (col_ok) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rl = mt * 16 + lg * 4 + r;
                if (row0 + rl < p.M) {
                    const float* src = base + rl * kStripN + lc * 4;
                    float4 v = *reinterpret_cast<const float4*>(src);
                    for (int s = 1; s < p.splits; ++s) {
                        const float4 o = *reinterpret_cast<const float4*>(src + s * slab);
                        v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
                    }
                    store_y(rl, v);
                }
            }
    }
    if (lane == 0) atomicExch(&p.counters[counter], 0u);   // ready for the next call
}

}  // namespace

int launch_skinny(const SkinnyParams& p, void* stream) {
    const dim3 grid((unsigned)(p.n_strips * p.splits), (unsigned)p.row_blocks);
    const dim3 block(64 * kSkinnyWaves);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int u = p.kc >= kGS ? kGS : p.kc;
    if ((p.kc >= kGS && p.kc % kGS != 0) || u == 3 || u < 1 || p.row_tiles < 1 || p.row_tiles > 4)
        return (int)hipErrorInvalidValue;
#define W4A16_SKINNY_CASE(MT, U) \
    if (p.row_tiles == MT && u == U) { hipLaunchKernelGGL((skinny_kernel<MT, U>), grid, block, 0, s, p); }
    W4A16_SKINNY_CASE(1, 1) W4A16_SKINNY_CASE(1, 2) W4A16_SKINNY_CASE(1, 4)
    W4A16_SKINNY_CASE(2, 1) W4A16_SKINNY_CASE(2, 2) W4A16_SKINNY_CASE(2, 4)
    W4A16_SKINNY_CASE(3, 1) W4A16_SKINNY_CASE(3, 2) W4A16_SKINNY_CASE(3, 4)
    W4A16_SKINNY_CASE(4, 1) W4A16_SKINNY_CASE(4, 2) W4A16_SKINNY_CASE(4, 4)
#undef W4A16_SKINNY_CASE
    return (int)hipGetLastError();
}

}  // namespace w4a16
