// Prefill-sized W4A16 kernel for gfx950, tile 1: weights straight from HBM into MFMA
// registers, only the activations staged in LDS.
//
// What it computes: y = x . dequant(Wq) ("Beating FP16 with 4-bit Weights: A Portable W4A16
// GEMM in Triton", section "The design": each packed int32 is loaded once, its eight
// nibbles are dequantised with the group's scale and zero, and the products accumulate in
// fp32 on the matrix cores).
#include <hip/hip_runtime.h>

#include "w4a16_device.hpp"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {

constexpr int BK = 64;                 // K rows per stage (two 32-row K-steps)
constexpr int KCH = BK / 8;            // 16-byte activation chunks per row and stage
constexpr int LDSW = KCH + 1;          // padded chunks per LDS row
constexpr int NT = 256;                // threads per work-group
constexpr int kRsrcRaw = 0x00020000;   // buffer resource word 3 for raw (untyped) access on gfx9

// Tile 1: weights straight from HBM into MFMA registers; only the activations go through LDS.
//
// A work-group computes a 128 x 256 tile of y with 4 wavefronts side by side along N; each
// wavefront owns all 128 rows x 64 columns (8 x 4 tiles of v_mfma_f32_16x16x32_f16). The
// packed weights need no LDS: as in the decode kernel, lane (c, g) of a wavefront loads one
// 16-byte quad per K-step (packed row 4 * ks + g, columns 4c .. 4c+3 of the wavefront's
// strip), and word t of the quad is exactly that lane's B operand for column tile t (tile t
// holds columns {4c + t}). Each word is dequantised in registers to fp16 (q - zero) * scale
// (one rounding of the exact product, the same values the LDS tile above holds), so a
// weight is dequantised once per work-group and read from HBM once per 128 rows of M.
// The activations (128 rows x 64 K per stage) are staged in LDS once per work-group and
// read by all four wavefronts: per MFMA a wavefront reads 256 bytes of LDS, a third of
// what the 128 x 128 tile reads (where both operands go through LDS), which moves the
// bound from LDS bandwidth to the matrix cores.
// Two work-groups per compute unit (two wavefronts per SIMD), accumulators in VGPRs, which
// leaves registers for one activation set and two weight sets: activation loads one stage
// ahead (they mostly hit L2: every column strip re-reads the same rows), stored to LDS at
// the end of the stage (two buffers, one barrier per stage); weight quads and their
// scales/zeros two stages ahead. Deeper register rings need more than 256 registers (a
// three-set weight ring spills and measured slower). G32: 32-row groups (two scale/zero
// loads per 64-row stage); otherwise a stage lies inside one group.
template <int OCC, bool G32, bool NAT>
__global__ __launch_bounds__(NT, OCC) void prefill_rb_kernel(PrefillParams p) {
    constexpr int BM = 128;
    constexpr int WNC = 64;                    // columns per wavefront
    constexpr int BN = 4 * WNC;
    constexpr int TI = BM / 16;                // 16-row MFMA tiles per wavefront
    constexpr int AL = BM * KCH / NT;          // activation chunks loaded per thread per stage
    __shared__ uint4 a_lds[2][BM * LDSW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int nw = n0 + wave * WNC + 4 * lr;                 // the lane's first column
    const bool col_ok = nw < p.N;                            // N % 4 == 0: all four or none
    const int nl = col_ok ? nw : 0;                          // in-bounds; such columns are not stored
    const size_t nq = (size_t)(p.N >> 2);
    // Loads take a wave-uniform 64-bit base (scalar registers) plus a 32-bit per-lane offset,
    // which keeps one VGPR per address instead of a 64-bit pointer per load.
    const uint32_t q_off = (uint32_t)lg * (uint32_t)nq + (uint32_t)(nl >> 2);   // in uint4 units
    const int ar = tid / KCH, ac = tid % KCH;
    uint32_t x_off[AL];                                          // in uint16 units
#pragma unroll
    for (int i = 0; i < AL; ++i)
        x_off[i] = (uint32_t)min(m0 + ar + (NT / KCH) * i, p.M - 1) * (uint32_t)p.K + (uint32_t)(ac * 8);
    const UnpackConsts uc = unpack_consts();

    floatx4 acc[TI][4];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int KT = p.K / BK;                                 // even: K is a multiple of 128
    struct RegsA { uint4 av[AL]; };
    constexpr int NSZ = G32 ? 2 : 1;                        // scale/zero loads per stage
    struct RegsB { uint4 bw[2]; uint2 sv[NSZ], zv[NSZ]; };   // the stage's two K-steps
    // raw buffer loads: the resource (base address) is built in scalar registers from a
    // wave-uniform pointer, the per-lane part is a 32-bit byte offset; every access is in
    // bounds by construction, so the range check is left wide open
    auto rsrc = [](const void* base) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, kRsrcRaw);
    };
    auto load_a = [&](RegsA& r, int kt) {
        const auto rs = rsrc(p.x + (size_t)kt * BK);
#pragma unroll
        for (int i = 0; i < AL; ++i)
            r.av[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(x_off[i] * 2u), 0, 0));
    };
    auto load_b = [&](RegsB& r, int kt) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const auto rs = rsrc(reinterpret_cast<const uint4*>(p.qweight) + (size_t)(8 * kt + 4 * j) * nq);
            r.bw[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(q_off * 16u), 0, 0));
        }
#pragma unroll
        for (int j = 0; j < NSZ; ++j) {
            const size_t grp = (size_t)((kt * BK + 32 * j) >> p.group_shift);
            r.sv[j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsrc(p.scales + grp * p.N), nl * 2, 0, 0));
            r.zv[j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsrc(p.zeros + grp * p.N), nl * 2, 0, 0));
        }
    };
    auto store_a = [&](const RegsA& r, int buf) {
#pragma unroll
        for (int i = 0; i < AL; ++i)
            a_lds[buf][(ar + (NT / KCH) * i) * LDSW + ac] = __builtin_bit_cast(uint4, x_frag<NAT>(r.av[i]));
    };
    auto mma = [&](const RegsB& r, int buf) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int g = G32 ? j : 0;
            const half2_t z01 = as_h2(r.zv[g].x), z23 = as_h2(r.zv[g].y);
            const half2_t s01 = as_h2(r.sv[g].x), s23 = as_h2(r.sv[g].y);
            const _Float16 zc[4] = {z01[0], z01[1], z23[0], z23[1]};
            const _Float16 sc[4] = {s01[0], s01[1], s23[0], s23[1]};
            const uint32_t words[4] = {r.bw[j].x, r.bw[j].y, r.bw[j].z, r.bw[j].w};
            half8_t b[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) b[t] = dequant_frag(words[t], zero_offsets(zc[t]), sc[t], uc);
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                const half8_t a = __builtin_bit_cast(half8_t, a_lds[buf][(16 * i + lr) * LDSW + 4 * j + lg]);
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[t], acc[i][t], 0, 0, 0);
            }
            // LDS reads paced with the MFMAs (one activation fragment per four MFMAs) and one
            // K-step at a time: hoisting all reads, or the second step's dequant, above the
            // MFMAs would need more than 256 registers
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // 4 MFMA
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    RegsA ra;
    RegsB rb0, rb1;
    load_a(ra, 0);
    load_b(rb0, 0);
    load_b(rb1, 1);
    store_a(ra, 0);
    __syncthreads();
    load_a(ra, 1);
    for (int kt = 0; kt + 2 < KT; kt += 2) {
        __builtin_amdgcn_sched_barrier(0);
        mma(rb0, 0);                                      // stage kt
        load_b(rb0, kt + 2);
        store_a(ra, 1);                                   // stage kt + 1
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        load_a(ra, kt + 2);
        __builtin_amdgcn_sched_barrier(0);
        mma(rb1, 1);                                      // stage kt + 1
        load_b(rb1, kt + 3);
        store_a(ra, 0);                                   // stage kt + 2
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        load_a(ra, kt + 3);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma(rb0, 0);                                          // stage KT - 2
    store_a(ra, 1);                                       // stage KT - 1
    __syncthreads();
    mma(rb1, 1);

    // epilogue: lane holds rows 4*lg + r of columns nw + t (t = 0..3) of each row tile
    if (!col_ok) return;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m0 + 16 * i + 4 * lg + r;
            if (row < p.M) {
                const half2_t lo = half2_t{(_Float16)acc[i][0][r], (_Float16)acc[i][1][r]};
                const half2_t hi = half2_t{(_Float16)acc[i][2][r], (_Float16)acc[i][3][r]};
                *reinterpret_cast<uint2*>(p.y + (size_t)row * p.N + nw) = make_uint2(as_u32(lo), as_u32(hi));
            }
        }
}

}  // namespace

int launch_prefill_rb(const PrefillParams& p, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)((p.N + 255) / 256), (unsigned)((p.M + 127) / 128));
    const bool g32 = p.group_shift == 5, nat = p.layout == W4A16_LAYOUT_INTERLEAVED;
    if (g32 && nat) hipLaunchKernelGGL((prefill_rb_kernel<2, true, true>), grid, dim3(NT), 0, s, p);
    else if (g32) hipLaunchKernelGGL((prefill_rb_kernel<2, true, false>), grid, dim3(NT), 0, s, p);
    else if (nat) hipLaunchKernelGGL((prefill_rb_kernel<2, false, true>), grid, dim3(NT), 0, s, p);
    else hipLaunchKernelGGL((prefill_rb_kernel<2, false, false>), grid, dim3(NT), 0, s, p);
    return (int)hipGetLastError();
}

}  // namespace w4a16
