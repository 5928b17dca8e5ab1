// Prefill-sized W4A16 kernel for gfx950: LDS-staged fp16 tiles feeding MFMA.
//
// What it computes: y = x . dequant(Wq) ("Beating FP16 with 4-bit Weights: A Portable W4A16
// GEMM in Triton", section "The design": load each packed int32 once, unpack all eight
// nibbles, dequantise with the group's scale and zero, multiply on the matrix cores with
// fp32 accumulation). Once M is large the product is a dense contraction, so each
// work-group dequantises its weight tile once into LDS and every wavefront reuses it
// across 64 rows of M.
//
// Tiling: a work-group computes a BM x BN = 128 x 128 tile of y with 4 wavefronts in a
// 2 x 2 grid, each owning a 64 x 64 block = 4 x 4 tiles of v_mfma_f32_16x16x32_f16 with
// fp32 accumulators; two work-groups share a compute unit (two wavefronts per SIMD). K
// advances in stages of 64 rows through two LDS buffers:
//  * weights: thread t loads one 16-byte word quad (packed row t/32 of the stage, columns
//    4*(t%32) .. +3), dequantises each word to 8 fp16 values (q - zero) * scale (one
//    rounding of the exact product) and stores them as one 16-byte LDS chunk: B is held
//    column-major, a column's 64 K values in 8 chunks;
//  * activations: 128 rows x 64 K as 16-byte chunks, permuted to the unpacked K order;
//  * an MFMA operand of one lane is exactly one 16-byte LDS chunk (ds_read_b128);
//  * the global loads of stage k+2 are issued before the MFMAs of stage k, and stage k+1
//    (loaded a stage earlier) is dequantised and written to the other LDS buffer while
//    those MFMAs run, so a load has two stages of MFMAs to arrive and there is one
//    barrier per stage.
// LDS rows and columns are padded to 9 chunks (144 bytes): the 16 lanes that read one
// chunk of 16 consecutive rows then touch 16 disjoint groups of 4 banks.
#include <hip/hip_runtime.h>

#include "w4a16_device.hpp"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {

constexpr int BK = 64;                 // K rows per stage
constexpr int KCH = BK / 8;            // 16-byte chunks per row (activations) or column (weights)
constexpr int LDSW = KCH + 1;          // padded chunks per LDS row / column
constexpr int NT = 256;                // threads per work-group

// LDS slot of chunk `chunk` of weight-tile column `col`: the chunk index XOR bits 3..5 of
// the column. Each thread stores one chunk of 4 consecutive columns, 64 lanes cover 128
// columns, and an MFMA operand read takes one chunk of 16 consecutive columns; with the
// column stride of 9 chunks plus this swizzle both patterns are free of LDS bank conflicts
// (measured with the SQ_LDS_BANK_CONFLICT counter; without it the stores conflict 4-way).
__device__ __forceinline__ int bslot(int col, int chunk) { return chunk ^ ((col >> 3) & 7); }

template <int BM, int BN, int OCC, bool NAT>
__global__ __launch_bounds__(NT, OCC) void prefill_kernel(PrefillParams p) {
    constexpr int WM = BM / 2;         // rows per wavefront
    constexpr int WN = BN / 2;         // columns per wavefront
    constexpr int TI = WM / 16;        // 16-row MFMA tiles per wavefront
    constexpr int TJ = WN / 16;        // 16-column MFMA tiles per wavefront
    constexpr int AL = BM * KCH / NT;  // activation chunks loaded per thread per stage
    constexpr int BQ = BN / 4;         // 16-byte word quads per packed row of the tile
    constexpr int BL = BN * KCH / 4 / NT;   // word quads loaded per thread per stage
    __shared__ uint4 a_lds[2][BM * LDSW];
    __shared__ uint4 b_lds[2][BN * LDSW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const size_t nq = (size_t)(p.N >> 2);
    const uint4* __restrict__ qw = reinterpret_cast<const uint4*>(p.qweight);

    // weight loader: word quads tid + NT * h -> packed row br + (NT / BQ) * h, column quad bc
    const int br = tid / BQ, bc = tid % BQ;
    const int bn = n0 + 4 * bc;
    const int bnl = bn < p.N ? bn : 0;                   // in-bounds; such columns are not stored
    // activation loader: chunk id = tid + NT * i -> row ar + (NT / KCH) * i, chunk ac (rows
    // beyond M are clamped to row M - 1: they only feed output rows that are not stored)
    const int ar = tid / KCH, ac = tid % KCH;
    const uint16_t* __restrict__ xcol = p.x + ac * 8;
    const UnpackConsts uc = unpack_consts();

    floatx4 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int KT = p.K / BK;                              // even: K is a multiple of 128
    // One stage of global data in registers: activation chunks, weight quads, scale/zero.
    struct Regs {
        uint4 av[AL], bw[BL];
        uint2 sv, zv;
    };
    auto load_stage = [&](Regs& r, int kt) {
        // the thread's packed rows lie in one group: groups are >= 32 rows, packed rows
        // br + (NT / BQ) * h of a stage differ by multiples of 8 * (NT / BQ) >= 64 rows only
        // when BL > 1, which needs BN > 128 (not built)
        static_assert(BL == 1, "one word quad per thread per stage");
        const int grp = (kt * BK + 8 * br) >> p.group_shift;
#pragma unroll
        for (int h = 0; h < BL; ++h) r.bw[h] = qw[(size_t)(kt * KCH + br + (NT / BQ) * h) * nq + (bnl >> 2)];
        r.sv = *reinterpret_cast<const uint2*>(p.scales + (size_t)grp * p.N + bnl);
        r.zv = *reinterpret_cast<const uint2*>(p.zeros + (size_t)grp * p.N + bnl);
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const int row = min(m0 + ar + (NT / KCH) * i, p.M - 1);
            r.av[i] = *reinterpret_cast<const uint4*>(xcol + (size_t)row * p.K + (size_t)kt * BK);
        }
    };
    auto store_stage = [&](const Regs& r, int buf) {
#pragma unroll
        for (int i = 0; i < AL; ++i)
            a_lds[buf][(ar + (NT / KCH) * i) * LDSW + ac] = __builtin_bit_cast(uint4, x_frag<NAT>(r.av[i]));
        const half2_t z01 = as_h2(r.zv.x), z23 = as_h2(r.zv.y);
        const half2_t s01 = as_h2(r.sv.x), s23 = as_h2(r.sv.y);
        const _Float16 zc[4] = {z01[0], z01[1], z23[0], z23[1]};
        const _Float16 sc[4] = {s01[0], s01[1], s23[0], s23[1]};
#pragma unroll
        for (int h = 0; h < BL; ++h) {
            const uint32_t words[4] = {r.bw[h].x, r.bw[h].y, r.bw[h].z, r.bw[h].w};
#pragma unroll
            for (int c = 0; c < 4; ++c)
                b_lds[buf][(4 * bc + c) * LDSW + bslot(4 * bc + c, br + (NT / BQ) * h)] =
                    __builtin_bit_cast(uint4, dequant_frag(words[c], zero_offsets(zc[c]), sc[c], uc));
        }
    };
    auto mma_stage = [&](int buf) {
#pragma unroll
        for (int s = 0; s < KCH / 4; ++s) {
            half8_t a[TI];
#pragma unroll
            for (int i = 0; i < TI; ++i)
                a[i] = __builtin_bit_cast(half8_t, a_lds[buf][(wm * WM + 16 * i + lr) * LDSW + 4 * s + lg]);
#pragma unroll
            for (int jh = 0; jh < TJ; jh += 4) {   // B fragments four at a time
                half8_t b[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    b[j] = __builtin_bit_cast(half8_t, b_lds[buf][(wn * WN + 16 * (jh + j) + lr) * LDSW +
                                                                  bslot(wn * WN + 16 * (jh + j) + lr, 4 * s + lg)]);
#pragma unroll
                for (int i = 0; i < TI; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][jh + j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][jh + j], 0, 0, 0);
            }
        }
    };

    // Pipeline: global loads run two stages ahead of the MFMAs (register sets r0, r1), LDS
    // stores one stage ahead (buffers 0, 1); one barrier per stage. The loop body has no
    // branch (the last two stages are peeled): a branch inside it makes the register
    // allocator shuttle the accumulators between registers.
    // The MFMAs of a stage and the dequantisation + LDS stores of the next one form one
    // scheduling region, interleaved by sched_group_barrier: one MFMA, then a few VALU
    // instructions and one LDS access, repeated. The MFMA pipe then keeps working while the
    // wave unpacks weights, and the first MFMA never waits for the next stage's global
    // loads (left to itself the scheduler hoists the unpacking above the MFMAs).
    constexpr int NMFMA = TI * TJ * (KCH / 4);            // MFMAs per stage per wavefront
    auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < NMFMA; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // 3 VALU
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // 1 LDS write
        }
    };
    Regs r0, r1;
    load_stage(r0, 0);
    load_stage(r1, 1);
    store_stage(r0, 0);
    __syncthreads();
    for (int kt = 0; kt + 2 < KT; kt += 2) {
        load_stage(r0, kt + 2);
        __builtin_amdgcn_sched_barrier(0);
        mma_stage(0);                                     // stage kt
        store_stage(r1, 1);                               // stage kt + 1
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        load_stage(r1, kt + 3);
        __builtin_amdgcn_sched_barrier(0);
        mma_stage(1);                                     // stage kt + 1
        store_stage(r0, 0);                               // stage kt + 2
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    }
    mma_stage(0);                                         // stage KT - 2
    store_stage(r1, 1);                                   // stage KT - 1
    __syncthreads();
    mma_stage(1);

    // epilogue: lane holds rows 4*lg + r, column lr of each 16 x 16 tile
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int col = n0 + wn * WN + 16 * j + lr;
            if (col >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * WM + 16 * i + 4 * lg + r;
                if (row < p.M) p.y[(size_t)row * p.N + col] = f16_bits((_Float16)acc[i][j][r]);
            }
        }
}

}  // namespace

int launch_prefill(const PrefillParams& p, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p.tile == W4A16_TILE_REGISTER_B) return launch_prefill_rb(p, stream);
    if (p.tile == W4A16_TILE_ASYNC) return launch_prefill_async(p, stream);
    if (p.tile != W4A16_TILE_LDS) return (int)hipErrorInvalidValue;
    const dim3 grid((unsigned)((p.N + kPrefillBN - 1) / kPrefillBN), (unsigned)((p.M + kPrefillBM - 1) / kPrefillBM));
    if (p.layout == W4A16_LAYOUT_INTERLEAVED)
        hipLaunchKernelGGL((prefill_kernel<kPrefillBM, kPrefillBN, 2, true>), grid, dim3(NT), 0, s, p);
    else
        hipLaunchKernelGGL((prefill_kernel<kPrefillBM, kPrefillBN, 2, false>), grid, dim3(NT), 0, s, p);
    return (int)hipGetLastError();
}

}  // namespace w4a16
