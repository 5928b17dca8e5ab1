// Prefill-sized W4A16 kernel for gfx950: LDS-staged fp16 tiles feeding MFMA.
//
// What it computes: y = x . dequant(Wq) ("Beating FP16 with 4-bit Weights: A Portable W4A16
// GEMM in Triton", section "The design": load each packed int32 once, unpack all eight
// nibbles, dequantise with the group's scale and zero, multiply on the matrix cores with
// fp32 accumulation). Once M is large the product is a dense contraction, so each
// work-group dequantises its weight tile once into LDS and every wavefront reuses it
// across 64 rows of M.
//
// Tiling: a work-group computes a 128 x 128 tile of y with 4 wavefronts (2 x 2, 64 x 64
// each = 4 x 4 tiles of v_mfma_f32_16x16x32_f16) and walks K in steps of 64 rows:
//  * weights: thread t loads one 16-byte word quad (packed row t/32 of the step, columns
//    4*(t%32)..+3), dequantises the 4 words to fp16 (q - zero) * scale (one rounding of
//    the exact product) and stores each column's 8 values as one 16-byte LDS chunk;
//  * activations: 128 rows x 64 K as 16-byte chunks, permuted to the unpacked K order;
//  * an MFMA operand of one lane is then exactly one 16-byte LDS chunk (ds_read_b128);
//  * the global loads of step k+1 are issued before the MFMAs of step k.
// LDS rows are padded by one chunk so that the 16 lanes reading one column of chunks hit
// distinct bank groups.
#include <hip/hip_runtime.h>

#include "w4a16_device.hpp"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {

constexpr int BM = kPrefillBM, BN = kPrefillBN, BK = kPrefillBK;
constexpr int KCH = BK / 8;            // 16-byte chunks per row (activations) or column (weights)
constexpr int LDSW = KCH + 1;          // padded chunks per LDS row

__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams p) {
    __shared__ uint4 a_lds[BM * LDSW];
    __shared__ uint4 b_lds[BN * LDSW];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const size_t nq = (size_t)(p.N >> 2);
    const uint4* __restrict__ qw = reinterpret_cast<const uint4*>(p.qweight);

    // weight loader: packed row br of the step, column quad bc
    const int br = tid >> 5, bc = tid & 31;
    const int bn = n0 + 4 * bc;
    const int bnl = bn < p.N ? bn : 0;                   // in-bounds; such columns are not stored
    // activation loader: chunks tid + 256*i, row id/8, chunk id%8 (rows beyond M clamp)
    const uint16_t* arow[4];
    int aslot[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int id = tid + 256 * i;
        arow[i] = p.x + (size_t)min(m0 + id / KCH, p.M - 1) * p.K + (id % KCH) * 8;
        aslot[i] = (id / KCH) * LDSW + id % KCH;
    }
    const UnpackConsts uc = unpack_consts();

    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int KT = p.K / BK;
    uint4 av[4], bw;
    uint2 sv, zv;
    auto load_step = [&](int kt) {
        const int grp = (kt * BK) / kGroup;
        bw = qw[(size_t)(kt * KCH + br) * nq + (bnl >> 2)];
        sv = *reinterpret_cast<const uint2*>(p.scales + (size_t)grp * p.N + bnl);
        zv = *reinterpret_cast<const uint2*>(p.zeros + (size_t)grp * p.N + bnl);
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = *reinterpret_cast<const uint4*>(arow[i] + (size_t)kt * BK);
    };
    load_step(0);

    for (int kt = 0; kt < KT; ++kt) {
        __syncthreads();                                  // previous step's reads are done
#pragma unroll
        for (int i = 0; i < 4; ++i) a_lds[aslot[i]] = __builtin_bit_cast(uint4, permute_x(av[i]));
        {
            const half2_t z01 = as_h2(zv.x), z23 = as_h2(zv.y);
            const half2_t s01 = as_h2(sv.x), s23 = as_h2(sv.y);
            const _Float16 zc[4] = {z01[0], z01[1], z23[0], z23[1]};
            const _Float16 sc[4] = {s01[0], s01[1], s23[0], s23[1]};
            const uint32_t words[4] = {bw.x, bw.y, bw.z, bw.w};
#pragma unroll
            for (int c = 0; c < 4; ++c)
                b_lds[(4 * bc + c) * LDSW + br] =
                    __builtin_bit_cast(uint4, dequant_frag(words[c], zero_offsets(zc[c]), sc[c], uc));
        }
        __syncthreads();
        if (kt + 1 < KT) load_step(kt + 1);               // in flight during the MFMAs below

#pragma unroll
        for (int s = 0; s < KCH / 4; ++s) {
            half8_t a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = __builtin_bit_cast(half8_t, a_lds[(wm * 64 + 16 * i + lr) * LDSW + 4 * s + lg]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = __builtin_bit_cast(half8_t, b_lds[(wn * 64 + 16 * j + lr) * LDSW + 4 * s + lg]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }

    // epilogue: lane holds rows 4*lg + r, column lr of each 16 x 16 tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 64 + 16 * j + lr;
            if (col >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * 64 + 16 * i + 4 * lg + r;
                if (row < p.M) p.y[(size_t)row * p.N + col] = f16_bits((_Float16)acc[i][j][r]);
            }
        }
}

}  // namespace

int launch_prefill(const PrefillParams& p, void* stream) {
    const dim3 grid((unsigned)((p.N + BN - 1) / BN), (unsigned)((p.M + BM - 1) / BM));
    hipLaunchKernelGGL(prefill_kernel, grid, dim3(256), 0, reinterpret_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

}  // namespace w4a16
