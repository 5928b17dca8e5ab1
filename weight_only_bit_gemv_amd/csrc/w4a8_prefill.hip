// W4A8 on gfx950: 8-bit floating-point (E4M3) activations x the 4-bit weights of the W4A16
// path, on the 8-bit matrix cores ("Beating FP16 with 4-bit Weights: A Portable W4A16 GEMM
// in Triton", section "What's next": FP8 activations for a W4A8 variant; the GemLite
// README lists FP8 x Wn with activations quantised dynamically, one scale per row).
//
// Two kernels:
//   quantize_rows_kernel  x fp16 [M, K] -> codes xq [M, K] (E4M3), row scales sx [M] and
//                         block sums xsum [K/128, Ms] (Ms = M rounded up to 4): sx = amax /
//                         448 (1 for a zero row), xq = E4M3(x / sx), nearest-even,
//                         saturating (the hardware conversion rounds to nearest even; values
//                         are clamped to +-448 first, as it returns NaN above 464);
//                         xsum[b, m] = sum of dec(xq[m, k]) over the 128 k of block b.
//   w4a8_kernel           y = sx * sum_g s_g * sum_{k in g} dec(xq) * (q - z), q - z exact.
//
// The product kernel keeps the tiling of the async W4A16 tile (a work-group computes
// BM x 256 of y, BM = 128, or 64 or 32 when M is that small, 4 wavefronts side by side
// along N, each BM rows x 64 columns as BM/16 x 4 tiles of 16 x 16) and its direct
// global-to-LDS loads, but a stage is one 128-row K block:
// one v_mfma_f32_16x16x128_f8f6f4 per tile covers it. In that instruction lane (r, g)
// (r = lane % 16, g = lane / 16) holds 32 bytes of row r of A and of column r of B, and
// byte j of A pairs with byte j of B, so any assignment of K indices to (g, j) works if both
// sides use it. The kernel gives bytes 0..15 of lane group g the K indices 16 g .. 16 g + 15
// and bytes 16..31 the indices 64 + 16 g .. 64 + 16 g + 15: the activation bytes are then
// the 16-byte LDS chunks g and 4 + g of the row (the four lane groups of one instruction
// read four neighbouring chunks, which a bank-conflict probe showed conflict-free, while
// chunks 2g and 2g + 1 conflict two ways), and the weight bytes come from packed rows
// 2g, 2g + 1, 8 + 2g and 9 + 2g.
// Each tile's product over the block comes out with a zero accumulator and is added to the
// fp32 result times the group's scale of its column (four FMAs per instruction); the row
// scale multiplies the result once at the end.
//
// Weight operand: E4M3(q - zc) with zc the zero point clamped to [-1, 16], so that
// |q - zc| <= 16 and the operand is exact. The magic-number unpack of device.hpp gives
// q - zc exactly in fp16, and v_cvt_scalef32_pk_fp8_f16 (scale 1) converts pairs of it.
// A centred operand keeps the instruction's accumulation accurate: on rows with outlier
// activations its fp32 result differed from the exact sum by about 1.5e-4 of the sum of
// |products| with this operand, and by 5e-4 to 1.2e-3 with an uncentred one (the bare
// code q, exact in E4M3 as q * 2^-9, with the zero point applied afterwards as -z * sum(a)).
// A zero point outside [-1, 16] (a one-signed group) leaves z - zc != 0: a wavefront whose
// columns hold one adds the exact remainder -s (z - zc) S (S: the block sums of the
// activations) to each row tile in fp32 just before storing it, a loop over the
// work-group's blocks. Wavefronts whose zero points all lie in [-1, 16] skip it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "w4a16_device.hpp"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {

typedef int int8v __attribute__((ext_vector_type(8)));
typedef short short2v __attribute__((ext_vector_type(2)));
typedef uint32_t uint4_vec __attribute__((ext_vector_type(4)));

constexpr float kE4M3Max = 448.0f;
constexpr int kRsrcRaw = 0x00020000;     // buffer resource word 3 for raw (untyped) access on gfx9
constexpr int kCpolSc1 = 16;             // device-coherent (sc1) cache policy of a buffer access
// s_waitcnt immediate for vmcnt(0) with expcnt/lgkmcnt left at their maxima (gfx9 encoding)
constexpr int kWaitVmcnt0 = 0 | (0x7 << 4) | (0xf << 8);

// ---- activation quantiser ---------------------------------------------------------------

constexpr int QT = 256;   // threads per row

__global__ __launch_bounds__(QT) void quantize_rows_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ xq,
                                                          float* __restrict__ sx, float* __restrict__ xsum, int M,
                                                          int K, int Ms) {
    const int m = blockIdx.x;
    const uint4* row = reinterpret_cast<const uint4*>(x + (size_t)m * K);   // 8 fp16 per uint4
    const int n8 = K / 8;
    float amax = 0.f;
    for (int i = threadIdx.x; i < n8; i += QT) {
        const half8_t h = __builtin_bit_cast(half8_t, row[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)h[e]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    __shared__ float wmax[QT / 64];
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float s = amax > 0.f ? amax / kE4M3Max : 1.0f;
    if (threadIdx.x == 0) sx[m] = s;
    uint2* out = reinterpret_cast<uint2*>(xq + (size_t)m * K);              // 8 codes per uint2
    // Thread t converts 8 codes per pass; the 16 threads of one 128-code block (K % 128 == 0,
    // so a block's threads are all active together) sum their decoded codes, in a fixed order.
    for (int i = threadIdx.x; i < n8; i += QT) {
        const half8_t h = __builtin_bit_cast(half8_t, row[i]);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = fminf(fmaxf((float)h[e] / s, -kE4M3Max), kE4M3Max);
        int lo = 0, hi = 0;
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], lo, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], hi, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], hi, true);
        out[i] = make_uint2((uint32_t)lo, (uint32_t)hi);
        float sum = ((__builtin_amdgcn_cvt_f32_fp8(lo, 0) + __builtin_amdgcn_cvt_f32_fp8(lo, 1)) +
                     (__builtin_amdgcn_cvt_f32_fp8(lo, 2) + __builtin_amdgcn_cvt_f32_fp8(lo, 3))) +
                    ((__builtin_amdgcn_cvt_f32_fp8(hi, 0) + __builtin_amdgcn_cvt_f32_fp8(hi, 1)) +
                     (__builtin_amdgcn_cvt_f32_fp8(hi, 2) + __builtin_amdgcn_cvt_f32_fp8(hi, 3)));
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) sum += __shfl_xor(sum, off, 16);
        if ((threadIdx.x & 15) == 0) xsum[(size_t)(i >> 4) * Ms + m] = sum;
    }
    if (m == M - 1)                                    // padding rows M .. Ms - 1 of every block
        for (int j = threadIdx.x; j < (K / 128) * (Ms - M); j += QT)
            xsum[(size_t)(j / (Ms - M)) * Ms + M + j % (Ms - M)] = 0.f;
}

// ---- product kernel ---------------------------------------------------------------------

constexpr int NT = 256;                // threads per work-group
constexpr int WNC = 64;                // columns per wavefront
constexpr int BN = 4 * WNC;            // columns per work-group
constexpr int KS = 128;                // K rows per stage (one 8-bit MFMA, one group of 128)
constexpr int NS = 2;                  // LDS ring slots
// A work-group computes BM rows (32, 64 or 128: the library takes the smallest that holds M,
// so small M does not pay for padding rows) x 256 columns. LDS slot in 16-byte chunks:
// activations BM rows x 8 chunks (128 codes), swizzled; packed weights 16 rows x 64 column
// quads; scales then zeros of the stage's group, 32 chunks of 8 columns each.
constexpr int kBChunks = (KS / 8) * (BN / 4);
constexpr int kSzChunks = 64;
constexpr int a_chunks(int bm) { return bm * 8; }
constexpr int slot_chunks(int bm) { return a_chunks(bm) + kBChunks + kSzChunks; }
// loads per wavefront and stage: activations (BM / 32), weights (4), scales/zeros (1)
constexpr int dma_per_stage(int bm) { return bm / 32 + 4 + 1; }

// Wait until this wavefront has at most one later stage of loads (N) outstanding and every
// one of its LDS reads has completed, then barrier.
template <int N>
__device__ __forceinline__ void stage_barrier_one_later() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}
__device__ __forceinline__ void reads_done_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// Physical chunk of activation chunk `ch` (0..7) of tile row `row` (XOR swizzle: the lanes
// that read one chunk of 16 consecutive rows hit different 16-byte bank groups).
__device__ __forceinline__ int a_slot(int row, int ch) { return row * 8 + (ch ^ ((row >> 1) & 7)); }

// 16 bytes per lane from global memory (wave-uniform base in SGPRs + a 32-bit per-lane byte
// offset) to LDS (wave-uniform LDS base in M0; the s_nop is the one wait state the M0 write
// needs before an LDS-DMA load). Per-lane offsets instead of 64-bit pointers keep the
// addresses of the 9 loads of a stage in 9 VGPRs.
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds_addr)
                 : "memory");
}
__device__ __forceinline__ void dma16_lanes(uint32_t voff, const void* sbase, uint32_t lds_addr, uint64_t lanes) {
    uint64_t saved;
    asm volatile("s_mov_b64 %0, exec\n\ts_mov_b64 exec, %4\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %2\n\ts_mov_b64 exec, %0"
                 : "=&s"(saved) : "v"(voff), "s"(sbase), "s"(lds_addr), "s"(lanes) : "memory");
}

// E4M3 codes of q - z for the 8 codes of word w, in natural K order (two dwords).
template <bool NAT>
__device__ __forceinline__ uint2 fp8_word(uint32_t w, const ZeroOffsets& zo, const UnpackConsts& c) {
    const half8_t d = unpack_sub(w, zo, c);   // linear: (q0,q4) (q1,q5) (q2,q6) (q3,q7); NAT: (q0,q1) .. (q6,q7)
    // Each conversion writes one half of its destination and keeps the other. The first of
    // each pair starts from its own (dying) source register, whose other half the second
    // conversion overwrites: no register has to be cleared first.
    const half2_t d01 = half2_t{d[0], d[1]}, d45 = half2_t{d[4], d[5]};
    short2v p0 = __builtin_bit_cast(short2v, d01), p1 = __builtin_bit_cast(short2v, d45);
    p0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(p0, d01, 1.0f, false);
    p0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(p0, half2_t{d[2], d[3]}, 1.0f, true);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(p1, d45, 1.0f, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(p1, half2_t{d[6], d[7]}, 1.0f, true);
    const uint32_t u0 = __builtin_bit_cast(uint32_t, p0), u1 = __builtin_bit_cast(uint32_t, p1);
    if constexpr (NAT) return make_uint2(u0, u1);
    // u0 = bytes (q0, q4, q1, q5), u1 = (q2, q6, q3, q7)
    return make_uint2(__builtin_amdgcn_perm(u1, u0, 0x06040200u),    // (q0, q1, q2, q3)
                      __builtin_amdgcn_perm(u1, u0, 0x07050301u));   // (q4, q5, q6, q7)
}

template <bool NAT, int BM>
__global__ __launch_bounds__(NT, 2) void w4a8_kernel(W4A8Params p) {
    static_assert(BM == 32 || BM == 64 || BM == 128, "work-group rows");
    constexpr int TI = BM / 16;                              // 16-row tiles per wavefront
    constexpr int NA = BM / 32;                              // activation loads per wavefront and stage
    constexpr int kAChunks = a_chunks(BM);
    constexpr int kChunks = slot_chunks(BM);
    extern __shared__ uint4 lds[];                           // NS slots of kChunks chunks
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int nw = n0 + wave * WNC + 4 * lr;                 // the lane's first output column
    // this work-group's stages: [kbase, kbase + KT) of the K / 128 stages (split-K), KT >= 1
    const int split = blockIdx.z;
    const int kbase = split * p.stages_per_split;
    const int KT = min(p.stages_per_split, p.K / KS - kbase);
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

    // per-lane byte offsets of the loads (a stage moves only the wave-uniform bases);
    // instruction i of a wavefront fills chunks (4 i + wave) * 64 + lane of its region
    uint32_t a_off[NA], b_off[4];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int c = (4 * i + wave) * 64 + lane;
        const int row = c >> 3, ch = (c & 7) ^ ((row >> 1) & 7);
        a_off[i] = (uint32_t)(min(m0 + row, p.M - 1) * p.K + ch * 16);       // rows >= M: never stored
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int col = n0 + 4 * lane;
        b_off[i] = (uint32_t)(((4 * i + wave) * p.N + (col < p.N ? col : 0)) * 4);   // columns >= N: never stored
    }
    // scales/zeros: lanes 0..15 of wavefront w load chunk 16 w + lane (scales for chunks
    // 0..31, i.e. wavefronts 0 and 1, zeros for 32..63), 8 columns each (N % 8 == 0)
    const int sz_col = n0 + ((wave * 16 + lane) & 31) * 8;
    const uint32_t sz_off = (uint32_t)((sz_col < p.N ? sz_col : 0) * 2);
    const uint16_t* sz_base = wave >= 2 ? p.zeros : p.scales;

    auto issue = [&](int kt, int slot) {
        const uint32_t sb = lds_base + (uint32_t)(slot * kChunks) * 16u;
        const uint8_t* xa = p.xq + (size_t)kt * KS;
        const uint32_t* wb = p.qweight + (size_t)kt * (KS / 8) * p.N;
#pragma unroll
        for (int i = 0; i < NA; ++i) dma16(a_off[i], xa, sb + (uint32_t)((4 * i + wave) * 64) * 16u);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(b_off[i], wb, sb + (uint32_t)(kAChunks + (4 * i + wave) * 64) * 16u);
        const size_t grp = (size_t)((kt * KS) >> p.group_shift);
        dma16_lanes(sz_off, sz_base + grp * p.N, sb + (uint32_t)(kAChunks + kBChunks + wave * 16) * 16u, 0xFFFFull);
    };

    const UnpackConsts uc = unpack_consts();
    floatx4 acc[TI][4];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    bool far_lane = false;   // a zero point of this lane's columns outside [-1, 16] so far

    auto compute = [&](const uint4* sl) {
        // the lane's four columns: scales and zero offsets of the group
        const uint4* szl = sl + kAChunks + kBChunks + wave * 8 + (lr >> 1);
        const uint2 sv = reinterpret_cast<const uint2*>(szl)[lr & 1];
        const uint2 zv = reinterpret_cast<const uint2*>(szl + 32)[lr & 1];
        const half2_t s01 = as_h2(sv.x), s23 = as_h2(sv.y), z01 = as_h2(zv.x), z23 = as_h2(zv.y);
        const float sc[4] = {(float)s01[0], (float)s01[1], (float)s23[0], (float)s23[1]};
        const _Float16 zc[4] = {z01[0], z01[1], z23[0], z23[1]};
        // B operands: byte 8r .. 8r + 7 of the lane's 32 come from packed row
        // (r < 2 ? 2 lg + r : 8 + 2 lg + r - 2) (K 16 lg + 8r .. resp. 64 + 16 lg + 8(r-2) ..)
        uint4 raw[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) raw[r] = sl[kAChunks + ((r < 2 ? 0 : 6) + 2 * lg + r) * 64 + wave * 16 + lr];
        int8v b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const _Float16 zt = (_Float16)fminf(fmaxf((float)zc[t], -1.0f), 16.0f);   // |q - zt| <= 16: exact
            far_lane = far_lane || zt != zc[t];
            const ZeroOffsets zo = zero_offsets(zt);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t w = t == 0 ? raw[r].x : t == 1 ? raw[r].y : t == 2 ? raw[r].z : raw[r].w;
                const uint2 q8 = fp8_word<NAT>(w, zo, uc);
                b[t][2 * r] = (int)q8.x;
                b[t][2 * r + 1] = (int)q8.y;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // row tile i: its activation fragment (read one tile ahead) and 4 MFMAs with a zero
        // accumulator; the group's scale of each column takes tile i's products into the fp32
        // result after tile i + 1's MFMAs are issued, so the FMAs never wait on a matrix
        // instruction that has just started
        auto read_a = [&](int i) {
            const int row = 16 * i + lr;
            const uint4 a0 = sl[a_slot(row, lg)], a1 = sl[a_slot(row, 4 + lg)];
            return int8v{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        };
        auto scale_into = [&](int i, const floatx4 (&g)[4]) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][t][e] = fmaf(sc[t], g[t][e], acc[i][t][e]);
        };
        int8v a = read_a(0);
        floatx4 gp[4];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            int8v a_next = a;
            if (i + 1 < TI) a_next = read_a(i + 1);
            floatx4 g[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                g[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[t], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0,
                                                                        0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (i > 0) scale_into(i - 1, gp);
#pragma unroll
            for (int t = 0; t < 4; ++t) gp[t] = g[t];
            a = a_next;
            __builtin_amdgcn_sched_barrier(0);
        }
        scale_into(TI - 1, gp);
    };

    // Two-slot ring: stage kt + 1 loads while stage kt is computed. Past the last stage the
    // ring is fed copies of it (never read), so every wait has the same count and the loop
    // body is one basic block (branches in it make the compiler split and spill).
    issue(kbase, 0);
    issue(kbase + min(1, KT - 1), 1);
    for (int kt = 0; kt < KT; ++kt) {
        stage_barrier_one_later<dma_per_stage(BM)>();       // stage kt has landed
        compute(lds + (kt & 1) * kChunks);
        reads_done_barrier();                               // every wavefront is done with this slot
        issue(kbase + min(kt + 2, KT - 1), kt & 1);
    }
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");       // no load may outlive the work-group

    // The remainder of the zero point beyond the clamp, for wavefronts that met one: the
    // products used q - zc, so row tile i takes -s (z - zc) S[b, m] for every block b of the
    // work-group's range (S: the activation block sums), just before it is stored. The lane
    // holds rows 4 lg + r of the tile and its four columns. One tile at a time, so that only
    // that tile's sums are carried through the loop over blocks.
    const bool far_wave = __builtin_amdgcn_ballot_w64(far_lane) != 0;
    auto correct_tile = [&](int i) __attribute__((always_inline)) {
        // lane indices re-derived here, so that nothing of this block is computed before
        // the main loop and held through it
        int elg = lg, enw = nw;
        asm volatile("" : "+v"(elg), "+v"(enw));
        const int col = enw < p.N ? enw : 0;                 // nw % 4 == 0 and N % 8 == 0
        // rows m0 + 16 i + 4 lg .. + 3; a quad at or past Ms (a multiple of 4, so past
        // every stored row) reads the block's last four entries instead
        const int row = min(m0 + 16 * i + 4 * elg, p.Ms - 4);
        for (int kt = kbase; kt < kbase + KT; ++kt) {
            const size_t grp = (size_t)((kt * KS) >> p.group_shift);
            const uint2 sv = *reinterpret_cast<const uint2*>(p.scales + grp * p.N + col);
            const uint2 zv = *reinterpret_cast<const uint2*>(p.zeros + grp * p.N + col);
            const float4 sa = *reinterpret_cast<const float4*>(p.xsum + (size_t)kt * p.Ms + row);
            const half2_t s01 = as_h2(sv.x), s23 = as_h2(sv.y), z01 = as_h2(zv.x), z23 = as_h2(zv.y);
            const float sf[4] = {(float)s01[0], (float)s01[1], (float)s23[0], (float)s23[1]};
            const float zf[4] = {(float)z01[0], (float)z01[1], (float)z23[0], (float)z23[1]};
            const float sr[4] = {sa.x, sa.y, sa.z, sa.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float c = -(sf[t] * (zf[t] - fminf(fmaxf(zf[t], -1.0f), 16.0f)));   // exact
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][t][r] = fmaf(sr[r], c, acc[i][t][r]);
            }
        }
    };

    // y rows 4 lg + r of row tile i, columns nw .. nw + 3, from fp32 sums v[t][r] times the
    // row scale
    auto store_rows = [&](int i, const floatx4 (&v)[4]) {
        if (nw >= p.N) return;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m0 + 16 * i + 4 * lg + r;
            if (row < p.M) {
                const float s = p.sx[row];
                const half2_t lo = half2_t{(_Float16)(v[0][r] * s), (_Float16)(v[1][r] * s)};
                const half2_t hi = half2_t{(_Float16)(v[2][r] * s), (_Float16)(v[3][r] * s)};
                *reinterpret_cast<uint2*>(p.y + (size_t)row * p.N + nw) = make_uint2(as_u32(lo), as_u32(hi));
            }
        }
    };
    const int live_tiles = min(TI, (p.M - m0 + 15) / 16);   // row tiles with a row < M

    if (p.splits > 1) {
        // Split-K, as on the async W4A16 tile: every work-group publishes its fp32 partial
        // with device-coherent (sc1) stores; the last of the tile's work-groups to arrive
        // sums all of them in split order (so the result does not depend on arrival order),
        // two row tiles at a time with four splits' loads in flight, and writes y.
        __shared__ uint32_t ticket_lds;
        const int tile = blockIdx.y * gridDim.x + blockIdx.x;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            p.ws + (size_t)tile * p.splits * kPrefillTileFloats, 0, p.splits * kPrefillTileFloats * 4, kRsrcRaw);
        // float4 (i, t) of this lane: partial offset ((wave * TI + i) * 4 + t) * 64 + lane;
        // offsets of splits >= p.splits lie past the buffer's end, where loads return 0
        auto off = [&](int s, int i, int t) {
            return (s * (kPrefillTileFloats / 4) + ((wave * TI + i) * 4 + t) * 64 + lane) * 16;
        };
#pragma unroll
        for (int i = 0; i < TI; ++i)
            if (i < live_tiles) {
                if (far_wave) correct_tile(i);
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint4_vec, acc[i][t]), rs, off(split, i, t), 0,
                                                           kCpolSc1);
            }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);              // this wavefront's partial stores have completed
        __syncthreads();                                       // ... and every wavefront's
        if (tid == 0)
            ticket_lds = __hip_atomic_fetch_add(&p.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (ticket_lds != (uint32_t)(p.splits - 1)) return;
        if (tid == 0)                                          // ready for the next call
            __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int i0 = 0; i0 < TI; i0 += 2) {
            if (i0 >= live_tiles) break;
            floatx4 sum[2][4];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int t = 0; t < 4; ++t) sum[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};
            for (int s0 = 0; s0 < p.splits; s0 += 4) {
                floatx4 v[4][2][4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            v[u][i][t] = __builtin_bit_cast(
                                floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs, off(s0 + u, i0 + i, t), 0, kCpolSc1));
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (s0 + u < p.splits)
#pragma unroll
                        for (int i = 0; i < 2; ++i)
#pragma unroll
                            for (int t = 0; t < 4; ++t) sum[i][t] += v[u][i][t];
            }
            store_rows(i0, sum[0]);
            store_rows(i0 + 1, sum[1]);
        }
        return;
    }

    // epilogue: lane holds rows 4 lg + r of columns nw .. nw + 3 of each row tile
#pragma unroll
    for (int i = 0; i < TI; ++i) {
        if (far_wave && i < live_tiles) correct_tile(i);
        store_rows(i, acc[i]);
    }
}

template <bool NAT, int BM>
int launch_w4a8_t(const W4A8Params& p, hipStream_t s) {
    const size_t lds = (size_t)NS * slot_chunks(BM) * 16;
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [&] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&w4a8_kernel<NAT, BM>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    });
    if (attr != hipSuccess) return (int)attr;
    const dim3 grid((unsigned)((p.N + BN - 1) / BN), (unsigned)((p.M + BM - 1) / BM), (unsigned)p.splits);
    hipLaunchKernelGGL((w4a8_kernel<NAT, BM>), grid, dim3(NT), lds, s, p);
    return (int)hipGetLastError();
}

}  // namespace

int launch_w4a8_quantize(const uint16_t* x, uint8_t* xq, float* sx, float* xsum, int M, int K, void* stream) {
    const int Ms = (M + 3) / 4 * 4;
    hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)M), dim3(QT), 0, reinterpret_cast<hipStream_t>(stream),
                       x, xq, sx, xsum, M, K, Ms);
    return (int)hipGetLastError();
}

int launch_w4a8(const W4A8Params& p, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p.N % 8 != 0 || p.K % KS != 0 || (p.group_shift != 7 && p.group_shift != 8) || p.splits < 1 || !p.xsum ||
        p.Ms < p.M || p.Ms % 4 != 0 ||
        p.stages_per_split < 1 || (p.splits > 1 && (!p.ws || !p.counters)) || (p.bm != 32 && p.bm != 64 && p.bm != 128))
        return (int)hipErrorInvalidValue;
    const bool nat = p.layout == W4A16_LAYOUT_INTERLEAVED;
    if (p.bm == 32) return nat ? launch_w4a8_t<true, 32>(p, s) : launch_w4a8_t<false, 32>(p, s);
    if (p.bm == 64) return nat ? launch_w4a8_t<true, 64>(p, s) : launch_w4a8_t<false, 64>(p, s);
    return nat ? launch_w4a8_t<true, 128>(p, s) : launch_w4a8_t<false, 128>(p, s);
}

}  // namespace w4a16
