// Prefill-sized W4A16 kernel for gfx950, tile W4A16_TILE_ASYNC: every operand reaches LDS
// through direct global-to-LDS loads, three stages in flight.
//
// What it computes: y = x . dequant(Wq) ("Beating FP16 with 4-bit Weights: A Portable W4A16
// GEMM in Triton", section "The design": each packed int32 is loaded once, its eight
// nibbles are dequantised with the group's scale and zero, and the products accumulate in
// fp32 on the matrix cores).
//
// Tiling as the register tile: a work-group computes 128 x 256 of y with 4 wavefronts side
// by side along N, each owning all 128 rows x 64 columns (8 x 4 tiles of
// v_mfma_f32_16x16x32_f16, 128 fp32 accumulators per lane), two work-groups per compute
// unit. What differs is how the operands arrive: global_load_lds_dwordx4 writes 16 bytes
// per lane straight into LDS (lane i of an instruction lands at the wavefront's LDS base +
// 16 i) without passing through registers, so the pipeline depth is bounded by LDS, not by
// the 256 VGPRs the accumulators already half fill. Each 64-row K stage of a work-group
// (activations 128 x 64 fp16, packed weights 8 rows x 256 columns, scales and zeros of
// its groups) lands in one of three LDS slots; the loads of stage k + 2 are issued while
// stage k is multiplied.
//
// The activations land in LDS in their natural K order (a direct load cannot permute), so
// the weights are put into that order instead: the magic-number unpack yields the codes of
// a word in the order [0, 4, 1, 5, 2, 6, 3, 7], and four byte permutes per word reorder the
// dequantised halves to [0 .. 7].
//
// Synchronisation is explicit. The loads are issued from inline assembly, invisible to the
// compiler's wait-count pass (which otherwise waits for every outstanding load before each
// LDS read it cannot prove disjoint from them, draining the pipeline); every wavefront
// issues the same number of loads per stage (kDmaPerStage), so "s_waitcnt vmcnt(n)" with n
// the loads of one later stage means "this wavefront's loads of the current stage have
// landed", and the barrier that follows makes every wavefront's loads of it visible. The
// barrier also orders the reads of the slot about to be refilled before the loads that
// refill it. No load the compiler issues itself is in flight in the loop (nothing else
// loads from global memory there), so its own wait counts are unaffected.
#include <hip/hip_runtime.h>

#include <mutex>

#include "w4a16_device.hpp"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {

constexpr int NT = 256;                // threads per work-group
constexpr int BM = 128;                // rows of M per work-group
constexpr int WNC = 64;                // columns per wavefront
constexpr int BN = 4 * WNC;            // columns per work-group
constexpr int TI = BM / 16;            // 16-row MFMA tiles per wavefront
constexpr int NS = 3;                  // LDS slots (stages in flight)
// LDS slot layout in 16-byte chunks
constexpr int kAChunks = BM * 8;       // activations: 128 rows x 8 chunks (64 fp16), swizzled
constexpr int kBChunks = 8 * (BN / 4); // packed weights: 8 rows x 64 column quads
template <bool G32> struct Slot {
    static constexpr int kSzChunks = G32 ? 128 : 64;   // per group: 32 scale + 32 zero chunks
    static constexpr int kChunks = kAChunks + kBChunks + kSzChunks;
    static constexpr int kSzLanes = G32 ? 32 : 16;     // lanes per wavefront loading them
};
constexpr int kDmaPerStage = 4 + 2 + 1;  // per wavefront: activations, weights, scales/zeros
constexpr int kRsrcRaw = 0x00020000;     // buffer resource word 3 for raw (untyped) access on gfx9
constexpr int kCpolSc1 = 16;             // device-coherent (sc1) cache policy of a buffer access
// s_waitcnt immediate for vmcnt(0) with expcnt/lgkmcnt left at their maxima (gfx9 encoding)
constexpr int kWaitVmcnt0 = 0 | (0x7 << 4) | (0xf << 8);
typedef uint32_t uint4_vec __attribute__((ext_vector_type(4)));
static_assert(kDmaPerStage == 7, "the wait below counts 7 loads per stage");

// Physical chunk of activation chunk `ch` (0..7) of tile row `row`: the 16 lanes that read
// one chunk of 16 consecutive rows hit 16 different 16-byte bank groups.
__device__ __forceinline__ int a_slot(int row, int ch) { return row * 8 + (ch ^ ((row >> 1) & 7)); }

// 16 bytes per lane from global memory to LDS (wave-uniform LDS base in M0).
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "s"(lds_addr) : "memory");
}

// fp16 (q - z) * s of one word in natural K order. A word of the linear layout unpacks in
// the order [0, 4, 1, 5, 2, 6, 3, 7] and is reordered; one of the interleaved layout (NAT)
// unpacks in natural order already.
template <bool NAT>
__device__ __forceinline__ half8_t dequant_natural(uint32_t w, ZeroOffsets zo, _Float16 s, const UnpackConsts& uc) {
    if constexpr (NAT) return dequant_frag(w, zo, s, uc);
    const uint4 u = __builtin_bit_cast(uint4, dequant_frag(w, zo, s, uc));   // (q0,q4) (q1,q5) (q2,q6) (q3,q7)
    const uint4 n = make_uint4(__builtin_amdgcn_perm(u.y, u.x, 0x05040100u),  // (q0, q1)
                               __builtin_amdgcn_perm(u.w, u.z, 0x05040100u),  // (q2, q3)
                               __builtin_amdgcn_perm(u.y, u.x, 0x07060302u),  // (q4, q5)
                               __builtin_amdgcn_perm(u.w, u.z, 0x07060302u)); // (q6, q7)
    return __builtin_bit_cast(half8_t, n);
}

template <bool G32, bool NAT>
__global__ __launch_bounds__(NT, 2) void prefill_async_kernel(PrefillParams p) {
    typedef Slot<G32> S;
    extern __shared__ uint4 lds[];                           // NS slots of S::kChunks chunks
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int nw = n0 + wave * WNC + 4 * lr;                 // the lane's first output column
    // this work-group's stages: [kbase, kbase + KT) of the K / 64 stages (split-K), KT >= 2
    const int split = blockIdx.z;
    const int kbase = split * p.stages_per_split;
    const int KT = min(p.stages_per_split, p.K / 64 - kbase);
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

    // Per-lane sources of stage 0; stage kt adds a uniform offset. Instruction i of a
    // wavefront fills chunks (4 i + wave) * 64 + lane of its region.
    const uint16_t* a_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = (4 * i + wave) * 64 + lane;
        const int row = c >> 3, ch = (c & 7) ^ ((row >> 1) & 7);   // inverse of a_slot
        a_src[i] = p.x + (size_t)min(m0 + row, p.M - 1) * p.K + ch * 8;   // rows >= M: not stored
    }
    const uint32_t* b_src[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = (4 * i + wave) * 64 + lane;
        const int col = n0 + 4 * (c & 63);
        b_src[i] = p.qweight + (size_t)(c >> 6) * p.N + (col < p.N ? col : 0);   // columns >= N: not stored
    }
    // scales/zeros: lane < kSzLanes loads chunk wave * kSzLanes + lane = group * 64 +
    // (zeros ? 32 : 0) + 8-column chunk; N % 8 == 0, so a chunk never straddles the row end
    const int csz = wave * S::kSzLanes + lane;
    const int sz_group = csz >> 6;                           // uniform per wavefront
    const int sz_col = n0 + (csz & 31) * 8;
    const uint16_t* sz_src = ((csz >> 5) & 1 ? p.zeros : p.scales) + (sz_col < p.N ? sz_col : 0);

    auto issue = [&](int kt, int slot) {
        const uint32_t sb = lds_base + (uint32_t)(slot * S::kChunks) * 16u;
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(a_src[i] + (size_t)kt * 64, sb + (uint32_t)((4 * i + wave) * 64) * 16u);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            dma16(b_src[i] + (size_t)kt * 8 * p.N, sb + (uint32_t)(kAChunks + (4 * i + wave) * 64) * 16u);
        const size_t grp = G32 ? (size_t)(2 * kt + sz_group) : (size_t)((kt * 64) >> p.group_shift);
        if (lane < S::kSzLanes)
            dma16(sz_src + grp * p.N, sb + (uint32_t)(kAChunks + kBChunks + wave * S::kSzLanes) * 16u);
    };

    const UnpackConsts uc = unpack_consts();
    floatx4 acc[TI][4];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    // The B operands of one K-step: 4 words of the lane's columns, dequantised to natural
    // K order with their group's scales and zeros.
    auto load_b = [&](const uint4* sl, int j, half8_t (&b)[4]) {
        const uint4* szl = sl + kAChunks + kBChunks + (G32 ? j * 64 : 0) + wave * 8 + (lr >> 1);
        const uint2 sv = reinterpret_cast<const uint2*>(szl)[lr & 1];
        const uint2 zv = reinterpret_cast<const uint2*>(szl + 32)[lr & 1];
        const uint4 bw = sl[kAChunks + (4 * j + lg) * 64 + wave * 16 + lr];
        const half2_t z01 = as_h2(zv.x), z23 = as_h2(zv.y);
        const half2_t s01 = as_h2(sv.x), s23 = as_h2(sv.y);
        b[0] = dequant_natural<NAT>(bw.x, zero_offsets(z01[0]), s01[0], uc);
        b[1] = dequant_natural<NAT>(bw.y, zero_offsets(z01[1]), s01[1], uc);
        b[2] = dequant_natural<NAT>(bw.z, zero_offsets(z23[0]), s23[0], uc);
        b[3] = dequant_natural<NAT>(bw.w, zero_offsets(z23[1]), s23[1], uc);
    };
    auto read_a = [&](const uint4* sl, int j, half8_t (&a)[TI]) {
#pragma unroll
        for (int i = 0; i < TI; ++i) a[i] = __builtin_bit_cast(half8_t, sl[a_slot(16 * i + lr, 4 * j + lg)]);
    };
    auto mfma_step = [&](const half8_t (&a)[TI], const half8_t (&b)[4]) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[t], acc[i][t], 0, 0, 0);
    };
    // Per K-step all eight activation fragments are read first (the MFMAs then consume them
    // as they arrive). Within a stage the dequantisation of K-step 1 (its LDS reads and
    // about 70 VALU) runs between the 32 MFMAs of K-step 0: one MFMA, then two VALU,
    // repeated, so the matrix core does not wait for the unpack; K-step 0's dequantisation
    // comes first, alone.
    auto compute = [&](int slot) {
        const uint4* sl = lds + slot * S::kChunks;
        half8_t a[TI], b0[4], b1[4];
        load_b(sl, 0, b0);
        read_a(sl, 0, a);
        __builtin_amdgcn_sched_barrier(0);
        load_b(sl, 1, b1);
        mfma_step(a, b0);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // K-step 1's weight, scale, zero reads
#pragma unroll
        for (int i = 0; i < 4 * TI; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // 3 VALU
        }
        __builtin_amdgcn_sched_barrier(0);
        read_a(sl, 1, a);
        mfma_step(a, b1);
        __builtin_amdgcn_sched_group_barrier(0x100, TI, 0);  // all activation reads first
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * TI, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    issue(kbase, 0);
    issue(kbase + 1, 1);
    for (int kt = 0; kt < KT; ++kt) {
        // this wavefront's loads of stage kt have landed (those of stage kt + 1 may not);
        // after the barrier every wavefront's have, and every wavefront is done with the
        // slot of stage kt - 1, which the next issue refills
        asm volatile("s_waitcnt vmcnt(7) lgkmcnt(0)\n\ts_barrier" : : : "memory");
        issue(kbase + min(kt + 2, KT - 1), (kt + 2) % NS);   // past the end: a redundant copy
        compute(kt % NS);
    }
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");       // no load may outlive the work-group

    if (p.splits > 1) {
        // Split-K: publish this work-group's fp32 partial; the last of the tile's work-groups
        // to arrive sums all of them in split order (fixed, so the result does not depend
        // on arrival order) and writes y. As in the decode kernel, partials are written and
        // read with device-coherent (sc1) accesses and ordering needs only waits on this
        // wavefront's memory operations plus a work-group barrier before the ticket.
        __shared__ uint32_t ticket_lds;
        const int tile = blockIdx.y * gridDim.x + blockIdx.x;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            p.ws + (size_t)tile * p.splits * kPrefillTileFloats, 0, p.splits * kPrefillTileFloats * 4, kRsrcRaw);
        // float4 (i, t) of this lane: partial offset ((wave * TI + i) * 4 + t) * 64 + lane
        auto off = [&](int s, int i, int t) {
            return (s * (kPrefillTileFloats / 4) + ((wave * TI + i) * 4 + t) * 64 + lane) * 16;
        };
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint4_vec, acc[i][t]), rs, off(split, i, t), 0,
                                                       kCpolSc1);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);              // this wavefront's partial stores have completed
        __syncthreads();                                       // ... and every wavefront's
        if (tid == 0)
            ticket_lds = __hip_atomic_fetch_add(&p.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (ticket_lds != (uint32_t)(p.splits - 1)) return;
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        // sum in split order, half the row tiles at a time (register budget)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = 4 * h; i < 4 * h + 4; ++i)
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < p.splits; ++s) {
                floatx4 v[4][4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        v[i][t] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs, off(s, 4 * h + i, t), 0, kCpolSc1));
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int t = 0; t < 4; ++t) acc[4 * h + i][t] += v[i][t];
            }
        }
        if (tid == 0)                                          // ready for the next call
            __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // epilogue: lane holds rows 4*lg + r of columns nw + t (t = 0..3) of each row tile
    if (nw >= p.N) return;
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

template <bool G32, bool NAT>
int launch_async(const PrefillParams& p, hipStream_t s) {
    const size_t lds = (size_t)NS * Slot<G32>::kChunks * 16;
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [&] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_async_kernel<G32, NAT>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    });
    if (attr != hipSuccess) return (int)attr;
    const dim3 grid((unsigned)((p.N + BN - 1) / BN), (unsigned)((p.M + BM - 1) / BM), (unsigned)p.splits);
    hipLaunchKernelGGL((prefill_async_kernel<G32, NAT>), grid, dim3(NT), lds, s, p);
    return (int)hipGetLastError();
}

}  // namespace

int launch_prefill_async(const PrefillParams& p, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p.N % 8 != 0 || p.splits < 1 || p.stages_per_split < 2 || (p.splits > 1 && (!p.ws || !p.counters)))
        return (int)hipErrorInvalidValue;
    const bool g32 = p.group_shift == 5, nat = p.layout == W4A16_LAYOUT_INTERLEAVED;
    if (g32) return nat ? launch_async<true, true>(p, s) : launch_async<true, false>(p, s);
    return nat ? launch_async<false, true>(p, s) : launch_async<false, false>(p, s);
}

}  // namespace w4a16
