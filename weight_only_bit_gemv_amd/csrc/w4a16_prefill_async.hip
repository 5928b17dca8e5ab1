// Prefill-sized W4A16 kernel for gfx950, tile W4A16_TILE_ASYNC: every operand reaches LDS
// through direct global-to-LDS loads into a ring of LDS stages.
//
// What it computes: y = x . dequant(Wq) ("Beating FP16 with 4-bit Weights: A Portable W4A16
// GEMM in Triton", section "The design": each packed int32 is loaded once, its eight
// nibbles are dequantised with the group's scale and zero, and the products accumulate in
// fp32 on the matrix cores).
//
// Tiling as the register tile: a work-group computes BM x 256 of y (BM = 128; 64 or 32 rows
// when M is that small) with 4 wavefronts side by side along N, each owning all BM rows x
// 64 columns (BM/16 x 4 tiles of v_mfma_f32_16x16x32_f16, 128 fp32 accumulators per lane at
// BM = 128). What differs is how the
// operands arrive: global_load_lds_dwordx4 writes 16 bytes per lane straight into LDS
// (lane i of an instruction lands at the wavefront's LDS base + 16 i) without passing
// through registers, so the pipeline depth is bounded by LDS, not by the 256 VGPRs the
// accumulators already half fill. Each 64-row K stage of a work-group (activations
// BM x 64 fp16, packed weights 8 rows x 256 columns, scales and zeros of its groups) lands
// in one slot of a three-slot LDS ring (77-80 KB at BM = 128, room for two work-groups per
// compute unit). A six-slot ring (one work-group per compute unit, five stages in flight) measured
// no faster on any prefill shape: the loads are not what a lone work-group waits for.
//
// The activations land in LDS in their natural K order (a direct load cannot permute), so
// the weights are put into that order instead: the magic-number unpack yields the codes of
// a word in the order [0, 4, 1, 5, 2, 6, 3, 7], and four byte permutes per word reorder the
// dequantised halves to [0 .. 7].
//
// Schedule. A stage is two K-steps of 32 rows, each 32 MFMAs per wavefront. While the
// MFMAs of one K-step run, the operands of the next are prepared: its weights, scales and
// zeros are read from LDS and dequantised (about 70 VALU), and each activation fragment is
// re-read as soon as the four MFMAs that use it have issued. The next K-step may belong to
// the next stage, so the stage boundary falls between the two K-steps of a stage: after
// the first K-step's MFMAs every wavefront waits for the next stage's loads, a barrier
// makes them visible (and ends every read of the current slot), the current slot is
// refilled with the stage NS ahead, and the second K-step's MFMAs overlap the next stage's
// first operands. The matrix cores then see one unbroken stream of MFMAs per wavefront,
// which matters when a compute unit holds a single work-group and no other wavefront can
// fill the gaps.
//
// Synchronisation is explicit. The loads are issued from inline assembly, invisible to the
// compiler's wait-count pass (which otherwise waits for every outstanding load before each
// LDS read it cannot prove disjoint from them, draining the pipeline); every wavefront
// issues the same number of loads per stage (kDmaPerStage), so "s_waitcnt vmcnt(n)" with n
// the loads of the stages issued after the one awaited means "this wavefront's loads of
// that stage have landed", and the barrier that follows makes every wavefront's loads of
// it visible. No load the compiler issues itself is in flight in the loop (nothing else
// loads from global memory there), so its own wait counts are unaffected.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "w4a16_device.hpp"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {

constexpr int NT = 256;                // threads per work-group
constexpr int WNC = 64;                // columns per wavefront
constexpr int BN = 4 * WNC;            // columns per work-group
constexpr int NS = 3;                  // LDS ring slots
// A work-group computes BM rows (32, 64 or 128: the library takes the smallest that holds
// M) x 256 columns. LDS slot layout in 16-byte chunks: activations BM rows x 8 chunks (64
// fp16), swizzled; packed weights 8 rows x 64 column quads; scales and zeros.
constexpr int kBChunks = 8 * (BN / 4);
template <bool G32, int BM> struct Slot {
    static constexpr int kAChunks = BM * 8;
    static constexpr int kSzChunks = G32 ? 128 : 64;   // per group: 32 scale + 32 zero chunks
    static constexpr int kChunks = kAChunks + kBChunks + kSzChunks;
    static constexpr int kSzLanes = G32 ? 32 : 16;     // lanes per wavefront loading them
    // loads per wavefront and stage: activations (BM / 32), weights (2), scales/zeros (1)
    static constexpr int kDmaPerStage = BM / 32 + 2 + 1;
};
constexpr int kRsrcRaw = 0x00020000;     // buffer resource word 3 for raw (untyped) access on gfx9
constexpr int kCpolSc1 = 16;             // device-coherent (sc1) cache policy of a buffer access
// s_waitcnt immediate for vmcnt(0) with expcnt/lgkmcnt left at their maxima (gfx9 encoding)
constexpr int kWaitVmcnt0 = 0 | (0x7 << 4) | (0xf << 8);
typedef uint32_t uint4_vec __attribute__((ext_vector_type(4)));

// Wait until this wavefront has at most LATER stages of DMA loads each outstanding (the
// stages issued after the one awaited) and every one of its LDS reads has completed, then
// barrier.
template <int LATER, int DMA>
__device__ __forceinline__ void stage_barrier() {
    static_assert(LATER == 1 || LATER == 2, "the ring waits with one or two later stages in flight");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(LATER * DMA) : "memory");
}

// Physical chunk of activation chunk `ch` (0..7) of tile row `row`: the 16 lanes that read
// one chunk of 16 consecutive rows hit 16 different 16-byte bank groups.
__device__ __forceinline__ int a_slot(int row, int ch) { return row * 8 + (ch ^ ((row >> 1) & 7)); }

// 16 bytes per lane from global memory to LDS: source = wave-uniform base (scalar
// registers) + the lane's 32-bit byte offset, destination = the wave-uniform LDS base in M0
// (the one wait state between the M0 write and the LDS-DMA load is the s_nop). A stage moves
// only the scalar base, so the loop carries no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds_addr)
                 : "memory");
}

// The same for the lanes in `lanes` only. EXEC is switched inside the one asm statement,
// so the compiler sees straight-line code (a branch here would split the loop into blocks
// across which it moves the dequantisation away from the MFMAs it should overlap).
__device__ __forceinline__ void dma16_lanes(uint32_t voff, const void* sbase, uint32_t lds_addr, uint64_t lanes) {
    uint64_t saved;
    asm volatile("s_mov_b64 %0, exec\n\ts_mov_b64 exec, %4\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %2\n\ts_mov_b64 exec, %0"
                 : "=&s"(saved) : "v"(voff), "s"(sbase), "s"(lds_addr), "s"(lanes) : "memory");
}

// Half H of the fp16 (q - z) * s of one word, in natural K order: H = 0 dequantises the
// codes at K offsets 0, 1, 4, 5 of the fragment, H = 1 those at 2, 3, 6, 7 (the magic-number
// unpack of device.hpp, one pair of halves at a time). A word of the linear layout unpacks
// as the pairs (q0, q4) (q1, q5) (q2, q6) (q3, q7) and two byte permutes per half reorder
// them; one of the interleaved layout (NAT) unpacks in natural order already.
template <bool NAT, int H>
__device__ __forceinline__ void dequant_half(uint32_t w, const ZeroOffsets& zo, half2_t s2, const UnpackConsts& c,
                                             uint4& out) {
    const uint32_t v = H ? w >> 8 : w;
    const half2_t lo = (as_h2((v & c.mask_lo) | c.bias1024) - zo.lo) * s2;   // codes 2H, 2H + 4
    const half2_t hi = (as_h2((v & c.mask_hi) | c.bias64) - zo.hi) * s2;     // codes 2H + 1, 2H + 5
    if constexpr (NAT) {
        (H ? out.z : out.x) = as_u32(lo);
        (H ? out.w : out.y) = as_u32(hi);
    } else {
        (H ? out.y : out.x) = __builtin_amdgcn_perm(as_u32(hi), as_u32(lo), 0x05040100u);   // (q2H, q2H+1)
        (H ? out.w : out.z) = __builtin_amdgcn_perm(as_u32(hi), as_u32(lo), 0x07060302u);   // (q2H+4, q2H+5)
    }
}

// The packed weights, scales and zeros of one K-step of a lane's four columns, as read from
// LDS.
struct BRaw {
    uint2 s, z;
    uint4 w;
};

template <bool G32, bool NAT, int BM>
__global__ __launch_bounds__(NT, 2) void prefill_async_kernel(PrefillParams p) {
    static_assert(BM == 32 || BM == 64 || BM == 128, "work-group rows");
    typedef Slot<G32, BM> S;
    constexpr int TI = BM / 16;                              // 16-row MFMA tiles per wavefront
    constexpr int NA = BM / 32;                              // activation loads per wavefront and stage
    constexpr int kAChunks = S::kAChunks;
    extern __shared__ uint4 lds[];                           // NS slots of S::kChunks chunks
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int nw = n0 + wave * WNC + 4 * lr;                 // the lane's first output column
    // this work-group's stages: [kbase, kbase + KT) of the K / 64 stages (split-K), KT >= 1
    const int split = blockIdx.z;
    const int kbase = split * p.stages_per_split;
    const int KT = min(p.stages_per_split, p.K / 64 - kbase);
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

    // Per-lane byte offsets of the loads from the stage's wave-uniform bases (activations:
    // row m0 of x at the stage's first K; weights: its first packed row; scales/zeros: its
    // group's row). Instruction i of a wavefront fills chunks (4 i + wave) * 64 + lane of its
    // region. The dispatcher keeps BM K 2 and 32 N below 2^31.
    uint32_t a_off[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int c = (4 * i + wave) * 64 + lane;
        const int row = c >> 3, ch = (c & 7) ^ ((row >> 1) & 7);   // inverse of a_slot
        a_off[i] = (uint32_t)(((min(m0 + row, p.M - 1) - m0) * p.K + ch * 8) * 2);   // rows >= M: not stored
    }
    uint32_t b_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = (4 * i + wave) * 64 + lane;
        const int col = n0 + 4 * (c & 63);
        b_off[i] = (uint32_t)(((c >> 6) * p.N + (col < p.N ? col : 0)) * 4);   // columns >= N: not stored
    }
    // scales/zeros: lane < kSzLanes loads chunk wave * kSzLanes + lane = group * 64 +
    // (zeros ? 32 : 0) + 8-column chunk; N % 8 == 0, so a chunk never straddles the row end.
    // Group and array are uniform per wavefront.
    const int csz = wave * S::kSzLanes + lane;
    const int sz_group = (wave * S::kSzLanes) >> 6;
    const int sz_col = n0 + (csz & 31) * 8;
    const uint32_t sz_off = (uint32_t)((sz_col < p.N ? sz_col : 0) * 2);
    const uint16_t* sz_base = ((wave * S::kSzLanes) >> 5) & 1 ? p.zeros : p.scales;
    const uint16_t* x_base = p.x + (size_t)m0 * p.K;

    auto issue = [&](int kt, int slot) {
        const uint32_t sb = lds_base + (uint32_t)(slot * S::kChunks) * 16u;
        const uint16_t* xa = x_base + (size_t)kt * 64;
        const uint32_t* wb = p.qweight + (size_t)kt * 8 * p.N;
#pragma unroll
        for (int i = 0; i < NA; ++i) dma16(a_off[i], xa, sb + (uint32_t)((4 * i + wave) * 64) * 16u);
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16(b_off[i], wb, sb + (uint32_t)(kAChunks + (4 * i + wave) * 64) * 16u);
        const size_t grp = G32 ? (size_t)(2 * kt + sz_group) : (size_t)((kt * 64) >> p.group_shift);
        dma16_lanes(sz_off, sz_base + grp * p.N, sb + (uint32_t)(kAChunks + kBChunks + wave * S::kSzLanes) * 16u,
                    (uint64_t(1) << S::kSzLanes) - 1);
    };

    const UnpackConsts uc = unpack_consts();
    floatx4 acc[TI][4];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    // The B operands of one K-step: the 4 words of the lane's columns, dequantised to
    // natural K order with their group's scales and zeros.
    auto read_b = [&](const uint4* sl, int j) {
        const uint4* szl = sl + kAChunks + kBChunks + (G32 ? j * 64 : 0) + wave * 8 + (lr >> 1);
        BRaw r;
        r.s = reinterpret_cast<const uint2*>(szl)[lr & 1];
        r.z = reinterpret_cast<const uint2*>(szl + 32)[lr & 1];
        r.w = sl[kAChunks + (4 * j + lg) * 64 + wave * 16 + lr];
        return r;
    };
    auto dequant_word = [&](const BRaw& r, int t, uint4& b) {   // t: compile-time after unrolling
        const half2_t zp = as_h2(t < 2 ? r.z.x : r.z.y), sp = as_h2(t < 2 ? r.s.x : r.s.y);
        const _Float16 z = zp[t & 1], sc = sp[t & 1];
        const ZeroOffsets zo = zero_offsets(z);
        const uint32_t w = t == 0 ? r.w.x : t == 1 ? r.w.y : t == 2 ? r.w.z : r.w.w;
        dequant_half<NAT, 0>(w, zo, half2_t{sc, sc}, uc, b);
        dequant_half<NAT, 1>(w, zo, half2_t{sc, sc}, uc, b);
    };
    auto read_a = [&](const uint4* sl, int j, int i) {
        return __builtin_bit_cast(half8_t, sl[a_slot(16 * i + lr, 4 * j + lg)]);
    };
    // The 4 TI MFMAs of one K-step on (a, b), in TI chunks of 4 (one activation fragment
    // each). NEXT: the chunks also prepare the next K-step, K-step nj of slot nsl: its
    // weights, scales and zeros are read from LDS before the first chunk, their words
    // dequantised in chunks 1 to 4 (one each; chunk 0 covers the read latency; after the
    // last chunk when there are fewer), and fragment i is re-read into a[i] in chunk i,
    // after its four MFMAs. Scheduling barriers between the chunks
    // keep the compiler from gathering the VALU work in one place.
    auto kstep = [&](half8_t (&a)[TI], const uint4 (&b)[4], auto next, const uint4* nsl, int nj, uint4 (&nb)[4]) {
        constexpr bool NEXT = decltype(next)::value;
        BRaw r;
        if constexpr (NEXT) r = read_b(nsl, nj);
#pragma unroll
        for (int i = 0; i < TI; ++i) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], __builtin_bit_cast(half8_t, b[t]), acc[i][t], 0,
                                                                   0, 0);
            if constexpr (NEXT) {
                a[i] = read_a(nsl, nj, i);
                if (i >= 1 && i <= 4) dequant_word(r, i - 1, nb[i - 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // with fewer than 5 row tiles the chunks cover words 0 .. TI - 2; the rest follow
        if constexpr (NEXT) {
#pragma unroll
            for (int t = (TI - 1 < 4 ? TI - 1 : 4); t < 4; ++t) dequant_word(r, t, nb[t]);
        }
    };

    // Prologue: NS stages in flight, the first K-step's operands in registers. Past the
    // work-group's last stage the ring is fed copies of that stage (never read): every
    // wavefront then issues kDmaPerStage loads per stage, the waits have fixed counts and
    // the loop body is one basic block.
#pragma unroll
    for (int s = 0; s < NS; ++s) issue(kbase + min(s, KT - 1), s);
    stage_barrier<NS - 1, S::kDmaPerStage>();
    half8_t a[TI];
    uint4 b0[4], b1[4];
    {
        const BRaw r = read_b(lds, 0);
#pragma unroll
        for (int t = 0; t < 4; ++t) dequant_word(r, t, b0[t]);
    }
#pragma unroll
    for (int i = 0; i < TI; ++i) a[i] = read_a(lds, 0, i);

    int slot = 0;
    for (int kt = 0; kt + 1 < KT; ++kt) {
        kstep(a, b0, std::true_type{}, lds + slot * S::kChunks, 1, b1);   // K-step 0; prepares K-step 1
        // stage kt + 1 has landed and every wavefront is done with this slot, which takes
        // stage kt + NS
        stage_barrier<NS - 2, S::kDmaPerStage>();
        issue(kbase + min(kt + NS, KT - 1), slot);
        slot = slot + 1 == NS ? 0 : slot + 1;
        kstep(a, b1, std::true_type{}, lds + slot * S::kChunks, 0, b0);   // K-step 1; prepares the next stage's K-step 0
    }
    kstep(a, b0, std::true_type{}, lds + slot * S::kChunks, 1, b1);       // the last stage
    kstep(a, b1, std::false_type{}, lds, 0, b0);
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");       // no load may outlive the work-group

    // y rows 4*lg + r of row tile i, columns nw .. nw + 3, from fp32 values v[t][r]
    auto store_rows = [&](int i, const floatx4 (&v)[4]) {
        if (nw >= p.N) return;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m0 + 16 * i + 4 * lg + r;
            if (row < p.M) {
                const half2_t lo = half2_t{(_Float16)v[0][r], (_Float16)v[1][r]};
                const half2_t hi = half2_t{(_Float16)v[2][r], (_Float16)v[3][r]};
                *reinterpret_cast<uint2*>(p.y + (size_t)row * p.N + nw) = make_uint2(as_u32(lo), as_u32(hi));
            }
        }
    };
    // row tiles with at least one row < M (the rest of the tile is never stored)
    const int live_tiles = min(TI, (p.M - m0 + 15) / 16);

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
        // float4 (i, t) of this lane: partial offset ((wave * TI + i) * 4 + t) * 64 + lane;
        // offsets of splits >= p.splits lie past the buffer's end, where loads return 0
        auto off = [&](int s, int i, int t) {
            return (s * (kPrefillTileFloats / 4) + ((wave * TI + i) * 4 + t) * 64 + lane) * 16;
        };
#pragma unroll
        for (int i = 0; i < TI; ++i)
            if (i < live_tiles)
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
        if (tid == 0)                                          // ready for the next call
            __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // Sum in split order, two row tiles at a time, the loads of four splits in flight
        // together (the partials reach this compute unit only as fast as enough of them are
        // outstanding); each pair of row tiles is stored as soon as it is summed.
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

    // epilogue: lane holds rows 4*lg + r of columns nw + t (t = 0..3) of each row tile
#pragma unroll
    for (int i = 0; i < TI; ++i) store_rows(i, acc[i]);
}

template <bool G32, bool NAT, int BM>
int launch_async(const PrefillParams& p, hipStream_t s) {
    const size_t lds = (size_t)NS * Slot<G32, BM>::kChunks * 16;
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [&] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_async_kernel<G32, NAT, BM>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    });
    if (attr != hipSuccess) return (int)attr;
    const dim3 grid((unsigned)((p.N + BN - 1) / BN), (unsigned)((p.M + BM - 1) / BM), (unsigned)p.splits);
    hipLaunchKernelGGL((prefill_async_kernel<G32, NAT, BM>), grid, dim3(NT), lds, s, p);
    return (int)hipGetLastError();
}

}  // namespace

int launch_prefill_async(const PrefillParams& p, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p.N % 8 != 0 || p.splits < 1 || p.stages_per_split < 1 || (p.splits > 1 && (!p.ws || !p.counters)) ||
        (p.bm != 32 && p.bm != 64 && p.bm != 128) || (int64_t)32 * p.N > INT32_MAX ||
        (int64_t)p.bm * p.K * 2 > INT32_MAX)
        return (int)hipErrorInvalidValue;
    const bool g32 = p.group_shift == 5, nat = p.layout == W4A16_LAYOUT_INTERLEAVED;
#define W4A16_ASYNC_BM(BM_)                                                                       \
    if (p.bm == BM_) {                                                                            \
        if (g32) return nat ? launch_async<true, true, BM_>(p, s) : launch_async<true, false, BM_>(p, s); \
        return nat ? launch_async<false, true, BM_>(p, s) : launch_async<false, false, BM_>(p, s);       \
    }
    W4A16_ASYNC_BM(32)
    W4A16_ASYNC_BM(64)
    W4A16_ASYNC_BM(128)
#undef W4A16_ASYNC_BM
    return (int)hipErrorInvalidValue;
}

}  // namespace w4a16
