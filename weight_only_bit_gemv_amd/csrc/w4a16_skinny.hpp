// Decode / skinny-M W4A16 kernel for gfx950: a single pass over the packed weight stream.
//
// What it computes: y = x . dequant(Wq) ("Beating FP16 with 4-bit Weights: A Portable W4A16
// GEMM in Triton", section "The design"), with the split-K decode strategy of the same page
// (extra parallelism along K when M is small: sections "The design" and "Things I got
// wrong along the way") but with a deterministic fixed-order reduction instead of fp32
// atomics.
//
// Mapping (one work-group = W wavefronts = one strip of CW = 16*LW columns x one K range):
//  * lane l reads LW consecutive packed words per K-step: packed row 4*ks + l/16, columns
//    strip*CW + LW*(l%16) .. +LW-1. A wavefront's load is 4 rows x 64*LW contiguous bytes
//    (LW = 4: 16-byte loads, 256 bytes per row; LW = 1: 4-byte loads, 64 bytes per row);
//    every packed int32 of qweight is read exactly once per 16*MT-row block of M.
//  * each of the lane's LW words is the B operand of one v_mfma_f32_16x16x32_f16: a lane
//    of that MFMA holds 8 K values of one column, which is exactly one packed word. LW MFMA
//    tiles cover columns {LW*j + t}; their outputs land back on the lane that loaded the
//    column, so the lane's own scales apply.
//  * the words are unpacked to exact fp16 (q - zero) values; x (rows padded to 16) is the A
//    operand in the same K order; products accumulate in fp32 per 128-row group and the
//    group's fp32 partial is multiplied by the column's scale once:
//    sum_k x_k (q_k - z) s = s * sum_k x_k (q_k - z) over a group, which keeps every
//    product exact.
//  * the W wavefronts of a work-group stream consecutive K ranges and are summed in LDS in
//    wave order; with more than one work-group along K (splits > 1) each writes its fp32
//    partial to the workspace, and the last to arrive (arrival counter) sums the splits in
//    index order 0..splits-1 and writes y. Results are bitwise reproducible.
// Narrow strips (LW < 4) give more work-groups for the same N, so small-N shapes fill the
// 256 compute units without a cross-work-group reduction.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "w4a16_device.hpp"
#include "w4a16_internal.h"

namespace w4a16 {
namespace skinny {

// s_waitcnt immediate for vmcnt(0) with expcnt/lgkmcnt left at their maxima (gfx9 encoding).
constexpr int kWaitVmcnt0 = 0 | (0x7 << 4) | (0xf << 8);
// Buffer-instruction cache policy: sc1, the device-coherent level (another XCD's L2 may
// hold stale lines; sc1 loads miss the local L2 and sc1 stores write through it).
constexpr int kCpolSc1 = 16;
// Buffer resource word 3 for raw (untyped) buffer access on gfx9.
constexpr int kRsrcWord3 = 0x00020000;

typedef uint32_t uint4_vec_t __attribute__((ext_vector_type(4)));
typedef uint32_t uint2_vec_t __attribute__((ext_vector_type(2)));

// LW consecutive 32-bit words (weights) or fp16 halves (scales, zeros) of one lane.
template <int LW> struct Lanes;
template <> struct Lanes<1> { typedef uint32_t Words; typedef uint16_t Halves; };
template <> struct Lanes<2> { typedef uint2 Words; typedef uint32_t Halves; };
template <> struct Lanes<4> { typedef uint4 Words; typedef uint2 Halves; };

__device__ __forceinline__ uint32_t word_at(uint32_t v, int) { return v; }
__device__ __forceinline__ uint32_t word_at(uint2 v, int t) { return t == 0 ? v.x : v.y; }
__device__ __forceinline__ uint32_t word_at(uint4 v, int t) {
    return t == 0 ? v.x : t == 1 ? v.y : t == 2 ? v.z : v.w;
}
__device__ __forceinline__ _Float16 half_at(uint16_t v, int) { return __builtin_bit_cast(_Float16, v); }
__device__ __forceinline__ _Float16 half_at(uint32_t v, int t) {
    return __builtin_bit_cast(_Float16, (uint16_t)(t == 0 ? v : v >> 16));
}
__device__ __forceinline__ _Float16 half_at(uint2 v, int t) {
    return half_at(t < 2 ? v.x : v.y, t & 1);
}

// The weight, activation and scale/zero streams of one wavefront as buffer resources:
// the scalar base of the weights and activations sits at the wavefront's first K-step,
// every lane adds a fixed 32-bit byte offset, and the K-step (or group) offset is a scalar
// register, so the loop carries no 64-bit address arithmetic. A load beyond a resource's
// range returns 0 instead of faulting.
template <int MT>
struct Streams {
    __amdgpu_buffer_rsrc_t w, x, s, z;
    int w_lane;          // bytes: packed row lg, column nl
    int w_step;          // bytes per K-step: 4 packed rows of N words
    int x_lane[MT];      // bytes: activation row of each M tile, K offset 8 lg
    int sz_lane;         // bytes: column nl
    int sz_step;         // bytes per group row: N halves
    int gshift;          // log2(K-steps per group)
};

// Weights are read once per call: non-temporal loads (cache policy nt) keep them from
// displacing the activations and partial sums in the caches.
constexpr int kCpolNt = 2;

template <int LW>
__device__ __forceinline__ typename Lanes<LW>::Words load_words(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    if constexpr (LW == 4) return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCpolNt));
    else if constexpr (LW == 2) return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kCpolNt));
    else return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kCpolNt);
}

template <int LW>
__device__ __forceinline__ typename Lanes<LW>::Halves load_halves(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    if constexpr (LW == 4) return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
    else if constexpr (LW == 2) return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    else return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

// One segment: U consecutive K-steps (U * 32 rows) of one wavefront: U packed word groups
// per lane, the matching activations, and the scale/zero of every group the segment
// touches: SG = min(U, K-steps per group) K-steps of one group each, U / SG groups (a
// segment starts on a multiple of U, so it never straddles a group boundary).
// The loads only issue memory requests: nothing in load() reads the returned registers,
// so a wavefront can keep a prefetched segment in flight while it works on the current
// one (the activation permutation happens in accumulate(), at first use).
template <int MT, int LW, int U, int SG, bool NAT>
struct Segment {
    typedef typename Lanes<LW>::Words Words;
    typedef typename Lanes<LW>::Halves Halves;
    static_assert(U % SG == 0, "a segment holds whole groups or lies inside one");
    static constexpr int NG = U / SG;                    // groups per segment
    Words wv[U];
    uint4 xv[U][MT];
    Halves sv[NG], zv[NG];

    // j: K-step of the segment's start counted from the wavefront's first K-step (weights and
    // activations); ks: the same K-step counted from 0 (scale/zero group).
    __device__ __forceinline__ void load(const Streams<MT>& st, int ks, int j) {
        const int grp = ks >> st.gshift;
#pragma unroll
        for (int u = 0; u < U; ++u) wv[u] = load_words<LW>(st.w, st.w_lane, (j + u) * st.w_step);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            sv[g] = load_halves<LW>(st.s, st.sz_lane, (grp + g) * st.sz_step);
            zv[g] = load_halves<LW>(st.z, st.sz_lane, (grp + g) * st.sz_step);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                xv[u][mt] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          st.x, st.x_lane[mt], (j + u) * kKStep * 2, 0));
    }

    // acc += scale * sum over each group of x * (q - zero), per column, in fp32.
    __device__ __forceinline__ void accumulate(floatx4 (&acc)[MT][LW], const UnpackConsts& uc) const {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            ZeroOffsets zo[LW];
#pragma unroll
            for (int t = 0; t < LW; ++t) zo[t] = zero_offsets(half_at(zv[g], t));
            floatx4 part[MT][LW];
#pragma unroll
            for (int uu = 0; uu < SG; ++uu) {
                const int u = g * SG + uu;
                half8_t xa[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) xa[mt] = x_frag<NAT>(xv[u][mt]);
#pragma unroll
                for (int t = 0; t < LW; ++t) {
                    const half8_t b = unpack_sub(word_at(wv[u], t), zo[t], uc);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        part[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            xa[mt], b, uu == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : part[mt][t], 0, 0, 0);
                }
            }
#pragma unroll
            for (int t = 0; t < LW; ++t) {
                const float sc = (float)half_at(sv[g], t);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt][t] += sc * part[mt][t];
            }
        }
    }
};

// LW fp32 values of one lane (one output row, the lane's LW columns).
template <int LW> struct Row { float v[LW]; };

template <int LW>
__device__ __forceinline__ void lds_store(float* dst, const Row<LW>& r) {
    if constexpr (LW == 4) *reinterpret_cast<float4*>(dst) = make_float4(r.v[0], r.v[1], r.v[2], r.v[3]);
    else if constexpr (LW == 2) *reinterpret_cast<float2*>(dst) = make_float2(r.v[0], r.v[1]);
    else *dst = r.v[0];
}

template <int LW>
__device__ __forceinline__ void lds_add(Row<LW>& r, const float* src) {
    if constexpr (LW == 4) {
        const float4 o = *reinterpret_cast<const float4*>(src);
        r.v[0] += o.x; r.v[1] += o.y; r.v[2] += o.z; r.v[3] += o.w;
    } else if constexpr (LW == 2) {
        const float2 o = *reinterpret_cast<const float2*>(src);
        r.v[0] += o.x; r.v[1] += o.y;
    } else {
        r.v[0] += *src;
    }
}

// fp32 -> fp16 (RNE) for the lane's LW columns of one output row.
template <int LW>
__device__ __forceinline__ void store_y(uint16_t* dst, const Row<LW>& r) {
    if constexpr (LW == 4) {
        const half2_t a = half2_t{(_Float16)r.v[0], (_Float16)r.v[1]};
        const half2_t b = half2_t{(_Float16)r.v[2], (_Float16)r.v[3]};
        *reinterpret_cast<uint2*>(dst) = make_uint2(as_u32(a), as_u32(b));
    } else if constexpr (LW == 2) {
        *reinterpret_cast<uint32_t*>(dst) = as_u32(half2_t{(_Float16)r.v[0], (_Float16)r.v[1]});
    } else {
        *dst = f16_bits((_Float16)r.v[0]);
    }
}

// Device-coherent (sc1) store / load of a lane's LW partial sums through a buffer resource.
template <int LW>
__device__ __forceinline__ void partial_store(__amdgpu_buffer_rsrc_t rs, int byte_off, const Row<LW>& r) {
    if constexpr (LW == 4) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint4_vec_t, f4{r.v[0], r.v[1], r.v[2], r.v[3]}),
                                               rs, byte_off, 0, kCpolSc1);
    } else if constexpr (LW == 2) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uint2_vec_t, f2{r.v[0], r.v[1]}),
                                              rs, byte_off, 0, kCpolSc1);
    } else {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, r.v[0]), rs, byte_off, 0, kCpolSc1);
    }
}

// Takes the bits as a scalar: __builtin_bit_cast of a vector-element lvalue (o[t]) reads
// element 0 whatever t is.
__device__ __forceinline__ float f32_bits(uint32_t b) { return __builtin_bit_cast(float, b); }

template <int LW>
__device__ __forceinline__ void partial_add(Row<LW>& r, __amdgpu_buffer_rsrc_t rs, int byte_off) {
    if constexpr (LW == 4) {
        const uint4_vec_t o = __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, kCpolSc1);
        r.v[0] += f32_bits(o.x);
        r.v[1] += f32_bits(o.y);
        r.v[2] += f32_bits(o.z);
        r.v[3] += f32_bits(o.w);
    } else if constexpr (LW == 2) {
        const uint2_vec_t o = __builtin_amdgcn_raw_buffer_load_b64(rs, byte_off, 0, kCpolSc1);
        r.v[0] += f32_bits(o.x);
        r.v[1] += f32_bits(o.y);
    } else {
        r.v[0] += f32_bits(__builtin_amdgcn_raw_buffer_load_b32(rs, byte_off, 0, kCpolSc1));
    }
}

// MT: 16-row MFMA tiles of M per work-group. LW: packed words per lane per K-step (strip
// width 16*LW). U: K-steps per segment; the dispatcher keeps kc a multiple of U and, for
// U = 8, K a multiple of 256, so every segment is exactly U K-steps inside whole groups and
// the loop below needs no predicates. SG: min(U, K-steps per group). W: wavefronts per
// work-group. NAT: the weights are packed in the interleaved layout (no activation permute).
// GM: the launch kind (SkinnyArgs): 1 matrix, up to kSharedXMats sharing x, or up to
// kMaxGroupMats each with its own x.
// Dynamic LDS: (W - 1) * rows * CW floats, rows = min(16 * MT, M - row0).
template <int MT, int LW, int U, int SG, int W, bool NAT, int GM>
__global__ __launch_bounds__(64 * W) void skinny_kernel(SkinnyArgs<GM> p) {
    static_assert(U == 1 || U == 2 || U == 4 || U == 8, "segment of 1, 2, 4 or 8 K-steps");
    constexpr int CW = 16 * LW;
    extern __shared__ float red[];                  // [W - 1][rows][CW]
    const int lane = threadIdx.x & 63;
    // wave-uniform: keeps the K range and the segment loop in scalar registers and branches
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lg = lane >> 4;            // which of the 4 packed rows of a K-step
    const int lc = lane & 15;            // column slot within the strip / A-operand row
    // Work-group b runs on XCD b % 8 (round-robin dispatch), and each XCD has its own L2.
    // With 16-column strips two neighbouring strips share every 128-byte line, so within
    // each block of 16 work-groups the pair (b, b + 8), which lands on one XCD, takes two
    // neighbouring strips: the second read of each line hits that XCD's L2 instead of
    // fetching the line from HBM again. Wider strips own whole lines.
    int b = blockIdx.x;
    if (LW == 1 && b < ((p.n_strips * p.splits) & ~15)) b = (b & ~15) | ((b & 7) << 1) | ((b >> 3) & 1);
    const int strip = b % p.n_strips;
    const int split = b / p.n_strips;
    // The matrix this strip belongs to (wave-uniform), and its activations. A single-matrix
    // launch has one entry, read at constant offsets in the same batch as the other
    // arguments. A grouped launch reads the entries' first strips (one batch), picks the
    // entry, then reads that entry: one more scalar round trip, where selecting among fully
    // loaded entries compiled to a chain of dependent loads.
    SkinnyMatrix mat;
    const uint16_t* x;
    int mrows = p.M;                     // rows of this matrix's x and y
    if constexpr (GM == kSharedXMats) {
        int mi = 0;
#pragma unroll
        for (int j = 1; j < GM; ++j) {
            int s0 = p.mat[j].strip0;
            asm volatile("" : "+s"(s0));
            mi = (j < p.n_mats && strip >= s0) ? j : mi;
        }
        mat = p.mat[mi];
        x = p.x;
    } else if constexpr (GM == kMaxGroupMats) {
        // the starts increase with the entry, so the entry is the number of later entries
        // (below n_mats) whose start the strip has reached
        int mi = 0;
#pragma unroll
        for (int j = 1; j < GM; ++j) mi += (j < p.n_mats && strip >= p.strip0[j]) ? 1 : 0;
        mat = p.mat[mi];
        x = mat.x;
        mrows = p.rows[mi];
    } else {
        mat = p.mat[0];
        x = p.x;
    }
    const int N = mat.N;
    const int row0 = blockIdx.y * 16 * MT;
    const int rows = min(16 * MT, mrows - row0);        // valid output rows of this work-group
    // a matrix with fewer rows than the launch has none in this block: nothing to load or
    // store (every work-group of the block and strip returns here, so its split-K counter
    // is never taken)
    if (GM == kMaxGroupMats && rows <= 0) return;
    const int n = (strip - mat.strip0) * CW + lc * LW;
    const bool col_ok = n < N;
    const int nl = col_ok ? n : 0;       // loads stay in bounds; results of such lanes are dropped
    const int KS = p.K / kKStep;
    const int chunk = split * W + wave;
    const int k0 = min(chunk * p.kc, KS);
    const int k1 = min(k0 + p.kc, KS);
    // Resources: weights from packed row 4 k0 on (clamped to the 32-bit range; a wavefront's
    // own K range is far smaller), activations from row row0 on, scales/zeros whole. The
    // lane offsets stay below 2^31: the dispatcher keeps 16 N kc, 2 K rows and 2 N K/g in
    // range.
    Streams<MT> st;
    {
        const size_t w_rows = (size_t)(p.K / 8 - 4 * k0) * N * 4;
        st.w = __builtin_amdgcn_make_buffer_rsrc((void*)(mat.qweight + (size_t)4 * k0 * N), 0,
                                                 (int)min(w_rows, (size_t)0xffffffffu), kRsrcWord3);
        st.x = __builtin_amdgcn_make_buffer_rsrc((void*)(x + (size_t)row0 * p.K + (size_t)k0 * kKStep), 0,
                                                 (int)min(((size_t)(mrows - row0) * p.K - (size_t)k0 * kKStep) * 2, (size_t)0xffffffffu), kRsrcWord3);
        const int sz_bytes = (p.K >> (p.gshift + 5)) * N * 2;
        st.s = __builtin_amdgcn_make_buffer_rsrc((void*)mat.scales, 0, sz_bytes, kRsrcWord3);
        st.z = __builtin_amdgcn_make_buffer_rsrc((void*)mat.zeros, 0, sz_bytes, kRsrcWord3);
    }
    st.w_lane = (lg * N + nl) * 4;
    st.w_step = 16 * N;
    // A-operand rows beyond M only feed output rows beyond M, which are never stored, so
    // their loads are clamped to row M-1 instead of being predicated (a predicated load
    // would put a branch between a segment's loads and their use, and the compiler then
    // waits for every outstanding load at the branch's end).
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        st.x_lane[mt] = ((min(row0 + mt * 16 + lc, mrows - 1) - row0) * p.K + lg * 8) * 2;
    st.sz_lane = nl * 2;
    st.sz_step = N * 2;
    st.gshift = p.gshift;
    const UnpackConsts uc = unpack_consts();

    floatx4 acc[MT][LW];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < LW; ++t) acc[mt][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Software pipeline over the nseg segments, unrolled twice so that the two buffers
    // alternate roles without register copies: the loads of segment i+1 are issued before
    // segment i is unpacked and multiplied, so every wavefront keeps two segments in flight.
    // The steady-state loop issues its loads unconditionally (a conditional load would end
    // in a wait for all outstanding loads); the last one or two segments are peeled.
    // sched_barrier(0) after each load keeps the instruction scheduler from sinking the
    // prefetch below the arithmetic of the previous segment (it otherwise does so to save
    // registers, which leaves one segment in flight and drains the queue between segments).
    Segment<MT, LW, U, SG, NAT> sa, sb;
    const int nseg = (k1 - k0) / U;
    if (nseg > 0) sa.load(st, k0, 0);
    __builtin_amdgcn_sched_barrier(0);
    int i = 0;
    for (; i + 2 < nseg; i += 2) {
        sb.load(st, k0 + (i + 1) * U, (i + 1) * U);
        __builtin_amdgcn_sched_barrier(0);
        sa.accumulate(acc, uc);
        sa.load(st, k0 + (i + 2) * U, (i + 2) * U);
        __builtin_amdgcn_sched_barrier(0);
        sb.accumulate(acc, uc);
    }
    if (i + 1 < nseg) {
        sb.load(st, k0 + (i + 1) * U, (i + 1) * U);
        __builtin_amdgcn_sched_barrier(0);
        sa.accumulate(acc, uc);
        sb.accumulate(acc, uc);
    } else if (i < nseg) {
        sa.accumulate(acc, uc);
    }

    // The MFMA D layout: lane holds rows 4*lg + r (r = 0..3) of column slot lc of each tile.
    auto row_of = [&](int mt, int r) {
        Row<LW> o;
#pragma unroll
        for (int t = 0; t < LW; ++t) o.v[t] = acc[mt][t][r];
        return o;
    };

    // ---- sum the W wavefronts of the work-group in wave order (LDS) ----
    if (W > 1) {
        if (wave > 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rl = mt * 16 + lg * 4 + r;
                    if (rl < rows) lds_store<LW>(&red[((wave - 1) * rows + rl) * CW + lc * LW], row_of(mt, r));
                }
        }
        __syncthreads();
        if (wave != 0) return;
    }

    Row<LW> out[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rl = mt * 16 + lg * 4 + r;
            out[mt][r] = row_of(mt, r);
            if (rl < rows) {
                for (int w = 0; w < W - 1; ++w) lds_add<LW>(out[mt][r], &red[(w * rows + rl) * CW + lc * LW]);
            }
        }

    if (p.splits == 1) {
        if (!col_ok) return;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rl = mt * 16 + lg * 4 + r;
                if (rl < rows) store_y<LW>(mat.y + (size_t)(row0 + rl) * N + n, out[mt][r]);
            }
        return;
    }

    // ---- split-K: publish this work-group's partial, the last arrival reduces ----
    // On gfx950 an agent-scope fence writes back and invalidates the whole L2, which costs
    // far more than this kernel's work when every work-group issues one. The partials are
    // therefore written and read with sc1 (device-coherent) buffer accesses, which bypass
    // stale cache lines, and ordering needs only a wait for this wavefront's memory
    // operations: partial stores complete before the arrival counter is incremented, and
    // the last arrival reads the partials only after its increment returns.
    const size_t counter = (size_t)blockIdx.y * p.n_strips + strip;
    constexpr int slab = 16 * MT * CW;                                    // floats per partial
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        p.ws + counter * p.splits * slab, 0, p.splits * slab * 4, kRsrcWord3);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rl = mt * 16 + lg * 4 + r;
            if (rl < rows) partial_store<LW>(rs, (split * slab + rl * CW + lc * LW) * 4, out[mt][r]);
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

    // The partials of kBatch splits x 4 rows are loaded together, then summed in split
    // order 0..splits-1 (fixed, so the result does not depend on arrival order). Loads of a
    // split index >= splits lie beyond the buffer resource's range and return 0, so the
    // batch needs no predicate; rows >= M are read (inside the slab) but never stored.
    if (col_ok) {
        constexpr int kBatch = 4;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            Row<LW> v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int t = 0; t < LW; ++t) v[r].v[t] = 0.f;
            for (int s0 = 0; s0 < p.splits; s0 += kBatch) {
                Row<LW> part[kBatch][4];
#pragma unroll
                for (int s = 0; s < kBatch; ++s)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
#pragma unroll
                        for (int t = 0; t < LW; ++t) part[s][r].v[t] = 0.f;
                        partial_add<LW>(part[s][r], rs, ((s0 + s) * slab + (mt * 16 + lg * 4 + r) * CW + lc * LW) * 4);
                    }
#pragma unroll
                for (int s = 0; s < kBatch; ++s)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int t = 0; t < LW; ++t) v[r].v[t] += part[s][r].v[t];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rl = mt * 16 + lg * 4 + r;
                if (rl < rows) store_y<LW>(mat.y + (size_t)(row0 + rl) * N + n, v[r]);
            }
        }
    }
    if (lane == 0)                                     // ready for the next call
        __hip_atomic_store(&p.counters[counter], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MT, int LW, int U, int SG, int W>
hipError_t launch_one(const SkinnyParams& p, hipStream_t s) {
    const dim3 grid((unsigned)(p.n_strips * p.splits), (unsigned)p.row_blocks);
    const int rows = std::min(16 * MT, p.M);
    const size_t lds = (size_t)(W - 1) * rows * 16 * LW * sizeof(float);
    const bool nat = p.layout == W4A16_LAYOUT_INTERLEAVED;
    // the launch kind: one matrix; up to kSharedXMats sharing the header's x (and M); or the
    // table with each matrix's own x and row count
    bool shared_x = p.n_mats <= kSharedXMats;
    for (int i = 0; i < p.n_mats; ++i) shared_x = shared_x && p.mat[i].x == p.x && p.rows[i] == p.M;
    if (p.n_mats == 1 && shared_x) {
        SkinnyArgs<1> a;
        static_cast<SkinnyHeader&>(a) = p;
        a.mat[0] = p.mat[0];
        if (nat) hipLaunchKernelGGL((skinny_kernel<MT, LW, U, SG, W, true, 1>), grid, dim3(64 * W), lds, s, a);
        else hipLaunchKernelGGL((skinny_kernel<MT, LW, U, SG, W, false, 1>), grid, dim3(64 * W), lds, s, a);
    } else if (shared_x) {
        SkinnyArgs<kSharedXMats> a;
        static_cast<SkinnyHeader&>(a) = p;
        for (int i = 0; i < kSharedXMats; ++i) a.mat[i] = p.mat[i];
        if (nat) hipLaunchKernelGGL((skinny_kernel<MT, LW, U, SG, W, true, kSharedXMats>), grid, dim3(64 * W), lds, s, a);
        else hipLaunchKernelGGL((skinny_kernel<MT, LW, U, SG, W, false, kSharedXMats>), grid, dim3(64 * W), lds, s, a);
    } else {
        if (nat) hipLaunchKernelGGL((skinny_kernel<MT, LW, U, SG, W, true, kMaxGroupMats>), grid, dim3(64 * W), lds, s, p);
        else hipLaunchKernelGGL((skinny_kernel<MT, LW, U, SG, W, false, kMaxGroupMats>), grid, dim3(64 * W), lds, s, p);
    }
    return hipGetLastError();
}

}  // namespace skinny
}  // namespace w4a16
