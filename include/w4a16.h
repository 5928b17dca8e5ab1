/*
 * w4a16.h - C ABI of the MI355X (gfx950) W4A16 weight-only GEMM/GEMV library.
 *
 *   y[M, N] = x[M, K] . dequant(Wq)[K, N],   dequant(q) = (q - zero) * scale
 *
 * The operation is the one described on "Beating FP16 with 4-bit Weights: A Portable
 * W4A16 GEMM in Triton", section "The design": fp16 activations, 4-bit weights with one
 * scale and one zero-point per group of 128 rows of the contraction dimension, eight
 * 4-bit values packed into one int32 along that dimension (packed row i, nibble j holds
 * K index 8*i + j), dequantised inside the product, fp32 accumulation.  The GemLite README
 * ("Packing") states the same (W_q - zeros) * scales convention, and its settings take
 * other group sizes: the library accepts groups of 32, 64, 128 and 256 rows.
 *
 * Layouts (all row-major, contiguous, no padding):
 *   W        fp32  [K, N]        host; input x output (y = x . W)
 *   qweight  int32 [K/8, N]      nibble j of word [i, n] (bits 4j..4j+3) is code q[8i+j, n]
 *   scales   fp16  [K/g, N]      one per (K-group, column), g = group_size
 *   zeros    fp16  [K/g, N]      integer-valued fp16 zero points, |zero| <= 1024
 *   x        fp16  [M, K]
 *   y        fp16  [M, N]        fully overwritten (never accumulated into)
 * fp16 values cross the ABI as their 16-bit patterns (uint16_t / void*).
 *
 * Ownership: every buffer is the caller's. The library never frees or keeps a pointer to
 * a caller buffer after a call returns. It owns one split-K workspace (fp32 partial sums
 * and arrival counters) per (device, stream) pair, allocated on first use and grown when a
 * larger one is needed; two calls on one stream are ordered by the stream, so they never
 * share it concurrently. A workspace that grows keeps its earlier buffers allocated until
 * the process ends, so a graph captured on the stream before the growth stays valid.
 *
 * Errors: every entry point returns W4A16_OK (0) or a negative W4A16_ERR_* code and never
 * throws. Arguments are validated before any HIP call is made; a call rejected by
 * validation changes no output. w4a16_strerror() names a code; w4a16_last_error_detail() gives the message of
 * the last failure on the calling thread.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_OK                 0
#define W4A16_ERR_INVALID_ARG   -1  /* null pointer, non-positive size, bad enum value   */
#define W4A16_ERR_UNSUPPORTED   -2  /* valid but not built: group size, K or N multiple  */
#define W4A16_ERR_ALIGNMENT     -3  /* a device pointer is not 16-byte aligned           */
#define W4A16_ERR_NONFINITE     -4  /* NaN/Inf in W, or a scale that overflows fp16      */
#define W4A16_ERR_HIP           -5  /* a HIP runtime call or kernel launch failed        */

/* Kernel selection for w4a16_matmul_ex / w4a16_plan. */
#define W4A16_KERNEL_AUTO     0   /* shape-based dispatcher (what w4a16_matmul uses)        */
#define W4A16_KERNEL_SKINNY   1   /* decode: weight stream, split-K, M <= 64 per row block  */
#define W4A16_KERNEL_PREFILL  2   /* prefill: fp16 dequant tiles feeding MFMA (tile below)  */

/* Packed-weight layouts: which K offset of its 8 K indices nibble p (bits 4p..4p+3) of a
 * packed word holds. Codes, scales and zeros are the same in both; only the packing differs.
 * LINEAR: offset p ("The design": packed row i, nibble j holds K index 8i + j).
 * INTERLEAVED: offset (0, 2, 4, 6, 1, 3, 5, 7)[p] - even offsets in the low nibbles, odd
 * in the high ones: the order in which the kernels' fp16 unpack yields consecutive K
 * values, so neither operand is permuted (weights pre-permuted offline, as "Beating FP16
 * with 4-bit Weights", section "What's next", proposes). */
#define W4A16_LAYOUT_LINEAR       0
#define W4A16_LAYOUT_INTERLEAVED  1

/* Prefill tile configurations (w4a16_plan_t.tile; 0 = the dispatcher's choice). */
#define W4A16_TILE_LDS         1  /* 128 x 128 output tile, weights and activations in LDS  */
#define W4A16_TILE_REGISTER_B  2  /* 128 x 256 output tile, weights dequantised in registers,*/
                                  /* activations in LDS (fewer LDS bytes per MFMA)          */
#define W4A16_TILE_ASYNC       3  /* 128 x 256 output tile (64 or 32 rows when M is that     */
                                  /* small), all operands loaded straight into a 3-stage    */
                                  /* LDS ring (needs N % 8 == 0)                            */

/*
 * Execution plan of one w4a16_matmul call (what the dispatcher chose, or what a caller
 * forces through w4a16_matmul_ex). Fields a caller sets to 0 are chosen by the library.
 *   kernel     W4A16_KERNEL_*.
 *   kc         SKINNY: K-steps of 32 rows that one wavefront streams: 1, 2 or a multiple
 *              of 4 (a multiple of seg). The kernel addresses a wavefront's weights with
 *              32-bit byte offsets: 16 * N * (kc + 1) must stay below 2^31, else
 *              UNSUPPORTED (also when 32 * row_tiles * K or 2 * N * K / group_size
 *              reaches 2^31).
 *   splits     SKINNY: work-groups along K per column strip (output: derived from kc and
 *              waves; a caller may leave it 0 or give the matching value).
 *              PREFILL with W4A16_TILE_ASYNC: work-groups along K per output tile, each over
 *              an even number of 64-row stages (0: about 256 work-groups with >= 16 stages
 *              each, or for M <= 64, whose work-groups hold 32 or 64 rows, about 512 with
 *              >= 12 stages each and a power of two; 1 when the tiles alone reach that);
 *              at most K/128; the completed plan holds the count actually used. Other
 *              tiles: 0 or 1 (output 1).
 *   row_tiles  SKINNY: 16-row MFMA tiles per work-group (1..4; default ceil(M/16) <= 4;
 *              at most 2 when cols < 64).
 *   tile       PREFILL: W4A16_TILE_LDS, W4A16_TILE_REGISTER_B or W4A16_TILE_ASYNC (0: ASYNC
 *              when N % 8 == 0, else REGISTER_B when the 128 x 256 output tiles number
 *              >= 384, else LDS). W4A16_TILE_ASYNC with N % 8 != 0 is UNSUPPORTED.
 *   waves      SKINNY: wavefronts per work-group, 4, 8 or 16 (the cross-wave reduction
 *              must fit in 64 KiB of LDS: (waves-1) * 16*row_tiles * cols * 4 bytes).
 *   cols       SKINNY: output columns per work-group strip, 16, 32 or 64 (each lane loads
 *              cols/16 consecutive packed words of a row: 4, 8 or 16 bytes).
 *   seg        SKINNY: K-steps one wavefront loads ahead as a unit, 1, 2, 4 or 8 (8 needs
 *              K % 256 == 0 and kc % 8 == 0); default from kc.
 */
typedef struct w4a16_plan {
    int32_t kernel;
    int32_t kc;
    int32_t splits;
    int32_t row_tiles;
    int32_t tile;
    int32_t waves;
    int32_t cols;
    int32_t seg;
} w4a16_plan_t;

/*
 * w4a16_pack - quantise and pack a weight matrix on the host (CPU only, synchronous).
 *
 * Follows "The design" (one scale and zero per 128-row K-group per column, eight codes per
 * int32 along K) with the asymmetric min/max quantiser, per (group, column):
 *   scale = fp16_rne((max - min) / 15)          (1.0 if that rounds to 0)
 *   zero  = rne(-min / scale)                   (stored as fp16; not clamped)
 *   q     = clamp(rne(w / scale) + zero, 0, 15) (rne = round half to even)
 * every step an IEEE fp32 operation (true division, no fused multiply-add).
 * Deterministic and independent of the number of threads used.
 *
 *   W          host fp32 [K, N]
 *   K, N       K >= group_size, K % group_size == 0; N >= 1
 *   group_size 32, 64, 128 or 256
 *   qweight    host int32 [K/8, N]     (written)
 *   scales     host fp16 bits [K/g, N] (written)
 *   zeros      host fp16 bits [K/g, N] (written)
 * Errors: INVALID_ARG (null, K or N <= 0), UNSUPPORTED (group size, K % g, |zero| > 1024),
 * NONFINITE (NaN/Inf in W, scale overflow). Argument errors and NaN/Inf in W are found
 * before anything is written; after a scale overflow or an out-of-domain zero point
 * (found while packing) the contents of qweight / scales / zeros are unspecified.
 * Same as w4a16_pack_ex(W, K, N, group_size, 0, qweight, scales, zeros).
 */
int w4a16_pack(const float* W, int64_t K, int64_t N, int64_t group_size,
               int32_t* qweight, uint16_t* scales, uint16_t* zeros);

/*
 * w4a16_pack_ex - w4a16_pack with a choice of quantiser.
 *   symmetric  0: the asymmetric min/max quantiser of w4a16_pack;
 *              1: the symmetric one with the +8 zero point of "Triton Kernel Matches
 *                 bitsandbytes: Why Both Lose to Math", section "Three Kernel Versions and
 *                 Two Bugs", per (group, column):
 *                   scale = fp16_rne(max|w| / 7)           (1.0 if that rounds to 0)
 *                   zero  = 8
 *                   q     = clamp(rne(w / scale) + 8, 0, 15)
 *                 with the same fp32 steps. The output layout is unchanged (zeros holds 8),
 *                 so w4a16_matmul runs both kinds of weights.
 *   group_size 32, 64, 128 or 256.
 *   layout     W4A16_LAYOUT_LINEAR or W4A16_LAYOUT_INTERLEAVED (packing of qweight).
 * Other arguments, errors and ownership as w4a16_pack; INVALID_ARG when symmetric is not
 * 0 or 1 or layout is not a W4A16_LAYOUT_* value.
 */
int w4a16_pack_ex(const float* W, int64_t K, int64_t N, int64_t group_size, int symmetric,
                  int layout, int32_t* qweight, uint16_t* scales, uint16_t* zeros);

/*
 * w4a16_unpack - host inverse of the packing that "Beating FP16 with 4-bit Weights", section
 * "The design", defines (eight codes per int32 along K, packed row i / nibble j holding K
 * index 8i + j): codes[8i + j, n] = (qweight[i, n] >> 4j) & 15.
 *   qweight host int32 [K/8, N]; codes host uint8 [K, N] (written). K % 8 == 0.
 * Errors: INVALID_ARG.
 */
int w4a16_unpack(const int32_t* qweight, int64_t K, int64_t N, uint8_t* codes);

/* w4a16_unpack_ex - w4a16_unpack for either layout (codes in natural K order): the linear
 * packing of "The design", or the interleaved one that section "What's next" of the same page
 * motivates (weights pre-permuted offline into the order the matrix instruction consumes).
 * Errors: INVALID_ARG (also for an unknown layout). */
int w4a16_unpack_ex(const int32_t* qweight, int64_t K, int64_t N, int layout, uint8_t* codes);

/*
 * w4a16_matmul - y = x . dequant(qweight, scales, zeros) on the GPU ("The design": the
 * weights cross HBM packed and are dequantised in registers inside the product; fp32
 * accumulation; y rounded to fp16 once at the end).
 *
 *   x, qweight, scales, zeros, y   device pointers (layouts above), 16-byte aligned
 *   M >= 1, N >= 4 with N % 4 == 0, K >= 128 with K % 128 == 0 and K % group_size == 0
 *   group_size 32, 64, 128 or 256
 *   stream     hipStream_t as void* (NULL = the null stream)
 * Asynchronous: returns once the kernel is enqueued on `stream`. y is fully overwritten.
 * The result is deterministic: the same call gives the same bits (split-K partial sums are
 * combined in a fixed order; no floating-point atomics).
 * Graph capture: a plan with splits > 1 uses the library's split-K workspace for `stream`;
 * if it is not yet large enough it is allocated (hipMalloc) on the call. Under stream
 * capture that allocation is not possible, and the call returns HIP without enqueueing
 * anything (the capture itself stays usable): make one call of the shape on the stream
 * before capturing. The captured kernels use that stream's workspace: replay the graph on
 * the capturing stream, or at least never concurrently with other calls on it.
 * Errors: INVALID_ARG, UNSUPPORTED, ALIGNMENT (no HIP call made), HIP (launch failure,
 * workspace allocation failure, or a workspace that would have to grow during capture).
 */
int w4a16_matmul(const void* x, const int32_t* qweight, const void* scales,
                 const void* zeros, void* y, int64_t M, int64_t N, int64_t K,
                 int64_t group_size, void* stream);

/*
 * w4a16_matmul_ex - w4a16_matmul with the plan forced by the caller (tuning and tests). The
 * product is the one of "The design"; the plan is what "Things I got wrong along the way" on
 * the same page says must be tuned per shape (block sizes and the split-K factor, whose best
 * value differed between attention and FFN projections).
 * plan->kernel == W4A16_KERNEL_AUTO behaves as w4a16_matmul. Fields left 0 are filled by
 * the dispatcher. Errors as w4a16_matmul, plus INVALID_ARG for an unusable plan.
 */
int w4a16_matmul_ex(const void* x, const int32_t* qweight, const void* scales,
                    const void* zeros, void* y, int64_t M, int64_t N, int64_t K,
                    int64_t group_size, void* stream, const w4a16_plan_t* plan);

/*
 * w4a16_matmul_fmt - the general entry point: w4a16_matmul_ex for weights packed in either
 * layout (w4a16_matmul and w4a16_matmul_ex are this call with W4A16_LAYOUT_LINEAR). The
 * product is that of "Beating FP16 with 4-bit Weights", section "The design"; the interleaved
 * layout is the offline pre-permutation its section "What's next" proposes.
 *   layout  W4A16_LAYOUT_LINEAR or W4A16_LAYOUT_INTERLEAVED, as given to w4a16_pack_ex
 *   plan    NULL or a plan as for w4a16_matmul_ex
 * Errors as w4a16_matmul_ex, plus INVALID_ARG for an unknown layout.
 */
int w4a16_matmul_fmt(const void* x, const int32_t* qweight, const void* scales,
                     const void* zeros, void* y, int64_t M, int64_t N, int64_t K,
                     int64_t group_size, int layout, void* stream, const w4a16_plan_t* plan);

/*
 * w4a16_matrix_t - one weight matrix of a grouped product (w4a16_matmul_grouped): device
 * pointers in the layouts above, N its output columns (N >= 4, N % 4 == 0), the activations
 * it multiplies (x NULL for the call's x, or its own fp16 [M_i, K], 16-byte aligned) and
 * their row count M_i (0 for the call's M; otherwise 1..M): the experts of a
 * mixture-of-experts layer, whose down projections each read their own input, and which at
 * a batch of several tokens each see their own number of tokens.
 */
typedef struct w4a16_matrix {
    const int32_t* qweight;   /* int32 [K/8, N] */
    const void* scales;       /* fp16 [K/g, N]  */
    const void* zeros;        /* fp16 [K/g, N]  */
    void* y;                  /* fp16 [M_i, N], fully overwritten */
    int64_t N;
    const void* x;            /* fp16 [M_i, K], or NULL: the call's x (its first M_i rows) */
    int64_t M;                /* M_i, or 0: the call's M */
} w4a16_matrix_t;

/*
 * w4a16_matmul_grouped - y_i = x_i . dequant(W_i) for 1..16 weight matrices with the same
 * K, group size and layout and M_i <= M rows each, in one launch of the decode kernel: the projections that read
 * one input, such as the query, key and value projections of an attention layer or the gate
 * and up projections of an FFN or of the active experts of a mixture-of-experts layer (x_i
 * = x), and the experts' down projections (each its own x_i). "Beating FP16 with 4-bit
 * Weights", section "Takeaways", calls decode a parallelism problem, and "Triton Kernel
 * Matches bitsandbytes: Why Both Lose to Math", section "Limitations and Next Steps", names
 * launch overhead among the costs of a decode step: one launch over the matrices' combined
 * columns pays the per-launch cost once and gives the chip more work-groups.
 *   x        device fp16 [M, K], 16-byte aligned: the activations of every matrix whose x is
 *            NULL (non-NULL even when every matrix has its own); M the largest M_i (the
 *            plan is made for it)
 *   mats     host array of n_mats w4a16_matrix_t (read during the call only)
 *   n_mats   1..16
 *   plan     NULL or a forced plan. The plan is chosen (or completed) for M, the summed N and
 *            K; when it selects the decode kernel (W4A16_KERNEL_SKINNY) one launch covers
 *            every matrix with that plan, and each y_i is bitwise equal to
 *            w4a16_matmul_fmt(x_i, W_i, M_i, ...) under the same plan. When it selects the prefill
 *            kernel, each matrix is launched on its own (with the forced plan, or with the
 *            dispatcher's plan for its shape), as the prefill tiles fill the chip per matrix.
 * Asynchronous on `stream`; split-K uses the stream's workspace as w4a16_matmul does.
 * Errors: INVALID_ARG (null pointers, n_mats, layout, plan, M_i outside 0..M), UNSUPPORTED (a matrix's shape,
 * or the summed N, outside what w4a16_matmul accepts), ALIGNMENT, HIP; all found before any
 * launch except HIP errors of a later matrix when the prefill kernel is launched per matrix.
 */
int w4a16_matmul_grouped(const void* x, const w4a16_matrix_t* mats, int n_mats, int64_t M, int64_t K,
                         int64_t group_size, int layout, void* stream, const w4a16_plan_t* plan);

/*
 * w4a16_matmul_noalloc - w4a16_matmul_fmt that allocates nothing, for callers that cannot
 * call hipMalloc: code under HIP graph capture, tight serving loops, harnesses that forbid
 * device allocation. Same arguments, plans, kernels and results as w4a16_matmul_fmt; a plan
 * with split-K keeps its fp32 partials and arrival counters in a static scratch array of the
 * library (one per device, held until the process ends: 64 MiB of partials and 65536
 * counters) instead of the per-stream workspace. No hipMalloc, hipFree or other allocating
 * call is made. The first call on a device takes the array's device address and clears its
 * counters with a kernel on `stream`; every kernel returns the counters it takes to zero.
 * Every call on one device shares that device's array: calls that overlap in time on one
 * device (on different streams, or graphs replayed concurrently) race and give undefined
 * results; calls ordered on one stream do not.
 * Errors as w4a16_matmul_fmt, plus UNSUPPORTED (before any HIP call) when the plan needs
 * more partials or counters than the scratch holds: force fewer splits (plan->splits for the
 * async prefill tile, larger kc or more waves for the decode kernel).
 */
int w4a16_matmul_noalloc(const void* x, const int32_t* qweight, const void* scales,
                         const void* zeros, void* y, int64_t M, int64_t N, int64_t K,
                         int64_t group_size, int layout, void* stream, const w4a16_plan_t* plan);

/*
 * w4a16_plan - the plan w4a16_matmul would use for (M, N, K, group_size), or the completed
 * version of a forced plan when `plan->kernel` is non-zero on entry. Host only; no HIP call.
 * The dispatcher takes, in this order: a plan set for the shape by w4a16_autotune or
 * w4a16_set_plan; the library's table of plans measured on MI355X for common decoder
 * projection shapes (per bucket of M); otherwise a rule fitted to those measurements.
 * The choice is per shape, from measurements, as "Beating FP16 with 4-bit Weights", section
 * "Things I got wrong along the way", asks (autotune per shape; the best split factor is not
 * the same for every projection), and as "Triton Kernel Matches bitsandbytes: Why Both Lose to
 * Math", section "Three Kernel Versions and Two Bugs", bears out (split-K lost on some shapes).
 * Errors: INVALID_ARG, UNSUPPORTED.
 */
int w4a16_plan(int64_t M, int64_t N, int64_t K, int64_t group_size, w4a16_plan_t* plan);

/*
 * w4a16_autotune - measure the plans of one shape on the device and keep the fastest for
 * later calls: the per-shape tuning, with the winner cached, that "Beating FP16 with 4-bit
 * Weights", section "Things I got wrong along the way", asks for (the best block sizes and
 * split factor differ between projections of one model).
 *   x, qweight, scales, zeros, y, M, N, K, group_size, layout  as for w4a16_matmul_fmt
 *   stream   the caller's stream: the call first waits for the work enqueued on it
 *   best     NULL, or receives the chosen plan (complete)
 *   seconds  NULL, or receives its measured time per call
 * The candidates are the dispatcher's plan, every built decode-kernel plan (M <= 128) and
 * the prefill tiles with each split count (M >= 17). Each is timed on a stream of the
 * library's own as a HIP graph of calls that rotate over copies of the weights (512 MiB in
 * all, 2 to 512 copies: allocated by the call and freed before it returns), so that every
 * call reads its weights from HBM; the five fastest are timed again and the fastest is kept,
 * the dispatcher's own plan unless another is more than 1 % faster. From then on, in this
 * process, calls of that (M, N, K, group_size) that leave the plan to the dispatcher take it:
 * w4a16_matmul, w4a16_matmul_ex/_fmt/_noalloc with a NULL or all-zero plan,
 * w4a16_matmul_grouped (for its summed N) and w4a16_plan. (w4a16_matmul_noalloc returns
 * UNSUPPORTED if the plan's split-K needs more than its static scratch.)
 * Synchronous; allocates device memory; not allowed while `stream` is being captured. On
 * return y holds the product, computed with the chosen plan.
 * Errors: INVALID_ARG, UNSUPPORTED, ALIGNMENT (all before any HIP call), HIP.
 */
int w4a16_autotune(const void* x, const int32_t* qweight, const void* scales, const void* zeros, void* y,
                   int64_t M, int64_t N, int64_t K, int64_t group_size, int layout, void* stream,
                   w4a16_plan_t* best, double* seconds);

/*
 * w4a16_set_plan - make `plan` the plan of (M, N, K, group_size) for later calls that leave
 * the plan to the dispatcher, as w4a16_autotune does with the plan it measures: for instance
 * to restore, at start-up, plans that an earlier process measured. The plan is completed and
 * validated as w4a16_plan does with a forced plan. NULL removes the shape's entry. Host only;
 * no HIP call. Errors: INVALID_ARG (a plan that names no kernel, or one not usable for the
 * shape), UNSUPPORTED.
 */
int w4a16_set_plan(int64_t M, int64_t N, int64_t K, int64_t group_size, const w4a16_plan_t* plan);

/* w4a16_clear_plans - forget every plan set by w4a16_autotune or w4a16_set_plan. Host only. */
int w4a16_clear_plans(void);

/*
 * w4a16_dequant - the GPU's unpack/dequant, exposed for bit-exact checks: the unpack and the
 * (q - zero) * scale dequantisation of "Beating FP16 with 4-bit Weights", section "The
 * design", that the product kernels perform in registers.
 *   codes  device uint8 [K, N] or NULL, 4-byte aligned: codes[8i + j, n] = nibble j of
 *          qweight[i, n]
 *   w      device fp16 [K, N] or NULL: fp16_rne((q - zero) * scale), i.e. one rounding of
 *          the exact product (the fp16 weight the prefill kernel stages in LDS)
 *   qweight, scales, zeros as for w4a16_matmul; N % 4 == 0, K % 128 == 0,
 *   K % group_size == 0, group_size 32, 64, 128 or 256; at least one of codes / w non-NULL.
 * Asynchronous on `stream`. Errors: INVALID_ARG, UNSUPPORTED, ALIGNMENT, HIP.
 */
int w4a16_dequant(const int32_t* qweight, const void* scales, const void* zeros,
                  uint8_t* codes, void* w, int64_t N, int64_t K, int64_t group_size,
                  void* stream);

/* w4a16_dequant_fmt - w4a16_dequant for weights packed in either layout ("The design" and
 * the pre-permuted layout of "What's next" on the same page); codes and w are in natural K
 * order whatever the layout. Errors as w4a16_dequant, plus INVALID_ARG for an unknown
 * layout. */
int w4a16_dequant_fmt(const int32_t* qweight, const void* scales, const void* zeros,
                      uint8_t* codes, void* w, int64_t N, int64_t K, int64_t group_size,
                      int layout, void* stream);

/*
 * W4A8: 8-bit floating-point activations x the 4-bit weights above ("Beating FP16 with
 * 4-bit Weights", section "What's next": FP8 activations for a W4A8 variant; GemLite README:
 * FP8 x Wn, activations quantised dynamically with one scale per row). E4M3 is the OCP
 * 8-bit format: bias 7, subnormals, largest finite value 448, no infinities. Only the
 * activations are 8-bit: the weights keep the exact (q - zero) * scale of "The design".
 *
 * w4a8_quantize_activations - per-row dynamic quantisation of x on the device:
 *   sx[m]    = amax_k |x[m, k]| / 448 (fp32 division; 1.0 for an all-zero row)
 *   xq[m, k] = E4M3(x[m, k] / sx[m])   (fp32 division, round to nearest even, saturating
 *                                       at +-448)
 *   xsum[b * Ms + m] = sum of dec(xq[m, k]) over the 128 k of block b (fp32; Ms = M rounded
 *                      up to a multiple of 4; entries m >= M are written 0): the per-row
 *                      sums the product needs for its zero points
 *   x   device fp16 [M, K], 16-byte aligned;  xq device uint8 [M, K], 16-byte aligned;
 *   sx  device fp32 [M], 4-byte aligned;  xsum device fp32 [K/128, Ms], 16-byte aligned;
 *   K % 128 == 0.
 * Asynchronous on `stream`. NaN/Inf in x give unspecified codes. Errors: INVALID_ARG (null,
 * M or K < 1), UNSUPPORTED (K % 128, size), ALIGNMENT, HIP (launch failure).
 */
int w4a8_quantize_activations(const void* x, uint8_t* xq, float* sx, float* xsum, int64_t M, int64_t K,
                              void* stream);

/*
 * w4a8_matmul - y[m, n] = sx[m] * sum_g s[g, n] * sum_{k in group g} dec(xq[m, k]) *
 * (q[k, n] - z[g, n]), q - z exact whatever the zero point, fp32 accumulation on the 8-bit
 * matrix cores, fp16 output (round to nearest even), y fully overwritten. The 8-bit weight
 * operand is q - zc with zc = z clamped to [-1, 16] (|q - zc| <= 16: exact in E4M3); a zero
 * point outside that range adds its remainder -(z - zc) s[g, n] xsum per 128-row block in
 * fp32 after the matrix products (so a far zero point costs extra work only in the
 * wavefronts whose columns hold one).
 *   xq, sx, xsum  as written by w4a8_quantize_activations (or any E4M3 codes, fp32 scales and
 *              the matching block sums, same layout)
 *   qweight, scales, zeros, layout   the W4A16 weight format (w4a16_pack / w4a16_pack_ex)
 *   group_size 128 or 256 (one 8-bit matrix instruction spans 128 rows of K, and a group's
 *              scale must not change inside it)
 *   N % 8 == 0, K % 128 == 0; device pointers 16-byte aligned (sx 4-byte).
 * Asynchronous on `stream`; deterministic (split-K partial sums are combined in a fixed
 * order). When the output tiles underfill the chip the K range is split over several
 * work-groups (w4a8_matmul_ex forces the count). Errors: INVALID_ARG, UNSUPPORTED (group
 * size, N % 8, K, size), ALIGNMENT, HIP (launch or workspace failure).
 */
int w4a8_matmul(const uint8_t* xq, const float* sx, const float* xsum, const int32_t* qweight, const void* scales,
                const void* zeros, void* y, int64_t M, int64_t N, int64_t K, int64_t group_size, int layout,
                void* stream);

/* w4a8_matmul_ex - w4a8_matmul with the split-K count forced: `splits` work-groups along K
 * per output tile of 128 x 256 (64 or 32 rows when M is that small; 0: the library's
 * choice; 1..K/128), summed in split order
 * (deterministic). With splits > 1 the call uses the split-K workspace of `stream` (see
 * w4a16_matmul on graph capture). Errors as w4a8_matmul, plus INVALID_ARG for splits out of
 * range. */
int w4a8_matmul_ex(const uint8_t* xq, const float* sx, const float* xsum, const int32_t* qweight,
                   const void* scales, const void* zeros, void* y, int64_t M, int64_t N, int64_t K,
                   int64_t group_size, int layout, int splits, void* stream);

/*
 * w4a16_read_probe - measurement hook: a plain read of `bytes` bytes of `buf` with the
 * decode kernel's load width (16 bytes per lane) and cache policy (non-temporal), and no
 * other work. "Triton Kernel Matches bitsandbytes: Why Both Lose to Math", section "Roofline
 * First: Calculate the Ceiling Before Writing Code", divides by the bandwidth measured on
 * the machine itself; this is that measurement for the weight stream.
 *   buf    device, 16-byte aligned; bytes a positive multiple of 16
 *   sink   device uint32 [256], 4-byte aligned: written only in the unlikely case that the
 *          XOR of a lane's 64 bytes equals 0x9E3779B9 (it keeps the loads alive)
 * Asynchronous on `stream`. Errors: INVALID_ARG, UNSUPPORTED, ALIGNMENT, HIP.
 */
int w4a16_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/* w4a16_strerror - static description of an error code (never NULL). */
const char* w4a16_strerror(int code);

/* w4a16_last_error_detail - message of the last failing call on this thread ("" if none). */
const char* w4a16_last_error_detail(void);

/* w4a16_version - library version as major*10000 + minor*100 + patch. */
int w4a16_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
