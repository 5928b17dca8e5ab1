"""Oracle: a plain, slow, obviously correct CPU statement of y = x . dequant(Wq).

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
bench.py may import this module. It shares no code with the HIP library and imports
nothing from it.

Sources (the pages this follows):
  [P1] "Beating FP16 with 4-bit Weights: A Portable W4A16 GEMM in Triton",
       section "The design" and its inner-loop listing: one scale and one zero-point per
       group of 128 rows (GPTQ/AWQ style); eight 4-bit values packed into one int32 along
       the contraction dimension, packed row i / nibble j holding K index 8i+j; dequant
       inside the loop as (w - zero) * scale; products accumulated in fp32.
  [P3] GemLite README, "Packing": the HQQ convention (W_q - zeros) * scales ~= W; its
       settings list takes any group size divisible by 32.
  [P2] "Triton Kernel Matches bitsandbytes: Why Both Lose to Math", section "Three Kernel
       Versions and Two Bugs": symmetric 4-bit codes carry a +8 zero point.
  [P1] section "Code": the tests cover several group sizes and both symmetric and
       asymmetric quantisation.

Readings taken where the pages are silent:
  R1  W is laid out [K, N] (input x output), so y[M,N] = x[M,K] @ W[K,N].
  R2  Asymmetric min/max quantisation per (K-group, column): scale = (max-min)/15 stored
      as fp16 (round-to-nearest-even), zero = round(-min/scale) using the stored fp16
      scale, stored as fp16; q = clamp(round(w/scale) + zero, 0, 15).  round() is
      round-half-to-even; every intermediate is an fp32 operation (true division, no
      fused multiply-add).
  R3  Nibble j of a packed word sits at bit shift 4j (least significant nibble first).
  R4  A group whose fp16 scale rounds to zero gets scale 1.0.
  R5  The zero point is not clamped; |zero| <= 1024 is the supported domain.
  R6  Non-finite W, an fp16 scale overflow or |zero| > 1024 are errors.
  R7  Symmetric mode: scale = max|w|/7 per (K-group, column) stored as fp16 (rne; 1.0 when
      it rounds to zero), zero = 8, q = clamp(round(w/scale) + 8, 0, 15); the same fp32
      steps as R2. Group sizes are multiples of 8 here (the library takes 32, 64, 128, 256).
  R8  Interleaved layout ([P1] "What's next": pre-permute the weights offline so they
      reach the matrix instruction in the order it wants, with no runtime reshape): nibble p
      of packed word i holds K index 8i + NIBBLE_K["interleaved"][p] = 8i + (0, 2, 4, 6, 1,
      3, 5, 7)[p], i.e. even K offsets in nibbles 0..3 and odd ones in nibbles 4..7. Codes,
      scales, zeros and the product are those of the linear layout; only the word packing
      differs.
Everything the GPU path must reproduce bit for bit (codes, fp16 dequant) is defined
here; the matmul is defined in fp64 on the exact fp32 dequantised weights.

Pins (tests/test_oracle_pins.py): hand-computed packed words, exact closed-form
quantisation and products on K=128/N=8 and multi-group cases, the min-code invariant,
the per-element error bound, math.fsum brute force, and a mutation suite.
"""
import numpy as np

GROUP_SIZE = 128          # [P1] "The design": one scale/zero per group of 128 rows
NIBBLES_PER_WORD = 8      # [P1] "The design": eight 4-bit values per int32 along K
QMAX = 15                 # 4-bit unsigned codes 0..15
ZERO_LIMIT = 1024.0       # R5


def _check_group(K, group_size):
    if group_size <= 0 or group_size % NIBBLES_PER_WORD != 0:
        raise ValueError("group_size must be a positive multiple of 8")
    if K % group_size != 0:
        raise ValueError("K must be a multiple of group_size")


SYM_ZERO = 8.0            # R7: [P2] "Three Kernel Versions and Two Bugs", the +8 zero point
SYM_QPOS = 7              # R7: largest positive code offset in symmetric mode


def quantize(W, group_size=GROUP_SIZE, symmetric=False):
    """Per-(group, column) 4-bit quantisation: asymmetric min/max (R2, R4-R6) or symmetric
    with a zero point of 8 (R7).

    W: float32 [K, N]. Returns (codes uint8 [K, N], scales fp16 [K/g, N], zeros fp16 [K/g, N]).
    [P1] "The design" fixes the grouping (one scale and zero per group of K-rows per column);
    [P3] "Packing" fixes that (codes - zeros) * scales approximates W.
    """
    if symmetric:
        return _quantize_symmetric(W, group_size)
    W = np.asarray(W)
    if W.dtype != np.float32 or W.ndim != 2:
        raise ValueError("W must be a 2-D float32 array")
    K, N = W.shape
    _check_group(K, group_size)
    if not np.all(np.isfinite(W)):
        raise ValueError("W holds a non-finite value")
    G = K // group_size
    Wg = W.reshape(G, group_size, N)                      # Wg[g, r, n] = W[g*gs + r, n]

    mn = Wg.min(axis=1)                                   # exact
    mx = Wg.max(axis=1)                                   # exact
    rng = mx - mn                                         # fp32 subtraction
    s32 = rng / np.float32(QMAX)                          # fp32 division
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)                      # round to nearest even
    if not np.all(np.isfinite(s16)):
        raise ValueError("scale overflows fp16")
    s16 = np.where(s16 == 0, np.float16(1.0), s16)        # R4
    s = s16.astype(np.float32)                            # exact widening

    z = np.rint(-mn / s)                                  # fp32 division, then round-half-even
    if np.any(np.abs(z) > ZERO_LIMIT):
        raise ValueError("zero point outside the supported domain |z| <= 1024")
    z16 = z.astype(np.float16)                            # exact: integer with |z| <= 1024

    q = np.rint(Wg / s[:, None, :]) + z[:, None, :]       # round first, then add the offset
    q = np.clip(q, 0, QMAX)
    codes = q.astype(np.uint8).reshape(K, N)
    return codes, s16, z16


def _quantize_symmetric(W, group_size):
    """R7: scale = fp16(max|w| / 7), zero = 8, q = clamp(rne(w / scale) + 8, 0, 15)."""
    W = np.asarray(W)
    if W.dtype != np.float32 or W.ndim != 2:
        raise ValueError("W must be a 2-D float32 array")
    K, N = W.shape
    _check_group(K, group_size)
    if not np.all(np.isfinite(W)):
        raise ValueError("W holds a non-finite value")
    G = K // group_size
    Wg = W.reshape(G, group_size, N)
    amax = np.abs(Wg).max(axis=1)                         # exact
    s32 = amax / np.float32(SYM_QPOS)                     # fp32 division
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)                      # round to nearest even
    if not np.all(np.isfinite(s16)):
        raise ValueError("scale overflows fp16")
    s16 = np.where(s16 == 0, np.float16(1.0), s16)        # R4
    s = s16.astype(np.float32)
    q = np.rint(Wg / s[:, None, :]) + np.float32(SYM_ZERO)
    q = np.clip(q, 0, QMAX)
    codes = q.astype(np.uint8).reshape(K, N)
    z16 = np.full((G, N), SYM_ZERO, dtype=np.float16)
    return codes, s16, z16


# K offset (within the word's 8 K indices) held by nibble p (bits 4p..4p+3) of a word
NIBBLE_K = {
    "linear": (0, 1, 2, 3, 4, 5, 6, 7),        # R3: [P1] "The design", nibble j <-> K 8i + j
    "interleaved": (0, 2, 4, 6, 1, 3, 5, 7),   # R8
}


def pack(codes, layout="linear"):
    """Pack codes [K, N] (values 0..15) into int32 words [K/8, N].

    linear ([P1] "The design", R3): packed row i, nibble j holds K index 8*i + j.
    interleaved (R8): nibble p holds K index 8*i + NIBBLE_K["interleaved"][p].
    """
    codes = np.asarray(codes)
    K, N = codes.shape
    if K % NIBBLES_PER_WORD != 0:
        raise ValueError("K must be a multiple of 8")
    if codes.max(initial=0) > QMAX:
        raise ValueError("codes must lie in 0..15")
    words = np.zeros((K // NIBBLES_PER_WORD, N), dtype=np.uint32)
    for p, k in enumerate(NIBBLE_K[layout]):
        words |= codes[k::NIBBLES_PER_WORD, :].astype(np.uint32) << np.uint32(4 * p)
    return words.view(np.int32)


def unpack(qweight, layout="linear"):
    """Inverse of pack: int32 [K/8, N] -> uint8 codes [K, N]. Shifts an unsigned view."""
    words = np.asarray(qweight).view(np.uint32)
    P, N = words.shape
    codes = np.zeros((P * NIBBLES_PER_WORD, N), dtype=np.uint8)
    for p, k in enumerate(NIBBLE_K[layout]):
        codes[k::NIBBLES_PER_WORD, :] = (words >> np.uint32(4 * p)) & np.uint32(0xF)
    return codes


def dequant(codes, scales, zeros, group_size=GROUP_SIZE):
    """fp32 dequant w = (q - zero) * scale, broadcast per (K-group, column) ([P1], [P3]).

    Exact in fp32 on the supported domain: |q - z| <= 1039 has at most 11 significant bits
    and an fp16 scale 11, so the product fits the 24-bit fp32 significand.
    """
    codes = np.asarray(codes)
    K, N = codes.shape
    _check_group(K, group_size)
    s = np.repeat(np.asarray(scales).astype(np.float32), group_size, axis=0)   # [K, N]
    z = np.repeat(np.asarray(zeros).astype(np.float32), group_size, axis=0)    # [K, N]
    return (codes.astype(np.float32) - z) * s


def dequant_fp16(codes, scales, zeros, group_size=GROUP_SIZE):
    """The fp16 weight a kernel holds after dequantising: fp16 round-to-nearest-even of
    the exact fp32 value (q - zero) * scale."""
    return dequant(codes, scales, zeros, group_size).astype(np.float16)


def matmul(x, qweight, scales, zeros, group_size=GROUP_SIZE, layout="linear"):
    """y[m, n] = sum_k x[m, k] * dequant(W)[k, n], accumulated in fp64.

    x: fp16 [M, K]. Returns fp64 [M, N]. Every product of an fp16 activation and an fp32
    dequantised weight is exact in fp64; only the summation rounds.
    """
    x = np.asarray(x)
    if x.dtype != np.float16 or x.ndim != 2:
        raise ValueError("x must be a 2-D float16 array")
    codes = unpack(qweight, layout)
    if x.shape[1] != codes.shape[0]:
        raise ValueError("x and qweight disagree on K")
    w = dequant(codes, scales, zeros, group_size).astype(np.float64)
    return x.astype(np.float64) @ w


def quantize_pack(W, group_size=GROUP_SIZE, symmetric=False, layout="linear"):
    """quantize then pack: W fp32 [K, N] -> (qweight int32 [K/8, N], scales, zeros)."""
    codes, s16, z16 = quantize(W, group_size, symmetric)
    return pack(codes, layout), s16, z16
