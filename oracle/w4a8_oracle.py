"""Oracle for the W4A8 variant: 8-bit floating-point activations x 4-bit weights.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
bench.py may import this module. It shares no code with the HIP library and imports
nothing from it (it uses the W4A16 oracle's unpacking, which is oracle code too).

Sources (the pages this follows):
  [P1] "Beating FP16 with 4-bit Weights: A Portable W4A16 GEMM in Triton", section
       "What's next": FP8 activations for a W4A8 variant of the same kernel.
  [P3] GemLite README: FP8 x Wn among the supported precisions, 8-bit activations
       quantised dynamically with one scale per row ("channelwise" activation quant).
  The E4M3 format itself is the OCP 8-bit floating-point one: sign, 4 exponent bits with
  bias 7, 3 mantissa bits, subnormals at exponent 0, no infinities, S.1111.111 is NaN,
  largest finite value 448.

Readings taken where the pages are silent:
  R18 Activations are quantised per row, dynamically: amax = max_k |x[m, k]| (exact in
      fp32), scale sx = fl32(amax / 448) (1.0 when amax is 0), codes
      xq = E4M3(fl32(x / sx)), true fp32 division, round-to-nearest-even, saturating at
      +-448 (the format has no infinity).
  R19 The weight side is the exact dequantisation of [P1] "The design", (q - z) * s, with
      q - z unrounded whatever the zero point: only the activations are 8-bit. (An
      implementation may use the identity sum_k a_k (q_k - z) = sum_k a_k q_k - z sum_k a_k,
      with the bare codes q, which E4M3 holds exactly, as the 8-bit operand.)
  R20 y[m, n] = sx[m] * sum_g s[g, n] * sum_{k in g} dec(xq[m, k]) * (q[k, n] - z[g, n]) with
      the W4A16 grouping (one fp16 scale per group and column). Groups of 128 or 256 rows:
      one 8-bit matrix instruction spans 128 rows of K, and a scale must not change inside it.
  R22 Block sums of the activation codes: S[b, m] = sum over the 128 K indices of block b of
      dec(xq[m, k]), the per-row quantity the zero-point term of R19's identity needs.
The matmul and the block sums are defined in fp64 (each product of an E4M3 value, an
integer below 2^11 and an fp16 scale is exact; only the sums round).

Pins (tests/oracle_pins_w4a8.py): the format's defining values, the round trip of every
finite code, hand-worked ties and saturation, the quantiser's invariants, closed-form
products (far zero points included), block sums, agreement with the W4A16 oracle on
activations the format holds exactly, and a mutation suite (tests/test_oracle_mutants_w4a8.py).
"""
import numpy as np

from .w4a16_oracle import unpack, _check_group

E4M3_MAX = 448.0          # largest finite E4M3 value, S.1111.110
E4M3_BIAS = 7
W4A8_GROUPS = (128, 256)  # R20


def e4m3_decode(codes):
    """Value of each E4M3 code (uint8), from the bit fields: fp64 array, NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - E4M3_BIAS)
    subnormal = (m / 8.0) * np.exp2(1.0 - E4M3_BIAS)
    v = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


# the non-negative finite values in code order (codes 0x00 .. 0x7E are increasing)
_POS_GRID = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(values):
    """Round each value to the nearest E4M3 value (ties to the even code), saturating at
    +-448. The sign of zero is kept. NaN input is an error."""
    v = np.asarray(values, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN has no E4M3 rounding here")
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_GRID, a, side="left"), 0, 0x7E)   # first grid value >= a
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - _POS_GRID[lo]
    d_hi = _POS_GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)


def quantize_activations(x):
    """R18: fp16 x [M, K] -> (codes uint8 [M, K], scales fp32 [M])."""
    x = np.asarray(x)
    if x.dtype != np.float16 or x.ndim != 2:
        raise ValueError("x must be a 2-D float16 array")
    x32 = x.astype(np.float32)
    amax = np.abs(x32).max(axis=1)
    sx = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    scaled = (x32 / sx[:, None]).astype(np.float32)        # one fp32 division per element
    return e4m3_encode(scaled), sx


BLOCK = 128               # R22: K rows per activation block sum (one 8-bit matrix instruction)


def activation_block_sums(xq):
    """R22: S[b, m] = sum_{k in block b} dec(xq[m, k]), fp64 [K/128, M] (block-major).

    Exact: every finite E4M3 value is a multiple of 2^-9 of magnitude at most 448, so every
    partial sum of 128 of them is a multiple of 2^-9 below 2^16, which fp64 holds exactly
    in any summation order."""
    xq = np.asarray(xq, dtype=np.uint8)
    M, K = xq.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 128")
    a = e4m3_decode(xq)
    return a.reshape(M, K // BLOCK, BLOCK).sum(axis=2).T


def weight_values(codes, zeros, group_size):
    """R19: the exact q - z [K, N] (q uint8 codes, zeros fp16 [K/g, N]), fp64."""
    codes = np.asarray(codes)
    K, N = codes.shape
    _check_group(K, group_size)
    z = np.repeat(np.asarray(zeros).astype(np.float64), group_size, axis=0)
    return codes.astype(np.float64) - z


def matmul_w4a8(xq, sx, qweight, scales, zeros, group_size=128, layout="linear"):
    """R20: fp64 [M, N] from activation codes xq [M, K], their row scales sx [M], and the
    W4A16 weight format."""
    if group_size not in W4A8_GROUPS:
        raise ValueError("W4A8 takes groups of 128 or 256 rows")
    xq = np.asarray(xq, dtype=np.uint8)
    codes = unpack(qweight, layout)
    K, N = codes.shape
    if xq.shape[1] != K:
        raise ValueError("xq and qweight disagree on K")
    a = e4m3_decode(xq)                                     # [M, K]
    w = weight_values(codes, zeros, group_size)             # [K, N]
    s = np.asarray(scales).astype(np.float64)               # [K/g, N]
    y = np.zeros((xq.shape[0], N))
    for g in range(K // group_size):
        rows = slice(g * group_size, (g + 1) * group_size)
        y += (a[:, rows] @ w[rows, :]) * s[g][None, :]
    return y * np.asarray(sx, dtype=np.float64)[:, None]
