"""Pins for the W4A8 oracle: what the E4M3 format, the quantiser's definition and the
W4A16 oracle (itself pinned) fix.

Each pin takes an oracle-like module ``o`` and raises AssertionError on a mismatch; they
run against the real oracle (test_oracle_pins_w4a8.py) and against copies of it with a
planted mistake (test_oracle_mutants_w4a8.py). Expected values are the format's defining
values, hand-worked roundings, invariants and closed forms; nothing retypes the oracle.

Pages cited: "Beating FP16 with 4-bit Weights", section "What's next" (FP8 activations for
a W4A8 variant); GemLite README (FP8 x Wn, dynamic per-row 8-bit activation quant).
"""
import math

import numpy as np

import oracle as w4a16_oracle
import synth


def _exact_weight():
    """K=128, N=8: W[k, n] = ((k + n) mod 16 - 8) * 2**-6: scale 2**-6, zero 8, codes
    (k + n) mod 16, so q - z = (k + n) mod 16 - 8 (exact in E4M3)."""
    k = np.arange(128)[:, None]
    n = np.arange(8)[None, :]
    return (((k + n) % 16 - 8) * 2.0 ** -6).astype(np.float32)


def pin_e4m3_defining_values(o):
    """Values the E4M3 format defines (bias 7, subnormals at exponent 0, 448 the largest
    finite value, S.1111.111 NaN)."""
    expect = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0,
              0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x58: 16.0, 0x5A: 20.0, 0x7E: 448.0, 0xB8: -1.0,
              0xFE: -448.0, 0x81: -(2.0 ** -9)}
    codes = np.array(list(expect), dtype=np.uint8)
    got = o.e4m3_decode(codes)
    assert np.array_equal(got, np.array(list(expect.values()))), got
    assert np.isnan(o.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    neg0 = o.e4m3_decode(np.array([0x80], np.uint8))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) < 0


def pin_e4m3_roundtrip(o):
    """Every finite code decodes to a value that encodes back to the same code; the 127
    non-negative finite values increase strictly with the code."""
    c = np.array([i for i in range(256) if i & 0x7F != 0x7F], dtype=np.uint8)
    assert np.array_equal(o.e4m3_encode(o.e4m3_decode(c)), c)
    pos = o.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


def pin_e4m3_rounding(o):
    """Hand-worked nearest-even roundings and saturation."""
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (1.06, 0x38), (1.07, 0x39), (-1.0625, 0xB8),
             (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (15 * 2.0 ** -10, 0x08), (17.0, 0x58), (19.0, 0x5A),
             (449.0, 0x7E), (464.0, 0x7E), (1e6, 0x7E), (-1e6, 0xFE), (440.0, 0x7E), (424.0, 0x7D),
             (432.0, 0x7E), (400.0, 0x7C)]
    v = np.array([c[0] for c in cases])
    got = o.e4m3_encode(v)
    assert np.array_equal(got, np.array([c[1] for c in cases], np.uint8)), [hex(g) for g in got]


def pin_activation_quantiser(o):
    """Per-row dynamic scale: a zero row, the row maximum at 448, power-of-two scaling,
    row independence and the rounding bound."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((4, 256)) * np.array([[1.0], [0.01], [30.0], [1.0]])).astype(np.float16)
    x[3] = 0
    x[1, 17] = np.float16(-0.5)                  # the largest magnitude of row 1, negative
    xq, sx = o.quantize_activations(x)
    assert xq.dtype == np.uint8 and sx.dtype == np.float32 and xq.shape == x.shape
    assert sx[3] == 1.0 and np.all(xq[3] & 0x7F == 0)
    for r in range(3):
        j = int(np.argmax(np.abs(x[r].astype(np.float32))))
        assert xq[r, j] & 0x7F == 0x7E, (r, hex(xq[r, j]))      # the maximum maps to 448
        assert (xq[r, j] >> 7) == (x[r, j] < 0)
    assert xq[1, 17] == 0xFE
    x2 = (x.astype(np.float32) * 4).astype(np.float16)           # exact in fp16
    xq2, sx2 = o.quantize_activations(x2)
    assert np.array_equal(xq2, xq) and np.array_equal(sx2[:3], sx[:3] * 4)
    x3 = x.copy()
    x3[2] *= np.float16(2)
    assert np.array_equal(o.quantize_activations(x3)[0][:2], xq[:2])
    # |dec * sx - x| <= 2**-4 |x| in the normal range, <= sx * 2**-10 below it
    d = o.e4m3_decode(xq) * sx[:, None].astype(np.float64)
    xf = x.astype(np.float64)
    err = np.abs(d - xf)
    tol = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * sx[:, None]) * (1 + 1e-6)
    assert np.all(err <= tol), err.max()


def pin_weight_values(o):
    """q - z exactly, whatever the zero point: zero 8 gives -8..7, zero -5 gives 5..20 (17 and
    19 included: no 8-bit rounding of the weight side), zeros -1000 and 1024 give 1000..1015
    and -1024..-1009."""
    codes = np.tile(np.arange(16, dtype=np.uint8), 8)[:, None].repeat(4, axis=1)   # K=128, N=4
    zeros = np.array([[8.0, -5.0, -1000.0, 1024.0]], dtype=np.float16)
    w = o.weight_values(codes, zeros, 128)
    q = np.arange(16.0)
    assert np.array_equal(w[:16, 0], q - 8) and np.array_equal(w[:16, 1], q + 5), w[:16, :2]
    assert np.array_equal(w[:16, 2], q + 1000) and np.array_equal(w[:16, 3], q - 1024), w[:16, 2:]


def pin_w4a8_closed_form(o):
    """Exact weights (scale 2**-6, zero 8) against activations of magnitude 448 (row scale
    exactly 1): x = 448 everywhere gives -448; 448 * e_k0 gives 7 * ((k0 + n) mod 16 - 8);
    (-1)**k * 448 gives -448 / +448 for even / odd columns."""
    qw, s, z = w4a16_oracle.quantize_pack(_exact_weight())
    assert np.all(s == np.float16(2.0 ** -6)) and np.all(z == 8)
    x = np.zeros((3, 128), dtype=np.float16)
    x[0] = 448
    k0 = 37
    x[1, k0] = 448
    x[2] = np.where(np.arange(128) % 2 == 0, 448, -448)
    xq, sx = o.quantize_activations(x)
    assert np.array_equal(sx, np.ones(3, np.float32))
    y = o.matmul_w4a8(xq, sx, qw, s, z)
    n = np.arange(8)
    assert np.array_equal(y[0], np.full(8, -448.0))
    assert np.array_equal(y[1], 7.0 * ((k0 + n) % 16 - 8))
    assert np.array_equal(y[2], np.where(n % 2 == 0, -448.0, 448.0))


def _grid_activations(M, K, seed, log2_scale):
    """fp16 activations on the E4M3 grid times 2**log2_scale, each row holding +-448 * 2**e
    once, so the row scale is exactly 2**e and the codes decode to x / sx exactly."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 0x7E, size=(M, K)).astype(np.uint8) | (rng.integers(0, 2, size=(M, K)) << 7).astype(np.uint8)
    codes[:, rng.integers(0, K)] = 0x7E
    vals = np.zeros((M, K))
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        e, m = (c >> 3) & 0xF, c & 7
        v = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        vals[codes == c] = -v if c & 0x80 else v
    return (vals * 2.0 ** log2_scale).astype(np.float16)


def pin_w4a8_matches_w4a16_on_exact_activations(o):
    """When every activation is held exactly (grid values, power-of-two row scale), W4A8
    computes the same product as the W4A16 oracle, for zero points near 8 and for one-signed
    groups whose zero points lie far from it."""
    for g, shape, ls, mean in [(128, (5, 512, 24), 0, 0.0), (256, (3, 768, 16), -8, 0.0), (128, (2, 256, 40), -3, 0.0),
                               (128, (3, 384, 16), 0, 1.0), (256, (2, 512, 8), -2, -1.0)]:
        M, K, N = shape
        qw, s, z = w4a16_oracle.quantize_pack(synth.weight_custom(K, N, seed=5 + K, std=0.02, mean=mean), g)
        if mean:
            assert np.all(np.abs(z.astype(np.float64)) > 60)              # far from [-1, 16]
        x = _grid_activations(M, K, seed=K + g, log2_scale=ls)
        xq, sx = o.quantize_activations(x)
        assert np.array_equal(sx, np.full(M, 2.0 ** ls, np.float32))
        y8 = o.matmul_w4a8(xq, sx, qw, s, z, g)
        y16 = w4a16_oracle.matmul(x, qw, s, z, g)
        assert np.allclose(y8, y16, rtol=1e-12, atol=1e-12 * np.abs(y16).max()), np.abs(y8 - y16).max()


def pin_w4a8_brute_force(o):
    """A tiny case summed product by product with math.fsum from the decoded codes."""
    K, N, M = 256, 3, 2
    qw, s, z = w4a16_oracle.quantize_pack(synth.weight(K, N, wid=6))
    x = (np.random.default_rng(9).standard_normal((M, K)) * 0.7).astype(np.float16)
    xq, sx = o.quantize_activations(x)
    y = o.matmul_w4a8(xq, sx, qw, s, z)
    a = o.e4m3_decode(xq)
    codes = w4a16_oracle.unpack(qw)
    for m in range(M):
        for n in range(N):
            terms = []
            for k in range(K):
                g = k // 128
                w = float(codes[k, n]) - float(z[g, n])          # exact: no 8-bit rounding of q - z
                terms.append(a[m, k] * w * float(s[g, n]))
            ref = math.fsum(terms) * float(sx[m])
            assert abs(y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref)), (m, n, y[m, n], ref)


def pin_w4a8_far_zero_exact(o):
    """One-signed groups keep q - z exact in the product: zero -5 with codes 12, 14, 13 gives
    17, 19, 18 (times the activation 448, row scale 1); zero 1000 with code 3 gives -997;
    zero -1000 with code 15 gives 1015."""
    codes = np.tile(np.arange(16, dtype=np.uint8), 8)[:, None].repeat(3, axis=1)   # K=128, N=3
    qw = w4a16_oracle.pack(codes)
    s = np.array([[1.0, 0.5, 2.0 ** -10]], dtype=np.float16)
    z = np.array([[-5.0, 1000.0, -1000.0]], dtype=np.float16)
    x = np.zeros((4, 128), dtype=np.float16)
    x[0, 12] = x[1, 14] = x[2, 13] = x[3, 3] = 448                        # row scale 1
    x[3, 15] = -448
    xq, sx = o.quantize_activations(x)
    assert np.array_equal(sx, np.ones(4, np.float32))
    y = o.matmul_w4a8(xq, sx, qw, s, z)
    assert np.array_equal(y[:3, 0], np.array([17.0, 19.0, 18.0]) * 448), y[:3, 0]
    # row 3: 448 at q = 3 and -448 at q = 15
    assert y[3, 1] == 0.5 * 448 * ((3 - 1000) - (15 - 1000)), y[3, 1]
    assert y[3, 2] == 2.0 ** -10 * 448 * ((3 + 1000) - (15 + 1000)), y[3, 2]
    assert y[0, 2] == 2.0 ** -10 * 448 * (12 + 1000), y[0, 2]


def pin_block_sums(o):
    """Per-(block, row) sums of the decoded codes: 128 x 448 gives 57344, alternating signs
    give 0, a single code its value; on random codes the math.fsum of the decoded values;
    and the identity sum_k a (q - z) = sum_k a q - z S that lets a kernel apply the zero
    point to the sums."""
    x = np.zeros((3, 256), dtype=np.float16)
    x[0] = 448
    x[1] = np.where(np.arange(256) % 2 == 0, 448, -448)
    x[2, 130] = 448
    x[2, 5] = 0.5 * 448
    xq, sx = o.quantize_activations(x)
    S = o.activation_block_sums(xq)
    assert S.shape == (2, 3)
    assert np.array_equal(S[:, 0], [57344.0, 57344.0]) and np.array_equal(S[:, 1], [0.0, 0.0])
    assert np.array_equal(S[:, 2], [224.0, 448.0]), S[:, 2]
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 256, size=(4, 384)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                                  # no NaN codes
    S = o.activation_block_sums(codes)
    for b in range(3):
        for m in range(4):
            ref = math.fsum(float(o.e4m3_decode(np.array([c], np.uint8))[0]) for c in codes[m, b * 128:(b + 1) * 128])
            assert S[b, m] == ref, (b, m, S[b, m], ref)
    qw, s, z = w4a16_oracle.quantize_pack(synth.weight_custom(384, 5, seed=3, std=0.02, mean=1.0))
    a = o.e4m3_decode(codes)
    q = w4a16_oracle.unpack(qw).astype(np.float64)
    for b in range(3):
        rows = slice(128 * b, 128 * (b + 1))
        lhs = a[:, rows] @ (q[rows] - z[b].astype(np.float64))
        rhs = a[:, rows] @ q[rows] - np.outer(S[b], z[b].astype(np.float64))
        assert np.allclose(lhs, rhs, rtol=0, atol=1e-9 * np.abs(lhs).max()), b


ALL_PINS = [pin_e4m3_defining_values, pin_e4m3_roundtrip, pin_e4m3_rounding, pin_activation_quantiser,
            pin_weight_values, pin_w4a8_closed_form, pin_w4a8_far_zero_exact, pin_block_sums,
            pin_w4a8_matches_w4a16_on_exact_activations,
            pin_w4a8_brute_force]
