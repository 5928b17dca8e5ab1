"""Pins for the oracle: checks against what the pages and the mathematics fix.

Each pin takes an oracle-like module ``o`` and raises AssertionError on a mismatch. The
same pins run against the real oracle (test_oracle_pins.py) and against copies of it with
a planted mistake (test_oracle_mutants.py), which every pin set must catch.

Nothing here retypes the oracle's formulas: expected values are hand-derived closed
forms, invariants of the quantiser, or exact sums.

Pages cited: "Beating FP16 with 4-bit Weights: A Portable W4A16 GEMM in Triton",
section "The design" (grouping, K-packing, dequant (w - zero) * scale, fp32 accumulate).
"""
import math

import numpy as np

import synth


def _exact_group_weight(K, N, centres, log2_spacing, group_size=128):
    """W[k, n] = ((k + n) mod 16 - c_g) * 2**e_g for K-group g = k // group_size.

    Each aligned block of 16 rows in a column visits every residue 0..15 once, so every
    group's min is -c_g * d_g and its max (15 - c_g) * d_g: the scale is exactly d_g
    (a power of two), the zero is exactly c_g and the codes are (k + n) mod 16.
    """
    k = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    g = k // group_size
    c = np.asarray(centres, dtype=np.float64)[g]
    d = np.exp2(np.asarray(log2_spacing, dtype=np.float64))[g]
    return (((k + n) % 16 - c) * d).astype(np.float32)


def pin_hand_words(o):
    """Packed words worked out by hand: nibble j of word i is K index 8i + j at shift 4j."""
    codes = np.zeros((8, 5), dtype=np.uint8)
    codes[:, 0] = np.arange(8)          # 0,1,...,7   -> 0x76543210
    codes[:, 1] = 15                    # all ones    -> 0xFFFFFFFF == int32 -1
    codes[7, 2] = 8                     # only top    -> 0x80000000 == int32 min
    codes[0, 3] = 1                     # only bottom -> 0x00000001
    codes[3, 4] = 0xA                   # nibble 3    -> 0x0000A000
    words = o.pack(codes)
    assert words.dtype == np.int32 and words.shape == (1, 5)
    expect = np.array([[0x76543210, -1, -2**31, 1, 0xA000]], dtype=np.int64)
    assert np.array_equal(words.astype(np.int64), expect), words
    assert np.array_equal(o.unpack(words), codes)


def pin_roundtrip(o):
    """pack and unpack are inverse bijections (codes <-> words), bit for bit."""
    for K, N, seed in [(8, 1, 0), (64, 24, 1), (256, 13, 2)]:
        c = synth.uniform_codes(K, N, seed)
        assert np.array_equal(o.unpack(o.pack(c)), c)
    rng = np.random.default_rng(7)
    words = rng.integers(-2**31, 2**31, size=(9, 11), dtype=np.int64).astype(np.int32)
    assert np.array_equal(o.pack(o.unpack(words)), words)


def pin_exact_group(o):
    """K=128, N=8 exact case: scale 2**-6, zero 8, codes (k+n) mod 16, zero error."""
    W = _exact_group_weight(128, 8, [8], [-6])
    codes, s, z = o.quantize(W)
    assert s.dtype == np.float16 and z.dtype == np.float16
    assert s.shape == (1, 8) and z.shape == (1, 8)
    assert np.all(s == np.float16(2.0 ** -6)) and np.all(z == 8)
    k = np.arange(128)[:, None]
    n = np.arange(8)[None, :]
    assert np.array_equal(codes, ((k + n) % 16).astype(np.uint8))
    assert np.array_equal(o.dequant(codes, s, z), W)
    qw, s2, z2 = o.quantize_pack(W)
    # column 0: rows 0..7 hold codes 0..7, rows 8..15 codes 8..15; column 4 is shifted by 4
    u = qw.view(np.uint32)
    assert u.shape == (16, 8)
    assert u[0, 0] == 0x76543210 and u[1, 0] == 0xFEDCBA98
    assert u[0, 4] == 0xBA987654 and u[1, 4] == 0x3210FEDC


def pin_exact_products(o):
    """Hand-summed products on the K=128, N=8 case (every value exact in fp16)."""
    W = _exact_group_weight(128, 8, [8], [-6])
    qw, s, z = o.quantize_pack(W)
    ones = np.ones((1, 128), dtype=np.float16)
    # sum over 8 blocks of sum_{r=0}^{15} (r - 8) / 64 = 8 * (-8) / 64 = -1 for every column
    assert np.array_equal(o.matmul(ones, qw, s, z), -np.ones((1, 8)))
    alt = ((-1.0) ** np.arange(128))[None, :].astype(np.float16)
    # (-1)^k (r - 8) summed over a block = (-1)^n * (-8); over 8 blocks / 64 -> -(-1)^n
    assert np.array_equal(o.matmul(alt, qw, s, z), -((-1.0) ** np.arange(8))[None, :])
    for k0 in (0, 5, 77, 127):
        e = np.zeros((1, 128), dtype=np.float16)
        e[0, k0] = 1
        expect = (((k0 + np.arange(8)) % 16) - 8) / 64.0
        assert np.array_equal(o.matmul(e, qw, s, z)[0], expect)


def pin_multigroup(o):
    """Three K-groups with different spacing and centre; zeros 8, 3, 12; y(ones) = -19."""
    centres, log2d = [8, 3, 12], [-6, -5, -4]
    W = _exact_group_weight(384, 5, centres, log2d)
    codes, s, z = o.quantize(W)
    assert s.shape == (3, 5) and z.shape == (3, 5)
    for g in range(3):
        assert np.all(s[g] == np.float16(2.0 ** log2d[g])) and np.all(z[g] == centres[g])
    assert np.array_equal(o.dequant(codes, s, z), W)
    qw = o.pack(codes)
    ones = np.ones((1, 384), dtype=np.float16)
    # per group 8 * sum_r (r - c) * d = 8 * (120 - 16 c) * d: -1 + 18 - 36 = -19
    assert np.array_equal(o.matmul(ones, qw, s, z), np.full((1, 5), -19.0))
    for k0 in (3, 130, 300, 383):
        e = np.zeros((2, 384), dtype=np.float16)
        e[1, k0] = 1
        g = k0 // 128
        expect = (((k0 + np.arange(5)) % 16) - centres[g]) * 2.0 ** log2d[g]
        y = o.matmul(e, qw, s, z)
        assert np.array_equal(y[1], expect) and np.array_equal(y[0], np.zeros(5))


def _bound_checks(o, W):
    codes, s16, z16 = o.quantize(W)
    K, N = W.shape
    G = K // 128
    s = s16.astype(np.float64)
    zz = z16.astype(np.float64)
    deq = o.dequant(codes, s16, z16).astype(np.float64)
    Wd = W.astype(np.float64)
    Wg = Wd.reshape(G, 128, N)
    cg = codes.reshape(G, 128, N)
    mn, mx = Wg.min(axis=1), Wg.max(axis=1)
    # fp16 scale is the nearest fp16 to (max - min)/15: within half an fp16 ulp (2**-11 rel.)
    target = (mx - mn) / 15.0
    assert np.all(np.abs(s - target) <= target * 2.0 ** -11 * (1 + 2.0 ** -10))
    # the zero point puts the group minimum at code 0 (round(mn/s) = -round(-mn/s))
    argmin = Wg.argmin(axis=1)
    assert np.all(np.take_along_axis(cg, argmin[:, None, :], axis=1) == 0)
    assert np.all(np.abs(zz * s + mn) <= 0.5 * s * (1 + 2.0 ** -20))
    # the group maximum lands on code 14 or 15
    argmax = Wg.argmax(axis=1)
    top = np.take_along_axis(cg, argmax[:, None, :], axis=1)
    assert np.all((top == 14) | (top == 15))
    # error bound: |W - deq| <= s/2 (plus the fp32 rounding of w/s) unless clamped at 15
    err = np.abs(Wd - deq).reshape(G, 128, N)
    slack = np.abs(Wg) * 2.0 ** -22
    half = 0.5 * s[:, None, :] + slack
    clamped = (cg == 15) & (Wg > deq.reshape(G, 128, N) + half)
    assert np.all(err[~clamped] <= np.broadcast_to(half, err.shape)[~clamped])
    # clamped codes only ever occur at the top and stay within s*(1/2 + 15*2**-11)
    wide = 0.5 * s[:, None, :] + 15 * 2.0 ** -11 * s[:, None, :] + slack
    assert np.all(err[clamped] <= np.broadcast_to(wide, err.shape)[clamped])
    # dequant of every code is the exact value (q - z) * s (no rounding in fp32)
    assert np.array_equal(deq.reshape(G, 128, N),
                          (cg.astype(np.float64) - zz[:, None, :]) * s[:, None, :])
    return int(clamped.sum())


def pin_bounds_random(o):
    """Min-code invariant, max code 14/15, fp16-nearest scale and the error bound on
    random weights: the N(0, 0.02) workload draw and one-signed / wide groups."""
    _bound_checks(o, synth.weight(512, 96, wid=0))
    _bound_checks(o, synth.weight_custom(256, 64, seed=1, std=0.02, mean=1.0))
    _bound_checks(o, synth.weight_custom(256, 64, seed=2, std=3.0, mean=-2.0))


def pin_fsum(o):
    """Oracle y within K * 2**-53 * sum|terms| of math.fsum over the exact products."""
    M, K, N = 3, 256, 7
    W = synth.weight(K, N, wid=0)
    x = synth.activations(M, K, wid=0)
    qw, s, z = o.quantize_pack(W)
    y = o.matmul(x, qw, s, z)
    assert y.dtype == np.float64 and y.shape == (M, N)
    codes = o.unpack(qw)
    deq = o.dequant(codes, s, z)
    for m in range(M):
        for n in range(N):
            terms = [float(x[m, k]) * float(deq[k, n]) for k in range(K)]
            exact = math.fsum(terms)
            bound = K * 2.0 ** -53 * sum(abs(t) for t in terms)
            assert abs(y[m, n] - exact) <= bound, (m, n, y[m, n], exact)


def pin_dequant_fp16_rounding(o):
    """fp16 dequant rounds the exact product half-to-even.

    scale = 1 + 3*2**-10 (an fp16 value), q - z = 3: the exact product 3 + 9*2**-10 lies
    halfway between the fp16 neighbours 3 + 4*2**-9 and 3 + 5*2**-9; the even one is
    3 + 4*2**-9 = 3.0078125.
    """
    codes = np.full((128, 1), 11, dtype=np.uint8)
    s = np.array([[1 + 3 * 2.0 ** -10]], dtype=np.float16)
    z = np.array([[8]], dtype=np.float16)
    d16 = o.dequant_fp16(codes, s, z)
    assert d16.dtype == np.float16
    assert np.all(d16 == np.float16(3.0078125))
    assert np.all(o.dequant(codes, s, z) == np.float32(3 + 9 * 2.0 ** -10))


def pin_scale_rounding(o):
    """A group whose (max - min)/15 is not an fp16 value stores the nearest fp16 scale.

    Values 0 .. 15 * 1.001 spread evenly: (max-min)/15 = 1.001, nearest fp16 is
    1 + 1*2**-10 = 1.0009765625 (1.001 lies 0.24 ulp above it).
    """
    W = np.zeros((128, 1), dtype=np.float32)
    W[:16, 0] = np.arange(16, dtype=np.float32) * np.float32(1.001)
    codes, s, z = o.quantize(W)
    assert s[0, 0] == np.float16(1.0009765625) and z[0, 0] == 0
    assert codes[15, 0] == 15 and codes[16:, 0].max() == 0


def pin_group_sizes(o):
    """Groups of 32, 64 and 256 rows: per-group exact scale 2**e_g and zero c_g, and the
    hand-summed y(ones) = sum_g (gs/16) * (120 - 16 c_g) * 2**e_g.

    Group sizes divisible by 32 are what the GemLite README's settings accept; the
    grouping itself is [P1] "The design" with another group height.
    """
    cases = [(32, 128, [8, 3, 12, 5], [-6, -5, -4, -7], -4.125),
             (64, 256, [8, 3, 12, 5], [-6, -5, -4, -7], -8.25),
             (256, 512, [4, 10], [-5, -6], 16 * 56 / 32 - 16 * 40 / 64)]
    for gs, K, centres, log2d, y_ones in cases:
        N = 6
        W = _exact_group_weight(K, N, centres, log2d, gs)
        codes, s, z = o.quantize(W, gs)
        G = K // gs
        assert s.shape == (G, N) and z.shape == (G, N)
        for g in range(G):
            assert np.all(s[g] == np.float16(2.0 ** log2d[g])) and np.all(z[g] == centres[g]), (gs, g)
        assert np.array_equal(o.dequant(codes, s, z, gs), W)
        qw = o.pack(codes)
        ones = np.ones((1, K), dtype=np.float16)
        assert np.array_equal(o.matmul(ones, qw, s, z, gs), np.full((1, N), y_ones)), gs
        for k0 in (1, gs + 2, K - 1):
            e = np.zeros((1, K), dtype=np.float16)
            e[0, k0] = 1
            g = k0 // gs
            expect = (((k0 + np.arange(N)) % 16) - centres[g]) * 2.0 ** log2d[g]
            assert np.array_equal(o.matmul(e, qw, s, z, gs)[0], expect), (gs, k0)


def pin_symmetric_exact(o):
    """Symmetric mode on W = ((k + n) mod 15 - 7) * 2**e_g: max|w| = 7 * 2**e_g in every
    group, so the scale is exactly 2**e_g, the zero 8 and the codes (k + n) mod 15 + 1;
    quantisation is lossless and x . dequant equals x . W computed from W itself.

    [P2] "Three Kernel Versions and Two Bugs": symmetric codes carry a +8 zero point.
    """
    for gs, K, log2d in [(32, 128, [-6, -5, -7, -4]), (128, 256, [-5, -6])]:
        N = 5
        k = np.arange(K)[:, None]
        n = np.arange(N)[None, :]
        d = np.exp2(np.asarray(log2d, dtype=np.float64))[k // gs]
        W = ((((k + n) % 15) - 7) * d).astype(np.float32)
        codes, s, z = o.quantize(W, gs, symmetric=True)
        for g in range(K // gs):
            assert np.all(s[g] == np.float16(2.0 ** log2d[g])) and np.all(z[g] == 8), (gs, g)
        assert np.array_equal(codes, (((k + n) % 15) + 1).astype(np.uint8))
        qw, s2, z2 = o.quantize_pack(W, gs, symmetric=True)
        x = synth.activations(3, K, wid=5)
        y = o.matmul(x, qw, s2, z2, gs)
        ref = x.astype(np.float64) @ W.astype(np.float64)
        assert np.allclose(y, ref, rtol=0, atol=1e-12 * np.abs(ref).max()), gs


def pin_symmetric_bounds(o):
    """Symmetric invariants on the N(0, 0.02) draw: the stored scale is the nearest fp16 to
    max|w| / 7, every code lies in 1..15 (|w| <= 7 s rounds to at most 7 away from 8),
    the largest-magnitude element maps to 1 or 15, and |W - deq| <= s/2."""
    for gs in (32, 128):
        W = synth.weight(256, 48, wid=0)
        codes, s16, z16 = o.quantize(W, gs, symmetric=True)
        K, N = W.shape
        G = K // gs
        s = s16.astype(np.float64)
        assert np.all(z16 == 8)
        Wg = W.astype(np.float64).reshape(G, gs, N)
        amax = np.abs(Wg).max(axis=1)
        target = amax / 7.0
        assert np.all(np.abs(s - target) <= target * 2.0 ** -11 * (1 + 2.0 ** -10))
        cg = codes.reshape(G, gs, N)
        assert cg.min() >= 1 and cg.max() <= 15
        am = np.abs(Wg).argmax(axis=1)
        top = np.take_along_axis(cg, am[:, None, :], axis=1)
        assert np.all((top == 1) | (top == 15))
        deq = o.dequant(codes, s16, z16, gs).astype(np.float64).reshape(G, gs, N)
        slack = np.abs(Wg) * 2.0 ** -22
        assert np.all(np.abs(Wg - deq) <= 0.5 * s[:, None, :] * (1 + 2.0 ** -10) + slack)


def pin_interleaved_words(o):
    """Interleaved layout, words worked out by hand: nibble p holds K offset
    (0, 2, 4, 6, 1, 3, 5, 7)[p] of its 8 K indices (even offsets low, odd offsets high)."""
    codes = np.zeros((8, 5), dtype=np.uint8)
    codes[:, 0] = np.arange(8)          # code k at K offset k -> nibbles 0,2,4,6,1,3,5,7 -> 0x75316420
    codes[1, 1] = 1                     # K offset 1 -> nibble 4 -> 0x00010000
    codes[7, 2] = 8                     # K offset 7 -> nibble 7 -> 0x80000000
    codes[2, 3] = 0xA                   # K offset 2 -> nibble 1 -> 0x000000A0
    codes[6, 4] = 0x3                   # K offset 6 -> nibble 3 -> 0x00003000
    words = o.pack(codes, "interleaved")
    expect = np.array([[0x75316420, 0x10000, -2**31, 0xA0, 0x3000]], dtype=np.int64)
    assert np.array_equal(words.astype(np.int64), expect), [hex(int(w) & 0xFFFFFFFF) for w in words[0]]
    assert np.array_equal(o.unpack(words, "interleaved"), codes)
    for K, N, seed in [(8, 3, 4), (128, 17, 5)]:
        c = synth.uniform_codes(K, N, seed)
        assert np.array_equal(o.unpack(o.pack(c, "interleaved"), "interleaved"), c)
    # same codes, other packing: the product is the linear layout's, exactly
    W = synth.weight_custom(256, 12, seed=9, std=0.02)
    x = synth.activations(3, 256, wid=6)
    ql, s, z = o.quantize_pack(W)
    qi, s2, z2 = o.quantize_pack(W, layout="interleaved")
    assert np.array_equal(s, s2) and np.array_equal(z, z2)
    assert not np.array_equal(ql, qi)
    assert np.array_equal(o.matmul(x, ql, s, z), o.matmul(x, qi, s, z, layout="interleaved"))


def pin_round_then_add_odd_zero(o):
    """Codes are rounded first and offset by the zero after: q = rne(w/s) + z.

    One group, s = 2**-6 exactly (min -3s, max 12s: (max - min)/15 = s) and zero
    rne(3) = 3, an odd zero, so the two orders differ on every half-way w/s. Worked by
    hand, w/s -> rne(w/s) + 3 (rne(w/s + 3) in brackets):
      -3 -> 0 (0), -1.5 -> -2 + 3 = 1 (rne(1.5) = 2), -0.5 -> -0 + 3 = 3 (rne(2.5) = 2),
      0.5 -> 0 + 3 = 3 (rne(3.5) = 4), 1.5 -> 2 + 3 = 5 (rne(4.5) = 4),
      2.5 -> 2 + 3 = 5 (rne(5.5) = 6), 12 -> 15 (15); the other rows hold 0 -> 3.
    Round-half-away codes would give 0.5 -> 4 and 2.5 -> 6 instead.
    """
    d = 2.0 ** -6
    ratios = [-3.0, -1.5, -0.5, 0.5, 1.5, 2.5, 12.0]
    W = np.zeros((128, 1), dtype=np.float32)
    W[:len(ratios), 0] = np.asarray(ratios) * d
    codes, s, z = o.quantize(W)
    assert s[0, 0] == np.float16(d) and z[0, 0] == 3, (s, z)
    expect = np.full(128, 3, dtype=np.uint8)
    expect[:len(ratios)] = [0, 1, 3, 3, 5, 5, 15]
    assert np.array_equal(codes[:, 0], expect), codes[:8, 0]
    # the dequantised values follow from the codes: (q - 3) * 2**-6
    deq = o.dequant(codes, s, z)[:len(ratios), 0]
    assert np.array_equal(deq, np.array([-3, -2, 0, 0, 2, 2, 12], dtype=np.float32) * np.float32(d))


def pin_zero_point_tie(o):
    """The zero point is rounded half to even: rne(-min/s) at exact ties.

    Three columns, each with scale 2**-6 exactly (max - min = 15 s):
      min -2.5s, max 12.5s: zero rne(2.5) = 2 (half-up or half-away: 3); codes of the
        min and max rne(-2.5) + 2 = 0 and rne(12.5) + 2 = 14;
      min -0.5s, max 14.5s: zero rne(0.5) = 0 (half-up: 1); codes 0 and rne(14.5) = 14;
      min -3.5s, max 11.5s: zero rne(3.5) = 4 (half-down or truncation: 3); codes
        rne(-3.5) + 4 = 0 and rne(11.5) + 4 = 16 -> clamped to 15.
    """
    d = 2.0 ** -6
    lo = [-2.5, -0.5, -3.5]
    W = np.zeros((128, 3), dtype=np.float32)
    for n, a in enumerate(lo):
        W[0, n] = a * d
        W[1, n] = (a + 15.0) * d
    codes, s, z = o.quantize(W)
    assert np.all(s[0] == np.float16(d)), s
    assert z[0].tolist() == [2.0, 0.0, 4.0], z
    assert codes[0].tolist() == [0, 0, 0] and codes[1].tolist() == [14, 14, 15], codes[:2]
    assert codes[2:].tolist() == [[2, 0, 4]] * 126


def pin_true_division(o):
    """w / scale is one correctly rounded fp32 division, not w times a rounded 1/scale.

    Asymmetric: scale 1070 * 2**-10 (an fp16 value; a group with min 0 and max 15 scale
    stores it exactly, zero 0) and w = 8025 * 2**-10 - 2**-21, one fp32 step below
    7.5 * scale. The exact quotient 7.5 - 2**-21 / scale lies nearer to the fp32 value
    7.5 - 2**-21 than to 7.5, so w / scale rounds below 7.5 and the code is 7; the
    reciprocal fl32(1 / scale) times w rounds to exactly 7.5, which half-even takes to 8.
    Symmetric: scale 141 * 2**-7 (max |w| = 7 scale) and w = 916.5 * 2**-7 + 2**-21, one
    step above 6.5 * scale: the quotient rounds above 6.5, code rne(6.5+) + 8 = 15 (and
    -w gives 1); the reciprocal route lands on exactly 6.5 and gives 14 (and 2).
    These values were found by a search over fp16 scales for a quotient within an fp32
    step of a half-way point; the reasoning above is what fixes the expected codes.
    """
    s_a = 1070 * 2.0 ** -10
    W = np.zeros((128, 1), dtype=np.float32)
    W[0, 0] = 15 * s_a
    W[1, 0] = np.float32(8025 * 2.0 ** -10) - np.float32(2.0 ** -21)
    codes, s, z = o.quantize(W)
    assert s[0, 0] == np.float16(s_a) and z[0, 0] == 0, (s, z)
    assert codes[0, 0] == 15 and codes[1, 0] == 7, codes[:2, 0]
    s_s = 141 * 2.0 ** -7
    W = np.zeros((128, 2), dtype=np.float32)
    W[0, :] = 7 * s_s
    w = np.float32(916.5 * 2.0 ** -7) + np.float32(2.0 ** -21)
    W[1, 0] = w
    W[1, 1] = -w
    codes, s, z = o.quantize(W, 128, symmetric=True)
    assert np.all(s[0] == np.float16(s_s)) and np.all(z == 8), (s, z)
    assert codes[0].tolist() == [15, 15] and codes[1].tolist() == [15, 1], codes[:2]


ALL_PINS = [pin_hand_words, pin_interleaved_words, pin_roundtrip, pin_exact_group, pin_exact_products,
            pin_multigroup, pin_bounds_random, pin_fsum, pin_dequant_fp16_rounding,
            pin_scale_rounding, pin_group_sizes, pin_symmetric_exact, pin_symmetric_bounds,
            pin_round_then_add_odd_zero, pin_zero_point_tie, pin_true_division]
