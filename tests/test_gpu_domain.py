"""GPU parity of every product kernel over the quantiser's whole supported domain.

The workload draw N(0, 0.02) keeps every zero point in about [4, 11]. These cases take the
weights where the unpack and dequantisation arithmetic is stressed ("Beating FP16 with
4-bit Weights", section "Code": the tests span shapes, group sizes and both kinds of
quantisation):
  * one-signed groups N(+1, 0.02) and N(-1, 0.02): zero points near -117 and +130;
  * wide groups N(-3, 5): scales near 2 and codes spread over 0..15;
  * subnormal fp16 scales (N(0, 3e-7)): every dequantised fp16 weight is subnormal;
  * hand-built packed weights with zero points anywhere in [-1024, 1024] (the ends
    included) and scales between 2**-12 and 2**-9;
  * an exact closed form: groups whose zero points are -1024 .. 1024 and whose scales are
    powers of two, where every product and partial sum is exact and y must be bit-exact.
Each case runs every kernel with its plan forced: the decode kernel with 16-, 32- and
64-column strips (without and with split-K, 1- and 4-step segments), the 128x128 LDS
tile, the register tile, and the async tile with 32/64- and 128-row work-groups, with and
without split-K; group sizes 32, 64, 128 and 256; linear and interleaved packing.

Two bars per output element. Let w' be the weight the kernel multiplies: the exact
(q - z) s for the decode kernel, which applies each group's scale to its fp32 partial sum,
and fp16_rne((q - z) s) for the prefill tiles, which stage fp16 weights as "The design"
dequantises them (both values come from the oracle: dequant and dequant_fp16), and let
y_w = x . w' in fp64.
  * The stated bar against the exact fp64 oracle, |y - y_ref| <= 1e-2 + 5e-3 |y_ref|,
    widened by |y_w - y_ref|: the deviation that the fp16 weights themselves cause, which
    is zero for the decode kernel. On these domains that deviation alone exceeds the bar
    (computed from the oracle on the CPU, K = 2048: 2.3x the bar for N(+1, 0.02), 10x for
    N(-3, 5), 1.7x for the far zero points), since each fp16 weight carries a relative
    error up to 2**-11 while |y| can be small by cancellation; on the workload's N(0, 0.02)
    weights it does not, and every other test holds the unwidened bar.
  * A bound derived from the arithmetic the kernel performs, which stays meaningful where
    y is tiny (subnormal scales): |y - y_w| <= 2K 2**-23 sum_k |x_k w'_k| + 2**-11 |y_w| +
    2**-25 (fp32 accumulation of exact products with at most 2K roundings, whatever the
    order, then one fp16 rounding of the output, subnormal outputs included).
"""
import numpy as np
import pytest

import oracle
import oracle_pins
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ATOL, RTOL = 1e-2, 5e-3
K = 2048
N = 328                       # a multiple of 8, not of 64 or 256: ragged strips and tiles


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import weight_only_bit_gemv_amd as L
    return L


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


# kernel configurations: (name, rows of M, forced plan, weights the kernel multiplies)
KERNELS = [
    ("skinny-c16", 37, dict(kernel=1, cols=16), "exact"),
    ("skinny-c16-seg1-w8", 5, dict(kernel=1, cols=16, kc=2, seg=1, waves=8), "exact"),
    ("skinny-c32-split4", 37, dict(kernel=1, cols=32, kc=4, waves=4), "exact"),
    ("skinny-c64-split2", 37, dict(kernel=1, cols=64, kc=8, waves=4), "exact"),
    ("lds-tile", 130, dict(kernel=2, tile=1), "fp16"),
    ("register-tile", 130, dict(kernel=2, tile=2), "fp16"),
    ("async-tile", 130, dict(kernel=2, tile=3, splits=1), "fp16"),
    ("async-tile-split4", 130, dict(kernel=2, tile=3, splits=4), "fp16"),
    ("async-tile-40rows-split2", 40, dict(kernel=2, tile=3, splits=2), "fp16"),
]
FORMATS = [(128, "linear"), (32, "interleaved"), (64, "linear"), (256, "interleaved")]
DOMAINS = ["one-signed N(+1,0.02)", "one-signed N(-1,0.02)", "wide N(-3,5)", "subnormal scales N(0,3e-7)",
           "zero points in [-1024,1024]"]

_W = {}


def weights(domain, g, layout):
    key = (domain, g, layout)
    if key in _W:
        return _W[key]
    if len(_W) > 8:
        _W.clear()
    seed = 20 + DOMAINS.index(domain)
    if domain == "zero points in [-1024,1024]":
        codes = synth.uniform_codes(K, N, seed)
        s, z = synth.scales_zeros_custom(K // g, N, seed)
        qw = oracle.pack(codes, layout)
    else:
        mean, std = {"one-signed N(+1,0.02)": (1.0, 0.02), "one-signed N(-1,0.02)": (-1.0, 0.02),
                     "wide N(-3,5)": (-3.0, 5.0), "subnormal scales N(0,3e-7)": (0.0, 3e-7)}[domain]
        qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed, std, mean), g, layout=layout)
    codes = oracle.unpack(qw, layout)
    w_exact = oracle.dequant(codes, s, z, g).astype(np.float64)
    w_fp16 = oracle.dequant_fp16(codes, s, z, g).astype(np.float64)
    _W[key] = (qw, s, z, {"exact": w_exact, "fp16": w_fp16})
    return _W[key]


def check(y_gpu, x, y_ref, w_kernel, what):
    y = y_gpu.detach().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    x64 = x.astype(np.float64)
    y_w = x64 @ w_kernel
    err = np.abs(y - y_ref)
    bar = ATOL + RTOL * np.abs(y_ref) + np.abs(y_w - y_ref)
    worst = np.unravel_index(np.argmax(err - bar), err.shape)
    assert np.all(err <= bar), (f"{what}: error {err[worst]:.3e} > {bar[worst]:.3e} at {worst} "
                                f"(y={y[worst]}, ref={y_ref[worst]}, y_w={y_w[worst]})")
    mag = np.abs(x64) @ np.abs(w_kernel)
    tight = 2 * K * 2.0 ** -23 * mag + 2.0 ** -11 * np.abs(y_w) + 2.0 ** -25
    e2 = np.abs(y - y_w)
    worst = np.unravel_index(np.argmax(e2 - tight), e2.shape)
    assert np.all(e2 <= tight), (f"{what}: derived bound exceeded at {worst}: |y - y_w| = {e2[worst]:.3e} > "
                                 f"{tight[worst]:.3e} (y={y[worst]:.6e}, y_w={y_w[worst]:.6e})")


@pytest.mark.parametrize("g,layout", FORMATS, ids=[f"g{g}-{l}" for g, l in FORMATS])
@pytest.mark.parametrize("name,M,plan,wkind", KERNELS, ids=[k[0] for k in KERNELS])
@pytest.mark.parametrize("domain", DOMAINS)
def test_domain_parity(lib, domain, name, M, plan, wkind, g, layout):
    qw, s, z, w = weights(domain, g, layout)
    pl = lib.w4a16_plan(M, N, K, group_size=g, **plan)
    print(f"\n[domain] {domain} {name} g={g} {layout} M={M} K={K} N={N} plan={pl}", flush=True)
    x = synth.activations(M, K, wid=10)
    y = lib.w4a16_matmul(dev(x), dev(qw), dev(s), dev(z), plan=plan, group_size=g, layout=layout)
    torch.cuda.synchronize()
    check(y, x, oracle.matmul(x, qw, s, z, g, layout=layout), w[wkind], f"{domain} {name} g={g} {layout}")


# exact closed form: zero points -1024 .. 1024, power-of-two scales -----------------------

CENTRES = [-500, 600, 8, -1000, 3, 1024, -1024, 12]
LOG2D = [-10, -11, -6, -12, -5, -13, -13, -4]


def _exact_case(g, layout):
    G = K // g
    centres = [CENTRES[i % 8] for i in range(G)]
    log2d = [LOG2D[i % 8] for i in range(G)]
    W = oracle_pins._exact_group_weight(K, 16, centres, log2d, g)
    qw, s, z = oracle.quantize_pack(W, g, layout=layout)
    assert np.array_equal(z.astype(np.float64), np.repeat(np.asarray(centres, np.float64)[:, None], 16, 1))
    x = np.zeros((3, K), dtype=np.float16)
    x[0] = 1
    x[1, 5] = 1
    x[2, K - 1] = 1
    n = np.arange(16)
    # y(ones): each group holds g/16 blocks of the residues 0..15, so it adds
    # (g/16) * (120 - 16 c) * 2**e; cycling the eight (c, e) pairs over 2048 rows gives
    # 2048/128 * (63.4375 - 37.03125 - 1 + 31.484375 + 18 - 15.8828125 + 16.1171875 - 36) / 2
    # = 78.25 for every group size
    expect = np.zeros((3, 16))
    expect[0] = 78.25
    expect[1] = (((5 + n) % 16) - centres[0]) * 2.0 ** log2d[0]
    expect[2] = (((K - 1 + n) % 16) - centres[-1]) * 2.0 ** log2d[-1]
    return qw, s, z, x, expect


@pytest.mark.parametrize("g,layout", FORMATS, ids=[f"g{g}-{l}" for g, l in FORMATS])
@pytest.mark.parametrize("name,M,plan,wkind", KERNELS, ids=[k[0] for k in KERNELS])
def test_far_zero_points_exact(lib, name, M, plan, wkind, g, layout):
    """Every product, partial sum and dequantised weight of this case is exactly
    representable (|q - z| <= 1039 times a power of two), so y must equal the hand sum."""
    qw, s, z, x, expect = _exact_case(g, layout)
    assert np.array_equal(oracle.matmul(x, qw, s, z, g, layout=layout), expect)
    print(f"\n[far zeros exact] {name} g={g} {layout}", flush=True)
    y = lib.w4a16_matmul(dev(x), dev(qw), dev(s), dev(z), plan=plan, group_size=g, layout=layout)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, expect), f"{name} g={g} {layout}: {got[:, :4]} vs {expect[:, :4]}"
