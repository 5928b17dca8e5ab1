"""GPU parity of the W4A8 path (E4M3 activations x 4-bit weights) against its oracle.

Bars: activation codes and row scales bit-exact (the quantiser's rounding is a decision the
GPU and the oracle take in the same fp32 arithmetic); y within |err| <= 1e-2 + 5e-3 |y_ref|
of the fp64 oracle on the same codes; repeated calls bitwise identical.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ATOL, RTOL = 1e-2, 5e-3


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import weight_only_bit_gemv_amd as L
    return L


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def check_y(y_gpu, y_ref, what=""):
    y = y_gpu.detach().cpu().numpy().astype(np.float64)
    assert y.shape == y_ref.shape
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y - y_ref)
    bound = ATOL + RTOL * np.abs(y_ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), f"{what}: max err {err.max():.3e} at {worst}, y={y[worst]} ref={y_ref[worst]}"


def block_sums(xq):
    """The oracle's block sums of the decoded codes, in the library's layout: fp32
    [K/128, M rounded up to 4], padding rows 0."""
    S = oracle.activation_block_sums(xq)
    out = np.zeros((S.shape[0], (xq.shape[0] + 3) // 4 * 4), dtype=np.float32)
    out[:, :xq.shape[0]] = S
    return out


def _activations(M, K, kind, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    if kind == "wide":
        x *= np.exp2(rng.integers(-12, 12, size=(M, 1)))             # rows of very different scale
    elif kind == "spiky":
        x[rng.random((M, K)) < 0.002] *= 300                           # a few large activations
    elif kind == "tiny":
        x *= 1e-6                                                       # fp16 subnormal range
    x = x.astype(np.float16)
    if M > 2:
        x[1] = 0                                                        # an all-zero row
    return x


QUANT_SHAPES = [(1, 128), (3, 4096), (17, 14336), (64, 2048), (130, 8192)]


@pytest.mark.parametrize("kind", ["normal", "wide", "spiky", "tiny"])
@pytest.mark.parametrize("M,K", QUANT_SHAPES, ids=[f"M{m}-K{k}" for m, k in QUANT_SHAPES])
def test_quantize_activations_bit_exact(lib, M, K, kind):
    print(f"\n[w4a8 quantise] {kind} M={M} K={K}", flush=True)
    x = _activations(M, K, kind, seed=M + K)
    xq, sx, xsum = lib.w4a8_quantize(dev(x))
    torch.cuda.synchronize()
    xq_ref, sx_ref = oracle.quantize_activations(x)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32)), "row scales differ"
    got = xq.cpu().numpy()
    bad = np.argwhere(got != xq_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0]}: {got[tuple(bad[0])]:#x} vs {xq_ref[tuple(bad[0])]:#x}"
    # block sums: fp32 sums of 128 exact values, within 128 * 2^-24 * sum |dec| of the exact sum
    S = oracle.activation_block_sums(xq_ref)
    mag = oracle.activation_block_sums(xq_ref & 0x7F)
    s_gpu = xsum.cpu().numpy()
    assert s_gpu.shape == (K // 128, (M + 3) // 4 * 4)
    assert np.all(np.abs(s_gpu[:, :M] - S) <= 128 * 2.0 ** -24 * mag), np.abs(s_gpu[:, :M] - S).max()
    assert np.all(s_gpu[:, M:] == 0)


MM_SHAPES = [(1, 128, 8), (3, 256, 104), (130, 384, 1416), (257, 1408, 264), (64, 768, 2056), (200, 128, 136),
             (511, 640, 520), (128, 4096, 256), (37, 2048, 1032)]


@pytest.mark.parametrize("layout", ["linear", "interleaved"])
@pytest.mark.parametrize("M,K,N", MM_SHAPES, ids=[f"M{m}-K{k}-N{n}" for m, k, n in MM_SHAPES])
def test_w4a8_matmul_matches_oracle(lib, M, K, N, layout):
    print(f"\n[w4a8 matmul] {layout} M={M} K={K} N={N}", flush=True)
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=900 + M, std=0.02), 128, False, layout)
    x = synth.activations(M, K, wid=9)
    xq, sx = oracle.quantize_activations(x)
    y = lib.w4a8_matmul(dev(xq), dev(sx), dev(block_sums(xq)), dev(qw), dev(s), dev(z), layout=layout)
    check_y(y, oracle.matmul_w4a8(xq, sx, qw, s, z, 128, layout), f"w4a8 {layout} M={M} K={K} N={N}")


@pytest.mark.parametrize("g,sym", [(128, True), (256, False), (256, True)])
@pytest.mark.parametrize("M,K,N", [(5, 512, 96), (140, 1024, 520), (64, 2048, 264)])
def test_w4a8_formats(lib, M, K, N, g, sym):
    print(f"\n[w4a8 format] g={g} sym={sym} M={M} K={K} N={N}", flush=True)
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=950 + M, std=0.02), g, sym)
    x = synth.activations(M, K, wid=9)
    xq, sx = oracle.quantize_activations(x)
    y = lib.w4a8_matmul(dev(xq), dev(sx), dev(block_sums(xq)), dev(qw), dev(s), dev(z), group_size=g)
    check_y(y, oracle.matmul_w4a8(xq, sx, qw, s, z, g), f"w4a8 g={g} sym={sym}")


FAR_ZERO_CASES = [
    # (M, K, N, forced splits (0: the library's), layout, group): every row-tile size (32, 64,
    # 128 rows), M not a multiple of 4 (padded block sums), ragged N and split-K
    (33, 512, 64, 0, "linear", 128),
    (7, 1024, 136, 1, "linear", 128),
    (150, 1024, 264, 4, "interleaved", 256),
    (130, 512, 520, 1, "linear", 128),
    (1, 2048, 72, 8, "interleaved", 128),
]


@pytest.mark.parametrize("M,K,N,splits,layout,g", FAR_ZERO_CASES)
def test_w4a8_zero_points_anywhere_in_the_domain(lib, M, K, N, splits, layout, g):
    """Zero points anywhere in [-1024, 1024] (|q - z| up to 1039, far beyond what an 8-bit
    weight operand holds) next to ordinary ones: q - z stays exact, through the block sums,
    with and without split-K."""
    print(f"\n[w4a8 far zeros] M={M} K={K} N={N} splits={splits} {layout} g={g}", flush=True)
    rng = np.random.default_rng((4, M, K, N))
    codes = rng.integers(0, 16, size=(K, N)).astype(np.uint8)
    zeros = rng.choice([-700.0, -449.0, -448.0, -300.0, -17.0, -5.0, -1.0, 8.0, 16.0, 17.0, 30.0, 463.0, 464.0,
                        600.0, 1024.0], size=(K // g, N)).astype(np.float16)
    zeros[:, ::3] = 7.0                                     # whole wavefronts with no far zero point
    scales = (rng.random((K // g, N)) * 2e-4 + 1e-5).astype(np.float16)
    qw = oracle.pack(codes, layout=layout)
    x = synth.activations(M, K, wid=9)
    xq, sx = oracle.quantize_activations(x)
    y = lib.w4a8_matmul(dev(xq), dev(sx), dev(block_sums(xq)), dev(qw), dev(scales), dev(zeros), group_size=g,
                        layout=layout, splits=splits)
    check_y(y, oracle.matmul_w4a8(xq, sx, qw, scales, zeros, g, layout), "w4a8 far zero points")


def test_w4a8_end_to_end_and_repeatable(lib):
    """Quantiser and product on the device against the oracle's, then the same call again."""
    M, K, N = 300, 2048, 1032
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=77, std=0.02))
    x = _activations(M, K, "spiky", seed=5)
    xq, sx, xsum = lib.w4a8_quantize(dev(x))
    args = [dev(qw), dev(s), dev(z)]
    y = lib.w4a8_matmul(xq, sx, xsum, *args).clone()
    xq_ref, sx_ref = oracle.quantize_activations(x)
    check_y(y, oracle.matmul_w4a8(xq_ref, sx_ref, qw, s, z), "w4a8 end to end")
    for _ in range(3):
        y2 = lib.w4a8_matmul(xq, sx, xsum, *args)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


PREFILL = [(2048, 8192, 28672), (512, 28672, 8192), (128, 8192, 8192), (32, 8192, 28672), (64, 28672, 8192)]


@pytest.mark.parametrize("M,K,N", PREFILL, ids=[f"M{m}-K{k}-N{n}" for m, k, n in PREFILL])
def test_w4a8_prefill_shapes_sampled(lib, M, K, N):
    """The prefill workload's shapes at full size, checked on sampled columns (M = 32 and 64
    run the 32- and 64-row work-group tiles)."""
    wid = synth.WORKLOADS["prefill"]["wid"]
    print(f"\n[w4a8 prefill] M={M} K={K} N={N}", flush=True)
    qw, s, z = oracle.quantize_pack(synth.weight(K, N, wid=wid))
    x = synth.activations(M, K, wid=wid)
    xq, sx, xsum = lib.w4a8_quantize(dev(x))
    y = lib.w4a8_matmul(xq, sx, xsum, dev(qw), dev(s), dev(z))
    xq_ref, sx_ref = oracle.quantize_activations(x)
    cols = np.unique(np.concatenate([np.arange(0, N, max(1, N // 40)), [N - 1]]))
    y_ref = oracle.matmul_w4a8(xq_ref, sx_ref, qw[:, cols], s[:, cols], z[:, cols])
    check_y(y[:, torch.from_numpy(cols).to(DEV)], y_ref, f"w4a8 prefill M={M} K={K} N={N}")


SPLITS = [(130, 1024, 520, 2), (257, 2048, 264, 4), (64, 4096, 256, 8), (3, 768, 1032, 3), (200, 14336, 1416, 7),
          (128, 256, 2056, 2), (70, 8192, 512, 0), (1, 4096, 4096, 0)]


@pytest.mark.parametrize("layout", ["linear", "interleaved"])
@pytest.mark.parametrize("M,K,N,splits", SPLITS, ids=[f"M{m}-K{k}-N{n}-S{s}" for m, k, n, s in SPLITS])
def test_w4a8_split_k(lib, M, K, N, splits, layout):
    print(f"\n[w4a8 split-K] S={splits} {layout} M={M} K={K} N={N}", flush=True)
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=990 + M, std=0.02), 128, False, layout)
    x = synth.activations(M, K, wid=9)
    xq, sx = oracle.quantize_activations(x)
    args = [dev(xq), dev(sx), dev(block_sums(xq)), dev(qw), dev(s), dev(z)]
    y = lib.w4a8_matmul(*args, layout=layout, splits=splits).clone()
    check_y(y, oracle.matmul_w4a8(xq, sx, qw, s, z, 128, layout), f"w4a8 split-K S={splits}")
    for _ in range(2):                                   # same bits again: counters were reset
        assert torch.equal(lib.w4a8_matmul(*args, layout=layout, splits=splits).view(torch.int16), y.view(torch.int16))


def test_w4a8_split_k_shares_counters_with_w4a16(lib):
    """W4A8 and W4A16 split-K calls alternate on one stream: each returns the arrival
    counters to zero for the other."""
    M, K, N = 96, 4096, 1024
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=3, std=0.02))
    x = synth.activations(M, K, wid=9)
    xq, sx = oracle.quantize_activations(x)
    a8 = [dev(xq), dev(sx), dev(block_sums(xq)), dev(qw), dev(s), dev(z)]
    a16 = [dev(x), dev(qw), dev(s), dev(z)]
    ref8 = oracle.matmul_w4a8(xq, sx, qw, s, z)
    ref16 = oracle.matmul(x, qw, s, z)
    for rep in range(3):
        check_y(lib.w4a8_matmul(*a8, splits=4), ref8, f"w4a8 rep {rep}")
        check_y(lib.w4a16_matmul(*a16, plan=dict(kernel=2, tile=3, splits=3)), ref16, f"w4a16 rep {rep}")


@pytest.mark.parametrize("layout", ["linear", "interleaved"])
@pytest.mark.parametrize("M,K,N,splits", [(70, 1280, 264, 3), (200, 2560, 520, 4), (5, 768, 136, 2)],
                         ids=["M70-K1280-S3", "M200-K2560-S4", "M5-K768-S2"])
def test_w4a8_split_k_groups_of_256(lib, M, K, N, splits, layout):
    """Groups of 256 rows span two 128-row stages; a split may start in the middle of a
    group, and both halves still take that group's scale."""
    print(f"\n[w4a8 split-K g=256] S={splits} {layout} M={M} K={K} N={N}", flush=True)
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=1200 + M, std=0.02), 256, False, layout)
    x = synth.activations(M, K, wid=9)
    xq, sx = oracle.quantize_activations(x)
    y = lib.w4a8_matmul(dev(xq), dev(sx), dev(block_sums(xq)), dev(qw), dev(s), dev(z), group_size=256, layout=layout, splits=splits)
    check_y(y, oracle.matmul_w4a8(xq, sx, qw, s, z, 256, layout), f"w4a8 g=256 split-K S={splits}")
