"""GPU parity: libw4a16.so against the oracle on the same seeded inputs (needs an MI355X).

Inputs come from synth.py and are quantised and packed by the oracle; nothing the GPU
computes feeds an expected value. Bars:
  * codes and fp16 dequantised weights: bit-exact (fp16_rne of the oracle's exact value);
  * y: |y_gpu - y_ref| <= 1e-2 + 5e-3 * |y_ref| per element (y_ref in fp64);
  * repeated calls: bitwise identical.
Full-size shapes whose oracle would be slow are checked on sampled columns (all rows),
with the kernel launched at its full size.
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


_QCACHE = {}


def quantised(K, N, wid, layer=0):
    key = (K, N, wid, layer)
    if key not in _QCACHE:
        _QCACHE.clear() if len(_QCACHE) > 6 else None
        W = synth.weight(K, N, wid=wid, layer=layer)
        _QCACHE[key] = oracle.quantize_pack(W)
    return _QCACHE[key]


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def check_y(y_gpu, y_ref, what=""):
    y = y_gpu.detach().cpu().numpy().astype(np.float64)
    assert y.shape == y_ref.shape
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y - y_ref)
    bound = ATOL + RTOL * np.abs(y_ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (f"{what}: max err {err.max():.3e} at {worst}, "
                                  f"y={y[worst]:.6f} ref={y_ref[worst]:.6f}")
    return float(err.max())


def run(lib, x, qw, s, z, plan=None, y=None, stream=None, group_size=128, layout="linear"):
    out = lib.w4a16_matmul(dev(x) if isinstance(x, np.ndarray) else x,
                           dev(qw) if isinstance(qw, np.ndarray) else qw,
                           dev(s) if isinstance(s, np.ndarray) else s,
                           dev(z) if isinstance(z, np.ndarray) else z,
                           y=y, plan=plan, stream=stream, group_size=group_size, layout=layout)
    torch.cuda.synchronize()
    return out


# ---------------------------------------------------------------------------------------
# dequant hook: bit-exact codes and fp16 weights

_DQ = {}


def _dequant_inputs():
    if _DQ:
        return _DQ
    cases = _DQ
    cases.update({
        "4096x4096 N(0,0.02)": quantised(4096, 4096, 0),
        "768x2048 N(0,0.02)": quantised(768, 2048, 2),
        "one-signed N(1,0.02)": oracle.quantize_pack(synth.weight_custom(256, 64, 1, 0.02, 1.0)),
        "wide N(-3,5)": oracle.quantize_pack(synth.weight_custom(256, 64, 2, 5.0, -3.0)),
        "subnormal scales": oracle.quantize_pack(synth.weight_custom(256, 64, 3, 3e-7, 0.0)),
    })
    codes = synth.uniform_codes(384, 100, seed=9)
    s = np.full((3, 100), 1 + 3 * 2.0 ** -10, dtype=np.float16)   # fp16 product ties
    z = np.full((3, 100), 8, dtype=np.float16)
    z[1] = -1000
    z[2] = 1000
    cases["uniform codes, tie scale, extreme zeros"] = (oracle.pack(codes), s, z)
    return cases


DEQUANT_CASES = ["4096x4096 N(0,0.02)", "768x2048 N(0,0.02)", "one-signed N(1,0.02)",
                 "wide N(-3,5)", "subnormal scales", "uniform codes, tie scale, extreme zeros"]


@pytest.mark.parametrize("name", DEQUANT_CASES)
def test_dequant_bit_exact(lib, name):
    qw, s, z = _dequant_inputs()[name]
    print(f"\n[dequant] {name} K={qw.shape[0] * 8} N={qw.shape[1]}", flush=True)
    c, w = lib.w4a16_dequant(dev(qw), dev(s), dev(z))
    torch.cuda.synchronize()
    codes_ref = oracle.unpack(qw)
    w_ref = oracle.dequant_fp16(codes_ref, s, z)
    assert np.array_equal(c.cpu().numpy(), codes_ref)
    got = w.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), w_ref.view(np.uint16)), \
        f"{np.count_nonzero(got.view(np.uint16) != w_ref.view(np.uint16))} fp16 weights differ"


# ---------------------------------------------------------------------------------------
# matmul against the oracle on every decode / MoE workload shape (full outputs)

DECODE = [("gemv_4096", m, k, n) for (m, k, n) in synth.WORKLOADS["gemv_4096"]["shapes"]] + \
         [("decode_sweep", m, k, n) for (m, k, n) in synth.WORKLOADS["decode_sweep"]["shapes"]] + \
         [("moe_expert", m, k, n) for (m, k, n) in synth.WORKLOADS["moe_expert"]["shapes"]]


@pytest.mark.parametrize("wl,M,K,N", DECODE, ids=[f"{w}-M{m}-K{k}-N{n}" for w, m, k, n in DECODE])
def test_matmul_decode_shapes(lib, wl, M, K, N):
    wid = synth.WORKLOADS[wl]["wid"]
    print(f"\n[matmul] {wl} M={M} K={K} N={N} plan={lib.w4a16_plan(M, N, K)}", flush=True)
    qw, s, z = quantised(K, N, wid)
    x = synth.activations(M, K, wid=wid)
    y = run(lib, x, qw, s, z)
    check_y(y, oracle.matmul(x, qw, s, z), f"{wl} M={M} K={K} N={N}")


# ---------------------------------------------------------------------------------------
# prefill-sized and 7B-chain shapes: full-size launches, sampled columns

def _sample_cols(N, count=160, seed=0):
    rng = np.random.default_rng((5, N, seed))
    cols = rng.choice(N, size=min(count, N), replace=False)
    return np.unique(np.concatenate([cols, [0, 1, N - 2, N - 1]]))


PREFILL = synth.WORKLOADS["prefill"]["shapes"]


@pytest.mark.parametrize("M,K,N", PREFILL, ids=[f"M{m}-K{k}-N{n}" for m, k, n in PREFILL])
def test_matmul_prefill_shapes_sampled(lib, M, K, N):
    wid = synth.WORKLOADS["prefill"]["wid"]
    print(f"\n[matmul] prefill M={M} K={K} N={N} plan={lib.w4a16_plan(M, N, K)}", flush=True)
    qw, s, z = quantised(K, N, wid)
    x = synth.activations(M, K, wid=wid)
    y = run(lib, x, qw, s, z)
    cols = _sample_cols(N)
    y_ref = oracle.matmul(x, qw[:, cols], s[:, cols], z[:, cols])
    check_y(y[:, torch.from_numpy(cols).to(DEV)], y_ref, f"prefill M={M} K={K} N={N}")


def test_chain_layer_in_one_stream(lib):
    """One transformer layer of the 7B-shaped decode chain, back to back on one stream."""
    wid = synth.WORKLOADS["decode_chain_7b"]["wid"]
    outs = []
    for name, K, N in synth.CHAIN_7B_LAYER:
        qw, s, z = quantised(K, N, wid, layer=0)
        x = synth.activations(1, K, wid=wid)
        print(f"\n[chain] {name} K={K} N={N}", flush=True)
        outs.append((name, x, (qw, s, z),
                     lib.w4a16_matmul(dev(x), dev(qw), dev(s), dev(z))))
    torch.cuda.synchronize()
    for name, x, (qw, s, z), y in outs:
        check_y(y, oracle.matmul(x, qw, s, z), f"chain {name}")


def test_chain_lm_head_sampled(lib):
    wid = synth.WORKLOADS["decode_chain_7b"]["wid"]
    _, K, N = synth.CHAIN_7B_LM_HEAD
    print(f"\n[chain] lm_head K={K} N={N} plan={lib.w4a16_plan(1, N, K)}", flush=True)
    W = synth.weight(K, N, wid=wid, layer=0)
    qw, s, z = oracle.quantize_pack(W)
    del W
    x = synth.activations(1, K, wid=wid)
    y = run(lib, x, qw, s, z)
    cols = _sample_cols(N, 512)
    y_ref = oracle.matmul(x, qw[:, cols], s[:, cols], z[:, cols])
    check_y(y[:, torch.from_numpy(cols).to(DEV)], y_ref, "lm_head")


# Projection shapes of other common decoder configurations, each with a plan of its own in
# the dispatcher's table (narrow key/value projections; 11008-, 13824- and 18944-wide
# feed-forward layers; their transposes; one GPU's column share of the 7B-shaped
# projections over 8 GPUs): full-size launches with the plan the dispatcher
# picks for one M of each of its buckets (1, 2..4, 5..16; ragged M pads the MFMA rows),
# checked on sampled columns. Two shapes outside the table exercise the rule for the others.
DECODER_KN = [(4096, 512), (4096, 1024), (5120, 1024), (8192, 1024), (16384, 1024), (2048, 512),
              (2048, 2048), (4096, 2048), (8192, 2048), (1024, 4096), (6144, 4096), (8192, 4096),
              (11008, 4096), (4096, 6144), (4096, 8192), (2048, 8192), (5120, 5120), (13824, 5120),
              (18944, 3584), (4096, 11008), (5120, 13824), (3584, 18944),
              (4096, 1792), (14336, 512), (4096, 16032),
              (7168, 1024), (2560, 10240)]
DECODER_SHAPES = [(m, k, n) for (k, n) in DECODER_KN for m in (1, 3, 11)]


@pytest.mark.parametrize("M,K,N", DECODER_SHAPES, ids=[f"M{m}-K{k}-N{n}" for m, k, n in DECODER_SHAPES])
def test_matmul_decoder_shapes_sampled(lib, M, K, N):
    wid = synth.WORKLOADS["decode_chain_7b"]["wid"]
    print(f"\n[matmul] decoder M={M} K={K} N={N} plan={lib.w4a16_plan(M, N, K)}", flush=True)
    qw, s, z = quantised(K, N, wid)
    x = synth.activations(M, K, wid=wid)
    y = run(lib, x, qw, s, z)
    cols = _sample_cols(N)
    y_ref = oracle.matmul(x, qw[:, cols], s[:, cols], z[:, cols])
    check_y(y[:, torch.from_numpy(cols).to(DEV)], y_ref, f"decoder M={M} K={K} N={N}")


# ---------------------------------------------------------------------------------------
# ragged edges, every plan, determinism, streams, overwrite

RAGGED = [(1, 128, 4), (3, 128, 100), (17, 384, 1412), (33, 256, 68), (65, 512, 260),
          (100, 1408, 196), (5, 768, 2052), (16, 128, 64), (64, 256, 8)]


@pytest.mark.parametrize("M,K,N", RAGGED, ids=[f"M{m}-K{k}-N{n}" for m, k, n in RAGGED])
def test_matmul_ragged(lib, M, K, N):
    print(f"\n[ragged] M={M} K={K} N={N} plan={lib.w4a16_plan(M, N, K)}", flush=True)
    W = synth.weight_custom(K, N, seed=M, std=0.02)
    qw, s, z = oracle.quantize_pack(W)
    x = synth.activations(M, K, wid=7)
    check_y(run(lib, x, qw, s, z), oracle.matmul(x, qw, s, z), f"ragged M={M} K={K} N={N}")


def _plan_is_built(plan, M, N, K):
    """Whether the library accepts a forced plan (host-side check, no GPU needed)."""
    import weight_only_bit_gemv_amd as L
    try:
        L.w4a16_plan(M, N, K, **plan)
        return True
    except L.W4A16Error:
        return False


PLAN_MKN = (37, 1024, 320)
_SEG_KC = {1: (1, 2, 4), 2: (2, 4, 8), 4: (4, 8, 16), 8: (8, 16, 32)}
PLANS = [p for p in (dict(kernel=1, kc=kc, row_tiles=rt, waves=w, cols=c, seg=sg)
                     for c in (16, 32, 64) for sg in (1, 2, 4, 8) for kc in _SEG_KC[sg]
                     for rt in (1, 2, 3, 4) for w in (4, 8, 16))
         if _plan_is_built(p, PLAN_MKN[0], PLAN_MKN[2], PLAN_MKN[1])]
_PLAN_CASE = {}


def _plan_case():
    if not _PLAN_CASE:
        M, K, N = PLAN_MKN
        W = synth.weight_custom(K, N, seed=11, std=0.02)
        qw, s, z = oracle.quantize_pack(W)
        x = synth.activations(M, K, wid=8)
        _PLAN_CASE.update(x=x, w=(qw, s, z), dev=[dev(x), dev(qw), dev(s), dev(z)],
                          ref=oracle.matmul(x, qw, s, z))
    return _PLAN_CASE


@pytest.mark.parametrize("plan", PLANS, ids=[f"c{p['cols']}-seg{p['seg']}-kc{p['kc']}-rt{p['row_tiles']}"
                                              f"-w{p['waves']}" for p in PLANS])
def test_matmul_every_skinny_plan(lib, plan):
    """Every built skinny configuration (strip width, segment, K-steps, row tiles, waves)
    on one ragged shape: M = 37 spans three 16-row tiles, N = 320 is not a multiple of 64."""
    M, K, N = PLAN_MKN
    print(f"\n[plan] {plan} M={M} K={K} N={N}", flush=True)
    c = _plan_case()
    check_y(run(lib, *c["dev"], plan=plan), c["ref"], f"plan {plan}")


@pytest.mark.parametrize("cols", [16, 32])
@pytest.mark.parametrize("M,K,N", RAGGED, ids=[f"M{m}-K{k}-N{n}" for m, k, n in RAGGED])
def test_matmul_ragged_narrow_strips(lib, M, K, N, cols):
    """16- and 32-column strips (4- and 8-byte weight loads) on the ragged shapes."""
    plan = dict(kernel=lib.W4A16_KERNEL_SKINNY, cols=cols)
    print(f"\n[ragged narrow] M={M} K={K} N={N} plan={lib.w4a16_plan(M, N, K, **plan)}", flush=True)
    W = synth.weight_custom(K, N, seed=M, std=0.02)
    qw, s, z = oracle.quantize_pack(W)
    x = synth.activations(M, K, wid=7)
    check_y(run(lib, x, qw, s, z, plan=plan), oracle.matmul(x, qw, s, z),
            f"ragged cols={cols} M={M} K={K} N={N}")


PREFILL_FORCED = [(1, 128, 4), (3, 256, 100), (130, 384, 1412), (257, 1408, 260), (64, 768, 2052),
                  (128, 4096, 256), (200, 128, 132), (129, 2048, 1408)]


@pytest.mark.parametrize("M,K,N", PREFILL_FORCED, ids=[f"M{m}-K{k}-N{n}" for m, k, n in PREFILL_FORCED])
def test_matmul_prefill_kernel_forced(lib, M, K, N):
    print(f"\n[prefill forced] M={M} K={K} N={N}", flush=True)
    W = synth.weight_custom(K, N, seed=100 + M, std=0.02)
    qw, s, z = oracle.quantize_pack(W)
    x = synth.activations(M, K, wid=9)
    check_y(run(lib, x, qw, s, z, plan=dict(kernel=lib.W4A16_KERNEL_PREFILL, tile=lib.W4A16_TILE_LDS)),
            oracle.matmul(x, qw, s, z), f"prefill forced M={M} K={K} N={N}")


# ---------------------------------------------------------------------------------------
# group sizes 32 / 64 / 256 and the symmetric (+8 zero point) quantiser

FORMATS = [(32, False), (64, False), (256, False), (32, True), (128, True)]
FMT_IDS = [f"g{g}{'-sym' if sym else ''}" for g, sym in FORMATS]


@pytest.mark.parametrize("g,sym", FORMATS, ids=FMT_IDS)
def test_dequant_bit_exact_formats(lib, g, sym):
    W = synth.weight_custom(768, 200, seed=g, std=0.02)
    qw, s, z = oracle.quantize_pack(W, g, sym)
    print(f"\n[dequant] g={g} sym={sym}", flush=True)
    c, w = lib.w4a16_dequant(dev(qw), dev(s), dev(z), group_size=g)
    torch.cuda.synchronize()
    codes_ref = oracle.unpack(qw)
    assert np.array_equal(c.cpu().numpy(), codes_ref)
    w_ref = oracle.dequant_fp16(codes_ref, s, z, g)
    assert np.array_equal(w.cpu().numpy().view(np.uint16), w_ref.view(np.uint16))


FMT_SHAPES = [(1, 4096, 4096), (5, 4096, 14336), (16, 14336, 4096), (1, 2048, 1408), (3, 1536, 2048)]


@pytest.mark.parametrize("g,sym", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("M,K,N", FMT_SHAPES, ids=[f"M{m}-K{k}-N{n}" for m, k, n in FMT_SHAPES])
def test_matmul_formats_decode(lib, M, K, N, g, sym):
    print(f"\n[format] g={g} sym={sym} M={M} K={K} N={N} "
          f"plan={lib.w4a16_plan(M, N, K, group_size=g)}", flush=True)
    qw, s, z = oracle.quantize_pack(synth.weight(K, N, wid=0), g, sym)
    x = synth.activations(M, K, wid=0)
    check_y(run(lib, x, qw, s, z, group_size=g), oracle.matmul(x, qw, s, z, g),
            f"g={g} sym={sym} M={M} K={K} N={N}")


def _fmt_plans():
    out = []
    M, K, N = PLAN_MKN
    import weight_only_bit_gemv_amd as L
    for g in (32, 64, 256):
        for c in (16, 32, 64):
            for sg in (1, 2, 4):
                for kc in _SEG_KC[sg][:2]:
                    for rt in (1, 3 if c == 64 else 2):
                        for w in (4, 8):
                            p = dict(kernel=1, kc=kc, row_tiles=rt, waves=w, cols=c, seg=sg)
                            try:
                                L.w4a16_plan(M, N, K, group_size=g, **p)
                            except L.W4A16Error:
                                continue
                            out.append((g, p))
    return out


FMT_PLANS = _fmt_plans()
_FMT_CASE = {}


@pytest.mark.parametrize("g,plan", FMT_PLANS,
                         ids=[f"g{g}-c{p['cols']}-seg{p['seg']}-kc{p['kc']}-rt{p['row_tiles']}-w{p['waves']}"
                              for g, p in FMT_PLANS])
def test_matmul_every_segment_per_group_size(lib, g, plan):
    """Segments of 1, 2 and 4 K-steps over groups of 1, 2, 4 and 8 K-steps (each segment
    inside one group, or holding 2 or 4 whole groups)."""
    M, K, N = PLAN_MKN
    if g not in _FMT_CASE:
        W = synth.weight_custom(K, N, seed=12, std=0.02)
        qw, s, z = oracle.quantize_pack(W, g)
        x = synth.activations(M, K, wid=8)
        _FMT_CASE[g] = ([dev(x), dev(qw), dev(s), dev(z)], oracle.matmul(x, qw, s, z, g))
    args, ref = _FMT_CASE[g]
    print(f"\n[format plan] g={g} {plan}", flush=True)
    check_y(run(lib, *args, plan=plan, group_size=g), ref, f"g={g} plan {plan}")


FMT_PREFILL = [(3, 256, 100), (130, 512, 1412), (257, 1536, 260), (128, 4096, 256)]


@pytest.mark.parametrize("g,sym", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("M,K,N", FMT_PREFILL, ids=[f"M{m}-K{k}-N{n}" for m, k, n in FMT_PREFILL])
def test_matmul_formats_prefill_forced(lib, M, K, N, g, sym):
    print(f"\n[format prefill] g={g} sym={sym} M={M} K={K} N={N}", flush=True)
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=200 + M, std=0.02), g, sym)
    x = synth.activations(M, K, wid=9)
    check_y(run(lib, x, qw, s, z, plan=dict(kernel=lib.W4A16_KERNEL_PREFILL, tile=lib.W4A16_TILE_LDS),
                group_size=g),
            oracle.matmul(x, qw, s, z, g), f"prefill g={g} sym={sym} M={M} K={K} N={N}")


PREFILL_RB = PREFILL_FORCED + [(511, 640, 516), (256, 1536, 260)]


@pytest.mark.parametrize("M,K,N", PREFILL_RB, ids=[f"M{m}-K{k}-N{n}" for m, k, n in PREFILL_RB])
def test_matmul_prefill_register_b_tile(lib, M, K, N):
    """The 128 x 256 register tile (weights dequantised in registers): ragged M and N, N not
    a multiple of 256 or of 64."""
    print(f"\n[prefill register tile] M={M} K={K} N={N}", flush=True)
    W = synth.weight_custom(K, N, seed=300 + M, std=0.02)
    qw, s, z = oracle.quantize_pack(W)
    x = synth.activations(M, K, wid=9)
    check_y(run(lib, x, qw, s, z, plan=dict(kernel=lib.W4A16_KERNEL_PREFILL, tile=lib.W4A16_TILE_REGISTER_B)),
            oracle.matmul(x, qw, s, z), f"prefill register tile M={M} K={K} N={N}")


@pytest.mark.parametrize("g,sym", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("M,K,N", FMT_PREFILL, ids=[f"M{m}-K{k}-N{n}" for m, k, n in FMT_PREFILL])
def test_matmul_formats_prefill_register_b_tile(lib, M, K, N, g, sym):
    print(f"\n[format prefill register tile] g={g} sym={sym} M={M} K={K} N={N}", flush=True)
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=400 + M, std=0.02), g, sym)
    x = synth.activations(M, K, wid=9)
    check_y(run(lib, x, qw, s, z, plan=dict(kernel=lib.W4A16_KERNEL_PREFILL, tile=lib.W4A16_TILE_REGISTER_B), group_size=g),
            oracle.matmul(x, qw, s, z, g), f"prefill register tile g={g} sym={sym} M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", PREFILL, ids=[f"M{m}-K{k}-N{n}" for m, k, n in PREFILL])
def test_matmul_prefill_shapes_register_b_tile_sampled(lib, M, K, N):
    wid = synth.WORKLOADS["prefill"]["wid"]
    print(f"\n[prefill register tile] M={M} K={K} N={N}", flush=True)
    qw, s, z = quantised(K, N, wid)
    x = synth.activations(M, K, wid=wid)
    y = run(lib, x, qw, s, z, plan=dict(kernel=lib.W4A16_KERNEL_PREFILL, tile=lib.W4A16_TILE_REGISTER_B))
    cols = _sample_cols(N)
    y_ref = oracle.matmul(x, qw[:, cols], s[:, cols], z[:, cols])
    check_y(y[:, torch.from_numpy(cols).to(DEV)], y_ref, f"prefill register tile M={M} K={K} N={N}")


PREFILL_ASYNC = [(1, 128, 8), (3, 256, 104), (130, 384, 1416), (257, 1408, 264), (64, 768, 2056),
                 (128, 4096, 256), (200, 128, 136), (129, 2048, 1408), (511, 640, 520), (256, 1536, 264),
                 (32, 512, 264), (17, 2048, 136), (40, 1024, 520), (65, 640, 264), (96, 1024, 136),
                 (90, 2048, 520)]   # 32-, 64- and 128-row tiles


@pytest.mark.parametrize("M,K,N", PREFILL_ASYNC, ids=[f"M{m}-K{k}-N{n}" for m, k, n in PREFILL_ASYNC])
def test_matmul_prefill_async_tile(lib, M, K, N):
    """The 128 x 256 tile fed by direct global-to-LDS loads (three-stage ring): ragged M and
    N (multiples of 8, not of 256), K from 2 to 64 stages (fewer stages than ring slots
    included)."""
    print(f"\n[prefill async tile] M={M} K={K} N={N}", flush=True)
    W = synth.weight_custom(K, N, seed=500 + M, std=0.02)
    qw, s, z = oracle.quantize_pack(W)
    x = synth.activations(M, K, wid=9)
    check_y(run(lib, x, qw, s, z, plan=dict(kernel=lib.W4A16_KERNEL_PREFILL, tile=lib.W4A16_TILE_ASYNC)),
            oracle.matmul(x, qw, s, z), f"prefill async tile M={M} K={K} N={N}")


FMT_ASYNC = [(3, 256, 104), (130, 512, 1416), (257, 1536, 264), (128, 4096, 256)]


@pytest.mark.parametrize("g,sym", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("M,K,N", FMT_ASYNC, ids=[f"M{m}-K{k}-N{n}" for m, k, n in FMT_ASYNC])
def test_matmul_formats_prefill_async_tile(lib, M, K, N, g, sym):
    print(f"\n[format prefill async tile] g={g} sym={sym} M={M} K={K} N={N}", flush=True)
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=600 + M, std=0.02), g, sym)
    x = synth.activations(M, K, wid=9)
    check_y(run(lib, x, qw, s, z, plan=dict(kernel=lib.W4A16_KERNEL_PREFILL, tile=lib.W4A16_TILE_ASYNC),
                group_size=g),
            oracle.matmul(x, qw, s, z, g), f"prefill async tile g={g} sym={sym} M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", PREFILL, ids=[f"M{m}-K{k}-N{n}" for m, k, n in PREFILL])
def test_matmul_prefill_shapes_async_tile_sampled(lib, M, K, N):
    wid = synth.WORKLOADS["prefill"]["wid"]
    print(f"\n[prefill async tile] M={M} K={K} N={N}", flush=True)
    qw, s, z = quantised(K, N, wid)
    x = synth.activations(M, K, wid=wid)
    y = run(lib, x, qw, s, z, plan=dict(kernel=lib.W4A16_KERNEL_PREFILL, tile=lib.W4A16_TILE_ASYNC))
    cols = _sample_cols(N)
    y_ref = oracle.matmul(x, qw[:, cols], s[:, cols], z[:, cols])
    check_y(y[:, torch.from_numpy(cols).to(DEV)], y_ref, f"prefill async tile M={M} K={K} N={N}")


def test_prefill_async_tile_repeated_calls_bitwise(lib):
    """Same inputs, same bits: the ring's waits leave no stage to chance."""
    M, K, N = 300, 2048, 1032
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=7, std=0.02))
    x = synth.activations(M, K, wid=9)
    args = [dev(x), dev(qw), dev(s), dev(z)]
    plan = dict(kernel=lib.W4A16_KERNEL_PREFILL, tile=lib.W4A16_TILE_ASYNC)
    a = lib.w4a16_matmul(*args, plan=plan).clone()
    for _ in range(5):
        b = lib.w4a16_matmul(*args, plan=plan)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    check_y(a, oracle.matmul(x, qw, s, z), "async repeated")


# ---------------------------------------------------------------------------------------
# split-K on the async prefill tile

SPLIT_CASES = [(130, 1024, 520, 2), (257, 2048, 264, 4), (64, 4096, 256, 8), (3, 768, 1032, 3),
               (200, 14336, 1416, 7), (128, 256, 2056, 2)]


@pytest.mark.parametrize("layout", ["linear", "interleaved"])
@pytest.mark.parametrize("g", [32, 128])
@pytest.mark.parametrize("M,K,N,splits", SPLIT_CASES, ids=[f"M{m}-K{k}-N{n}-S{s}" for m, k, n, s in SPLIT_CASES])
def test_matmul_prefill_async_split_k(lib, M, K, N, splits, g, layout):
    plan = dict(kernel=lib.W4A16_KERNEL_PREFILL, tile=lib.W4A16_TILE_ASYNC, splits=splits)
    print(f"\n[prefill split-K] {lib.w4a16_plan(M, N, K, group_size=g, **plan)} g={g} {layout} "
          f"M={M} K={K} N={N}", flush=True)
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=800 + M, std=0.02), g, layout=layout)
    x = synth.activations(M, K, wid=9)
    check_y(run(lib, x, qw, s, z, plan=plan, group_size=g, layout=layout),
            oracle.matmul(x, qw, s, z, g, layout=layout), f"split-K S={splits} g={g} M={M} K={K} N={N}")


def test_prefill_split_k_deterministic_and_counters_reset(lib):
    """Split-K sums in split order (bitwise repeatable); the arrival counters return to zero,
    so shapes with other tile counts and a decode split-K call can follow on the stream."""
    cases = [(512, 4096, 1024, 4), (130, 2048, 520, 3), (512, 4096, 1024, 4)]
    data = []
    for M, K, N, S in cases:
        qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=M + S, std=0.02))
        x = synth.activations(M, K, wid=9)
        data.append((dict(kernel=2, tile=3, splits=S), [dev(x), dev(qw), dev(s), dev(z)], oracle.matmul(x, qw, s, z)))
    first = [run(lib, *d, plan=p).clone() for p, d, _ in data]
    for rep in range(3):
        for (p, d, ref), a in zip(data, first):
            b = run(lib, *d, plan=p)
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (rep, p)
            check_y(b, ref, f"split-K rep {rep} {p}")
        qw, s, z = quantised(14336, 4096, 0)                  # decode split-K on the same stream
        x = synth.activations(4, 14336, wid=0)
        check_y(run(lib, x, qw, s, z), oracle.matmul(x, qw, s, z), "decode after prefill split-K")


# ---------------------------------------------------------------------------------------
# interleaved (pre-permuted) weight layout: every kernel, against the oracle

@pytest.mark.parametrize("g", [32, 128])
def test_dequant_bit_exact_interleaved(lib, g):
    W = synth.weight_custom(768, 200, seed=40 + g, std=0.02)
    qw, s, z = oracle.quantize_pack(W, g, layout="interleaved")
    print(f"\n[dequant interleaved] g={g}", flush=True)
    c, w = lib.w4a16_dequant(dev(qw), dev(s), dev(z), group_size=g, layout="interleaved")
    torch.cuda.synchronize()
    codes_ref = oracle.unpack(qw, "interleaved")
    assert np.array_equal(c.cpu().numpy(), codes_ref)
    w_ref = oracle.dequant_fp16(codes_ref, s, z, g)
    assert np.array_equal(w.cpu().numpy().view(np.uint16), w_ref.view(np.uint16))


IL_SHAPES = [(1, 4096, 4096), (5, 4096, 14336), (16, 14336, 4096), (37, 1024, 320), (3, 768, 2052)]


@pytest.mark.parametrize("M,K,N", IL_SHAPES, ids=[f"M{m}-K{k}-N{n}" for m, k, n in IL_SHAPES])
def test_matmul_interleaved_decode(lib, M, K, N):
    print(f"\n[interleaved] M={M} K={K} N={N} plan={lib.w4a16_plan(M, N, K)}", flush=True)
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=M, std=0.02), layout="interleaved")
    x = synth.activations(M, K, wid=3)
    check_y(run(lib, x, qw, s, z, layout="interleaved"), oracle.matmul(x, qw, s, z, layout="interleaved"),
            f"interleaved M={M} K={K} N={N}")


IL_PLANS = [dict(kernel=1, kc=kc, row_tiles=rt, waves=w, cols=c, seg=sg)
            for c in (16, 32, 64) for sg, kc in ((1, 2), (2, 4), (4, 8), (8, 16)) for rt in (1, 2)
            for w in (4, 8)]
IL_PLANS = [p for p in IL_PLANS if _plan_is_built(p, PLAN_MKN[0], PLAN_MKN[2], PLAN_MKN[1])]
_IL_CASE = {}


@pytest.mark.parametrize("plan", IL_PLANS, ids=[f"c{p['cols']}-seg{p['seg']}-kc{p['kc']}-rt{p['row_tiles']}"
                                                 f"-w{p['waves']}" for p in IL_PLANS])
def test_matmul_interleaved_skinny_plans(lib, plan):
    M, K, N = PLAN_MKN
    if not _IL_CASE:
        qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=13, std=0.02), layout="interleaved")
        x = synth.activations(M, K, wid=8)
        _IL_CASE.update(dev=[dev(x), dev(qw), dev(s), dev(z)],
                        ref=oracle.matmul(x, qw, s, z, layout="interleaved"))
    print(f"\n[interleaved plan] {plan}", flush=True)
    check_y(run(lib, *_IL_CASE["dev"], plan=plan, layout="interleaved"), _IL_CASE["ref"], f"interleaved {plan}")


IL_PREFILL = [(3, 256, 104), (130, 384, 1416), (257, 1408, 264), (200, 128, 136), (129, 2048, 1408)]


@pytest.mark.parametrize("tile", [1, 2, 3])
@pytest.mark.parametrize("g", [32, 128])
@pytest.mark.parametrize("M,K,N", IL_PREFILL, ids=[f"M{m}-K{k}-N{n}" for m, k, n in IL_PREFILL])
def test_matmul_interleaved_prefill_tiles(lib, M, K, N, g, tile):
    print(f"\n[interleaved prefill] tile={tile} g={g} M={M} K={K} N={N}", flush=True)
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=700 + M, std=0.02), g, layout="interleaved")
    x = synth.activations(M, K, wid=9)
    check_y(run(lib, x, qw, s, z, plan=dict(kernel=lib.W4A16_KERNEL_PREFILL, tile=tile), group_size=g,
                layout="interleaved"),
            oracle.matmul(x, qw, s, z, g, layout="interleaved"), f"interleaved tile={tile} g={g} M={M}")


@pytest.mark.parametrize("M,K,N", [(32, 8192, 8192), (128, 8192, 8192)])
def test_skinny_kernel_on_prefill_shapes(lib, M, K, N):
    """Both kernels must hold the bar where the dispatcher could pick either."""
    wid = synth.WORKLOADS["prefill"]["wid"]
    qw, s, z = quantised(K, N, wid)
    x = synth.activations(M, K, wid=wid)
    cols = _sample_cols(N)
    y_ref = oracle.matmul(x, qw[:, cols], s[:, cols], z[:, cols])
    for plan in (dict(kernel=lib.W4A16_KERNEL_SKINNY), dict(kernel=lib.W4A16_KERNEL_PREFILL)):
        y = run(lib, x, qw, s, z, plan=plan)
        check_y(y[:, torch.from_numpy(cols).to(DEV)], y_ref, f"{plan} M={M}")


@pytest.mark.parametrize("M,K,N,plan", [
    (1, 4096, 4096, dict(kernel=1, cols=64, waves=4, kc=8)),
    (16, 4096, 4096, dict(kernel=1, cols=16, waves=4, kc=4)),
    (1, 14336, 4096, None),
])
def test_deterministic_split_k(lib, M, K, N, plan):
    """Split-K sums are combined in a fixed order: repeated calls give the same bits."""
    qw, s, z = quantised(K, N, 0)
    x = synth.activations(M, K, wid=0)
    assert lib.w4a16_plan(M, N, K, **(plan or {}))["splits"] > 1
    args = [dev(x), dev(qw), dev(s), dev(z)]
    a = lib.w4a16_matmul(*args, plan=plan).clone()
    for _ in range(5):
        b = lib.w4a16_matmul(*args, plan=plan)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    check_y(a, oracle.matmul(x, qw, s, z), f"split-K {plan}")


def test_nondefault_stream_and_full_overwrite(lib):
    M, K, N = 4, 2048, 1408
    qw, s, z = quantised(K, N, 2)
    x = synth.activations(M, K, wid=2)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        args = [dev(x), dev(qw), dev(s), dev(z)]
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        lib.w4a16_matmul(*args, y=y, stream=st)
    st.synchronize()
    check_y(y, oracle.matmul(x, qw, s, z), "stream")


def test_alternating_shapes_reuse_counters(lib):
    """Split-K arrival counters must be back at zero after every call."""
    cases = [(1, 4096, 4096, 0), (4, 2048, 1408, 2), (16, 768, 2048, 2), (2, 4096, 4096, 0)]
    data = []
    for M, K, N, wid in cases:
        qw, s, z = quantised(K, N, wid)
        x = synth.activations(M, K, wid=wid)
        data.append((x, qw, s, z, [dev(x), dev(qw), dev(s), dev(z)]))
    for rep in range(3):
        for (x, qw, s, z, args) in data:
            y = lib.w4a16_matmul(*args)
            torch.cuda.synchronize()
            check_y(y, oracle.matmul(x, qw, s, z), f"alternating rep {rep}")


@pytest.mark.parametrize("kernel,tile", [(1, 0), (2, 1), (2, 2), (2, 3)])
def test_exact_closed_form_on_gpu(lib, kernel, tile):
    """K=128 exact case (W = ((k+n) mod 16 - 8) / 64): y(ones) = -1 for every column."""
    k = np.arange(128)[:, None]
    n = np.arange(64)[None, :]
    W = (((k + n) % 16 - 8) / 64.0).astype(np.float32)
    qw, s, z = oracle.quantize_pack(W)
    x = np.ones((3, 128), dtype=np.float16)
    y = run(lib, x, qw, s, z, plan=dict(kernel=kernel, tile=tile)).cpu().numpy()
    assert np.all(y == np.float16(-1.0))


# ---------------------------------------------------------------------------------------
# the dispatcher's switch points between the decode kernel and the async prefill tile

DISPATCH_EDGES = [(23, 8192, 16384, 1), (24, 8192, 16384, 2),     # K*N = 2^27: prefill from M = 24
                  (63, 4096, 8192, 1), (64, 4096, 8192, 2),       # 2^25, K <= N: from M = 64
                  (64, 8192, 4096, 1), (65, 8192, 4096, 2)]       # 2^25, K > N: from M = 65


@pytest.mark.parametrize("M,K,N,kernel", DISPATCH_EDGES, ids=[f"M{m}-K{k}-N{n}" for m, k, n, _ in DISPATCH_EDGES])
def test_dispatch_edges_automatic_plan(lib, M, K, N, kernel):
    """On either side of each switch point the automatic plan picks the documented kernel
    (the prefill tile with its 32-, 64- or 128-row work-groups) and matches the oracle."""
    pl = lib.w4a16_plan(M, N, K)
    print(f"\n[dispatch edge] M={M} K={K} N={N} plan={pl}", flush=True)
    assert pl["kernel"] == kernel
    qw, s, z = quantised(K, N, wid=3)
    x = synth.activations(M, K, wid=3)
    y = run(lib, x, qw, s, z)
    cols = _sample_cols(N)
    check_y(y[:, torch.from_numpy(cols).to(DEV)], oracle.matmul(x, qw[:, cols], s[:, cols], z[:, cols]),
            f"dispatch edge M={M} K={K} N={N}")
