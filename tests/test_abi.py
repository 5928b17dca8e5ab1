"""The C-ABI library loads, exports every function include/w4a16.h declares, and rejects
bad arguments before making any HIP call (so these run without a GPU)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import weight_only_bit_gemv_amd as lib
from weight_only_bit_gemv_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(w4a(?:16|8)_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["w4a16_pack", "w4a16_pack_ex", "w4a16_unpack_ex", "w4a16_matmul_fmt",
                     "w4a16_dequant_fmt", "w4a16_matmul", "w4a16_matmul_ex", "w4a16_plan",
                     "w4a16_dequant", "w4a16_unpack", "w4a16_strerror", "w4a8_quantize_activations",
                     "w4a8_matmul"]:
        assert required in names


def test_library_exports_every_declared_symbol():
    so = ctypes.CDLL(B.LIB_PATH)
    for name in declared_functions():
        assert hasattr(so, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (w4a(?:16|8)_\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_binding_covers_every_symbol():
    assert set(declared_functions()) == set(B._SIGS)


def test_strerror_and_version():
    for code in [0, -1, -2, -3, -4, -5]:
        assert lib.strerror(code) and lib.strerror(code) != "unknown error code"
    assert lib.strerror(-99) == "unknown error code"
    assert lib.w4a16_version() >= 100


# Fake, 16-byte aligned, never-dereferenced addresses: validation rejects every call below
# before any HIP call, so no device is needed.
A = 0x100000
P = [ctypes.c_void_p(A + 0x1000 * i) for i in range(5)]


def _mm(M, N, K, g=128, ptrs=None):
    p = ptrs or P
    return B.load().w4a16_matmul(p[0], p[1], p[2], p[3], p[4], M, N, K, g, None)


@pytest.mark.parametrize("M,N,K,g,code", [
    (0, 64, 128, 128, lib.W4A16_ERR_INVALID_ARG),
    (1, 0, 128, 128, lib.W4A16_ERR_INVALID_ARG),
    (1, 64, 0, 128, lib.W4A16_ERR_INVALID_ARG),
    (-3, 64, 128, 128, lib.W4A16_ERR_INVALID_ARG),
    (1, 64, 128, 96, lib.W4A16_ERR_UNSUPPORTED),
    (1, 64, 128, 16, lib.W4A16_ERR_UNSUPPORTED),
    (1, 64, 128, 256, lib.W4A16_ERR_UNSUPPORTED),
    (1, 64, 192, 64, lib.W4A16_ERR_UNSUPPORTED),
    (1, 64, 200, 128, lib.W4A16_ERR_UNSUPPORTED),
    (1, 66, 128, 128, lib.W4A16_ERR_UNSUPPORTED),
    (1, 1 << 20, 1 << 16, 128, lib.W4A16_ERR_UNSUPPORTED),
])
def test_matmul_rejects_bad_shapes(M, N, K, g, code):
    assert _mm(M, N, K, g) == code
    assert B.load().w4a16_last_error_detail().decode()


def test_matmul_rejects_null_and_misaligned():
    for i in range(5):
        ptrs = list(P)
        ptrs[i] = None
        assert _mm(1, 64, 128, ptrs=ptrs) == lib.W4A16_ERR_INVALID_ARG
        ptrs = list(P)
        ptrs[i] = ctypes.c_void_p(A + 8)
        assert _mm(1, 64, 128, ptrs=ptrs) == lib.W4A16_ERR_ALIGNMENT


def test_matmul_ex_rejects_bad_plans():
    so = B.load()
    for kw in [dict(kernel=7), dict(kernel=1, kc=3), dict(kernel=1, kc=6), dict(kernel=1, kc=-4),
               dict(kernel=1, row_tiles=5), dict(kernel=1, waves=6), dict(kernel=1, waves=16, row_tiles=2),
               dict(kernel=1, kc=4, waves=4, splits=3), dict(kernel=2, tile=4), dict(kernel=2, tile=-1), dict(kernel=2, kc=4),
               dict(kernel=2, waves=8)]:
        pl = B.w4a16_plan_t(**kw)
        rc = so.w4a16_matmul_ex(P[0], P[1], P[2], P[3], P[4], 1, 64, 128, 128, None,
                                ctypes.byref(pl))
        assert rc == lib.W4A16_ERR_INVALID_ARG, kw
    assert so.w4a16_matmul_ex(P[0], P[1], P[2], P[3], P[4], 1, 64, 128, 128, None,
                              None) == lib.W4A16_ERR_INVALID_ARG


def test_dequant_rejects_bad_arguments():
    so = B.load()
    assert so.w4a16_dequant(P[0], P[1], P[2], None, None, 64, 128, 128, None) == lib.W4A16_ERR_INVALID_ARG
    assert so.w4a16_dequant(None, P[1], P[2], P[3], None, 64, 128, 128, None) == lib.W4A16_ERR_INVALID_ARG
    assert so.w4a16_dequant(P[0], P[1], P[2], P[3], None, 62, 128, 128, None) == lib.W4A16_ERR_UNSUPPORTED
    assert so.w4a16_dequant(ctypes.c_void_p(A + 4), P[1], P[2], P[3], None, 64, 128, 128,
                            None) == lib.W4A16_ERR_ALIGNMENT


# ---- dispatcher (host only) ----

PLAN_SHAPES = [(m, k, n) for m in (1, 2, 4, 8, 16, 17, 23, 24, 33, 48, 49, 63, 64, 65, 96, 97, 128, 129, 512, 2048)
               for (k, n) in [(4096, 4096), (4096, 14336), (14336, 4096), (2048, 1408), (8192, 28672),
                              (768, 2048), (4096, 128256), (128, 4), (384, 100), (4096, 28676),
                              (4096, 1024), (5120, 5120), (13824, 5120), (3584, 18944), (7168, 1024),
                              (2560, 10240), (3072, 3072), (896, 4864)]]
# every (K, N) of the dispatcher's plan table beyond the shapes above, at the M of each bucket
# and around its edges
TABLE_KN = [(4096, 512), (5120, 1024), (8192, 1024), (16384, 1024), (2048, 512), (2048, 2048), (4096, 2048),
            (8192, 2048), (1024, 4096), (6144, 4096), (8192, 4096), (11008, 4096), (4096, 6144), (4096, 8192),
            (2048, 8192), (18944, 3584), (4096, 11008), (5120, 13824), (10240, 2560), (4864, 896),
            (1536, 8960), (8960, 1536), (3072, 8192), (8192, 3072), (4096, 3072), (12288, 4096), (4096, 28672),
            (4096, 12288), (2048, 11264), (2048, 12288), (1408, 8192), (768, 16384), (1408, 16384),
            (4096, 1792), (14336, 512), (4096, 16032), (8192, 8192), (8192, 28672), (28672, 8192)]
PLAN_SHAPES += [(m, k, n) for m in (1, 2, 4, 5, 16, 17) for (k, n) in TABLE_KN]


@pytest.mark.parametrize("M,K,N", PLAN_SHAPES)
def test_auto_plan_is_valid_and_covers_k(M, K, N):
    pl = lib.w4a16_plan(M, N, K)
    assert pl["kernel"] in (lib.W4A16_KERNEL_SKINNY, lib.W4A16_KERNEL_PREFILL)
    tiles = -(-M // 128) * -(-N // 128)
    if N % 8 == 0:
        expect_prefill = ((M >= 65 and (M > 128 or K * N >= 1 << 25)) or (M >= 24 and K * N >= 1 << 27) or
                          (M >= 64 and K * N >= 1 << 25 and K <= N))
    else:
        expect_prefill = M >= 65 and (tiles >= 128 or M > 1024)
    assert pl["kernel"] == (lib.W4A16_KERNEL_PREFILL if expect_prefill else lib.W4A16_KERNEL_SKINNY)
    if pl["kernel"] == lib.W4A16_KERNEL_PREFILL:
        groups = -(-M // 128) * -(-N // 256)
        expect = (lib.W4A16_TILE_ASYNC if N % 8 == 0 else
                  lib.W4A16_TILE_REGISTER_B if groups >= 384 else lib.W4A16_TILE_LDS)
        assert pl["tile"] == expect
        if expect == lib.W4A16_TILE_ASYNC:
            stages = K // 64
            bm = 32 if M <= 32 else 64 if M <= 64 else 128           # rows per work-group
            target, min_stages = (512, 12) if bm < 128 else (256, 16)
            groups = -(-M // bm) * -(-N // 256)
            want = 1 if groups > target else min(max(1, (target + groups // 2) // groups), max(1, stages // min_stages))
            if bm < 128:
                want = 1 << (want.bit_length() - 1)                 # power of two
            if groups * want <= target and stages // want > 128:
                want *= 2                                # two work-groups per compute unit
            assert pl["splits"] <= want and (pl["splits"] > 1) == (want > 1)
            per = 2 * -(-stages // (2 * pl["splits"]))   # even stages per split, all covered
            assert -(-stages // per) == pl["splits"]
    if pl["kernel"] == lib.W4A16_KERNEL_SKINNY:
        kc, splits, W = pl["kc"], pl["splits"], pl["waves"]
        assert kc in (1, 2) or kc % 4 == 0
        assert W in (4, 8, 16) and (W - 1) * pl["row_tiles"] * pl["cols"] <= 15 * 64
        KS = K // 32
        chunks = -(-KS // kc)
        assert splits == -(-chunks // W)
        assert splits * W * kc >= KS                 # every K-step is covered
        assert (splits - 1) * W * kc < KS            # no work-group is entirely empty
        assert pl["cols"] in (16, 32, 64) and kc % pl["seg"] == 0
        assert pl["seg"] != 8 or KS % 8 == 0
        assert 1 <= pl["row_tiles"] <= (4 if pl["cols"] == 64 else 2)
        assert pl["row_tiles"] * 16 >= min(M, 64 if pl["cols"] == 64 else 32)
        assert pl["row_tiles"] == min(4 if pl["cols"] == 64 else 2, -(-M // 16))


@pytest.mark.parametrize("g", [32, 64, 128, 256])
@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (1, 4096, 14336), (1, 14336, 4096),
                                   (16, 8192, 8192), (1, 2048, 1408), (4, 4096, 128256)])
def test_auto_plan_per_group_size_is_built(M, K, N, g):
    """Every group size gets a plan the library has compiled: 8-step segments only with
    128-row groups (they span two groups of four K-steps)."""
    pl = lib.w4a16_plan(M, N, K, group_size=g)
    assert pl["kernel"] == lib.W4A16_KERNEL_SKINNY
    assert pl["kc"] % pl["seg"] == 0
    assert pl["seg"] != 8 or g == 128


@pytest.mark.parametrize("g,ok", [(32, False), (64, False), (128, True), (256, False)])
def test_forced_seg8_needs_128_row_groups(g, ok):
    kw = dict(kernel=lib.W4A16_KERNEL_SKINNY, kc=8, seg=8, waves=4)
    if ok:
        assert lib.w4a16_plan(1, 4096, 4096, group_size=g, **kw)["seg"] == 8
    else:
        with pytest.raises(lib.W4A16Error) as e:
            lib.w4a16_plan(1, 4096, 4096, group_size=g, **kw)
        assert e.value.code == lib.W4A16_ERR_INVALID_ARG


@pytest.mark.parametrize("waves", [4, 8, 16])
@pytest.mark.parametrize("kc", [1, 2, 4, 8, 12, 16, 64])
def test_forced_kc_plan(kc, waves):
    pl = lib.w4a16_plan(3, 4096, 4096, kernel=lib.W4A16_KERNEL_SKINNY, kc=kc, waves=waves)
    assert pl["kc"] == kc and pl["waves"] == waves
    assert pl["splits"] == -(-(-(-128 // kc)) // waves)


def test_one_hip_runtime_per_process():
    """Importing the package (before or after torch) leaves exactly one libamdhip64 mapped:
    the library must call the runtime that owns torch's device memory and streams."""
    code = ("import weight_only_bit_gemv_amd as L, torch; "
            "import sys; r = L.hip_runtimes_loaded(); print(r); sys.exit(0 if len(r) == 1 else 1)")
    for src in (code, "import torch; " + code):
        r = subprocess.run([sys.executable, "-c", src], cwd=ROOT, capture_output=True, text=True,
                           timeout=300)
        assert r.returncode == 0, f"{src}\n{r.stdout}\n{r.stderr}"


def test_python_constants_match_header():
    """The binding's W4A16_* integers are the header's #define values."""
    text = open(HEADER).read()
    defs = dict((k, int(v)) for k, v in re.findall(r"^#define (W4A16_\w+)\s+(-?\d+)", text, flags=re.M))
    assert len(defs) >= 11
    for name, value in defs.items():
        assert getattr(lib, name) == value, name


def test_async_tile_needs_n_multiple_of_8():
    with pytest.raises(lib.W4A16Error) as e:
        lib.w4a16_plan(256, 1412, 1024, kernel=lib.W4A16_KERNEL_PREFILL, tile=lib.W4A16_TILE_ASYNC)
    assert e.value.code == lib.W4A16_ERR_UNSUPPORTED
    assert lib.w4a16_plan(256, 1416, 1024, kernel=lib.W4A16_KERNEL_PREFILL,
                          tile=lib.W4A16_TILE_ASYNC)["tile"] == lib.W4A16_TILE_ASYNC


def test_fmt_entry_points_reject_unknown_layout_and_misaligned_codes():
    so = B.load()
    assert so.w4a16_matmul_fmt(P[0], P[1], P[2], P[3], P[4], 1, 64, 128, 128, 2, None, None) == \
        lib.W4A16_ERR_INVALID_ARG
    assert so.w4a16_dequant_fmt(P[0], P[1], P[2], None, P[4], 64, 128, 128, -1, None) == \
        lib.W4A16_ERR_INVALID_ARG
    assert so.w4a16_dequant_fmt(P[0], P[1], P[2], ctypes.c_void_p(A + 2), None, 64, 128, 128, 0, None) == \
        lib.W4A16_ERR_ALIGNMENT


def test_prefill_split_plans():
    assert lib.w4a16_plan(512, 4096, 14336, kernel=2, tile=3)["splits"] == 4        # 64 tiles
    assert lib.w4a16_plan(2048, 28672, 8192, kernel=2, tile=3)["splits"] == 1       # 1792 tiles
    for S in (1, 2, 3, 5, 9, 100):
        pl = lib.w4a16_plan(512, 4096, 14336, kernel=2, tile=3, splits=S)
        per = 2 * -(-224 // (2 * pl["splits"]))
        assert -(-224 // per) == pl["splits"] and 224 - (pl["splits"] - 1) * per >= 2
    for kw in [dict(kernel=2, tile=1, splits=2), dict(kernel=2, tile=3, splits=113), dict(kernel=2, tile=3, splits=-1)]:
        with pytest.raises(lib.W4A16Error) as e:
            lib.w4a16_plan(512, 4096, 14336, **kw)
        assert e.value.code == lib.W4A16_ERR_INVALID_ARG, kw


def test_w4a8_entry_points_reject_bad_arguments():
    so = B.load()
    q = so.w4a8_quantize_activations
    X = ctypes.c_void_p(A + 0x6000)                        # block sums
    assert q(None, P[1], P[2], X, 4, 256, None) == lib.W4A16_ERR_INVALID_ARG
    assert q(P[0], P[1], P[2], None, 4, 256, None) == lib.W4A16_ERR_INVALID_ARG
    assert q(P[0], P[1], P[2], X, 0, 256, None) == lib.W4A16_ERR_INVALID_ARG
    assert q(P[0], P[1], P[2], X, 4, 200, None) == lib.W4A16_ERR_UNSUPPORTED
    assert q(ctypes.c_void_p(A + 8), P[1], P[2], X, 4, 256, None) == lib.W4A16_ERR_ALIGNMENT
    assert q(P[0], P[1], ctypes.c_void_p(A + 2), X, 4, 256, None) == lib.W4A16_ERR_ALIGNMENT
    assert q(P[0], P[1], P[2], ctypes.c_void_p(A + 0x6004), 4, 256, None) == lib.W4A16_ERR_ALIGNMENT
    m = so.w4a8_matmul

    def call(M=4, N=64, K=256, g=128, layout=0, ptrs=None):
        pp = ptrs or [P[0], P[1], X, P[2], P[3], P[4], ctypes.c_void_p(A + 0x5000)]
        return m(*pp, M, N, K, g, layout, None)
    assert call(M=0) == lib.W4A16_ERR_INVALID_ARG
    assert call(layout=3) == lib.W4A16_ERR_INVALID_ARG
    assert call(g=64) == lib.W4A16_ERR_UNSUPPORTED                 # 8-bit MFMA spans 128 rows
    assert call(g=32) == lib.W4A16_ERR_UNSUPPORTED
    assert call(N=60) == lib.W4A16_ERR_UNSUPPORTED                 # N % 8
    assert call(K=200) == lib.W4A16_ERR_UNSUPPORTED
    bad = [P[0], P[1], X, P[2], P[3], ctypes.c_void_p(A + 0x4008), ctypes.c_void_p(A + 0x5000)]
    assert call(ptrs=bad) == lib.W4A16_ERR_ALIGNMENT
    bad = [P[0], P[1], ctypes.c_void_p(A + 0x6008), P[2], P[3], P[4], ctypes.c_void_p(A + 0x5000)]
    assert call(ptrs=bad) == lib.W4A16_ERR_ALIGNMENT
    nul = [P[0], None, X, P[2], P[3], P[4], ctypes.c_void_p(A + 0x5000)]
    assert call(ptrs=nul) == lib.W4A16_ERR_INVALID_ARG
    nul = [P[0], P[1], None, P[2], P[3], P[4], ctypes.c_void_p(A + 0x5000)]
    assert call(ptrs=nul) == lib.W4A16_ERR_INVALID_ARG
    ex = so.w4a8_matmul_ex
    pp = [P[0], P[1], X, P[2], P[3], P[4], ctypes.c_void_p(A + 0x5000)]
    assert ex(*pp, 4, 64, 256, 128, 0, -1, None) == lib.W4A16_ERR_INVALID_ARG
    assert ex(*pp, 4, 64, 256, 128, 0, 3, None) == lib.W4A16_ERR_INVALID_ARG      # > K / 128


def test_skinny_plan_offsets_fit_31_bits():
    """The decode kernel addresses a wavefront's weights with 32-bit byte offsets: a forced
    K range of kc K-steps must keep 16 N (kc + 1) bytes below 2^31."""
    N, K = 1 << 20, 4096                                   # 16 N * 129 > 2^31 - 1 >= 16 N * 128
    with pytest.raises(lib.W4A16Error) as e:
        lib.w4a16_plan(1, N, K, kernel=lib.W4A16_KERNEL_SKINNY, kc=128, waves=4)
    assert e.value.code == lib.W4A16_ERR_UNSUPPORTED
    assert lib.w4a16_plan(1, N, K, kernel=lib.W4A16_KERNEL_SKINNY, kc=124, waves=4)["kc"] == 124


def test_missing_library_fails_loudly(monkeypatch):
    """Without the built library (and no build allowed) the binding raises instead of
    falling back to anything else."""
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", os.path.join(os.path.dirname(B.LIB_PATH), "missing", "libw4a16.so"))
    with pytest.raises(ImportError):
        B.load(build_if_missing=False)


def test_offsets_beyond_31_bits_are_rejected():
    """The W4A8 kernel addresses 16 packed rows of weights (64 N bytes), the async W4A16 tile
    8 packed rows and 128 activation rows of a stage, and both the split partials of an
    output tile (128 KiB each) with 32-bit offsets: shapes or split counts past that are
    rejected before any HIP call."""
    so = B.load()
    pp = [P[0], P[1], ctypes.c_void_p(A + 0x6000), P[2], P[3], P[4], ctypes.c_void_p(A + 0x5000)]
    assert so.w4a8_matmul_ex(*pp, 1, 1 << 25, 128, 128, 0, 0, None) == lib.W4A16_ERR_UNSUPPORTED
    assert "32-bit" in B.load().w4a16_last_error_detail().decode()
    assert so.w4a8_matmul_ex(*pp, 1, 8, 1 << 21, 128, 0, 16384, None) == lib.W4A16_ERR_UNSUPPORTED
    with pytest.raises(lib.W4A16Error) as e:
        lib.w4a16_plan(1, 8, 1 << 21, kernel=2, tile=3, splits=16384)
    assert e.value.code == lib.W4A16_ERR_UNSUPPORTED
    assert lib.w4a16_plan(1, 8, 1 << 21, kernel=2, tile=3, splits=16383)["splits"] <= 16383
    # the async tile's loads: 32 N bytes of weights and 128 K 2 bytes of activations per stage
    for M, N, K in [(8, (1 << 26) + 8, 128), (128, 8, 1 << 23)]:
        with pytest.raises(lib.W4A16Error) as e:
            lib.w4a16_plan(M, N, K, kernel=2, tile=3)
        assert e.value.code == lib.W4A16_ERR_UNSUPPORTED
        assert "load offsets" in B.load().w4a16_last_error_detail().decode()
    assert lib.w4a16_plan(8, (1 << 26) - 8, 128, kernel=2, tile=3)["tile"] == 3
    assert lib.w4a16_plan(128, 8, (1 << 23) - 128, kernel=2, tile=3)["tile"] == 3


def test_binding_dequant_checks_scale_shapes():
    """w4a16_dequant's binding checks scales/zeros against [K/group_size, N] on the host: the
    C entry point cannot see buffer sizes, and short scales would be read past their end."""
    torch = pytest.importorskip("torch")
    qw = torch.zeros((32, 64), dtype=torch.int32)          # K = 256, N = 64
    good = torch.zeros((2, 64), dtype=torch.float16)
    for s, z, g in [(torch.zeros((1, 64), dtype=torch.float16), good, 128),
                    (good, torch.zeros((2, 60), dtype=torch.float16), 128),
                    (good, good, 64), (good, good, 96)]:
        with pytest.raises(ValueError):
            lib.w4a16_dequant(qw, s, z, group_size=g)
    with pytest.raises(ValueError):
        lib.w4a16_dequant(torch.zeros(64, dtype=torch.int32), good, good)


def test_noalloc_rejects_plans_beyond_the_scratch():
    """w4a16_matmul_noalloc takes only plans whose split-K partials fit its static scratch;
    a larger one is rejected before any HIP call (the fake pointers are never used)."""
    so = B.load()
    pl = B.w4a16_plan_t(kernel=2, tile=3, splits=64)      # 64 output tiles x 64 splits x 128 KiB
    rc = so.w4a16_matmul_noalloc(P[0], P[1], P[2], P[3], P[4], 130, 8192, 8192, 128, 0, None, ctypes.byref(pl))
    assert rc == lib.W4A16_ERR_UNSUPPORTED
    assert "static scratch" in so.w4a16_last_error_detail().decode()
    assert so.w4a16_matmul_noalloc(P[0], None, P[2], P[3], P[4], 1, 64, 128, 128, 0, None,
                                   None) == lib.W4A16_ERR_INVALID_ARG


def test_grouped_rejects_bad_arguments():
    """w4a16_matmul_grouped validates every matrix (and the summed N) before any launch."""
    so = B.load()

    def mats(*ns, bad=None):
        arr = (B.w4a16_matrix_t * len(ns))()
        for i, n in enumerate(ns):
            base = A + 0x10000 * (i + 1)
            arr[i] = B.w4a16_matrix_t(base, base + 0x1000, base + 0x2000, base + 0x3000, n)
        if bad is not None:
            setattr(arr[bad[0]], bad[1], bad[2])
        return arr

    def call(arr, n=None, M=1, K=4096, g=128, layout=0, x=P[0], plan=None):
        return so.w4a16_matmul_grouped(x, arr, len(arr) if n is None else n, M, K, g, layout, None, plan)
    assert call(mats(64), n=0) == lib.W4A16_ERR_INVALID_ARG
    assert call(mats(*[64] * 17)) == lib.W4A16_ERR_INVALID_ARG                      # at most 16
    assert call(mats(64, 64, bad=(1, "x", A + 0x4008))) == lib.W4A16_ERR_ALIGNMENT  # a matrix's own x
    assert call(mats(64, 64, bad=(1, "M", 2))) == lib.W4A16_ERR_INVALID_ARG         # M_i > M
    assert call(mats(64, 64, bad=(1, "M", -1))) == lib.W4A16_ERR_INVALID_ARG
    assert call(mats(64, 64), x=None) == lib.W4A16_ERR_INVALID_ARG
    assert call(mats(64, 64, bad=(1, "zeros", None))) == lib.W4A16_ERR_INVALID_ARG
    assert call(mats(64, 62)) == lib.W4A16_ERR_UNSUPPORTED                         # N % 4
    assert call(mats(64, 64), K=200) == lib.W4A16_ERR_UNSUPPORTED
    assert call(mats(64, 64), layout=5) == lib.W4A16_ERR_INVALID_ARG
    assert call(mats(64, 64, bad=(0, "y", A + 0x3008))) == lib.W4A16_ERR_ALIGNMENT
    assert call(mats(64, 64), x=ctypes.c_void_p(A + 4)) == lib.W4A16_ERR_ALIGNMENT
    bad_plan = B.w4a16_plan_t(kernel=1, cols=24)
    assert call(mats(64, 64), plan=ctypes.byref(bad_plan)) == lib.W4A16_ERR_INVALID_ARG
    assert so.w4a16_matmul_grouped(P[0], None, 1, 1, 4096, 128, 0, None, None) == lib.W4A16_ERR_INVALID_ARG


# ---- plans set at run time (w4a16_set_plan / w4a16_autotune), host side ----

def test_set_plan_takes_precedence_until_removed():
    M, N, K = 1, 4096, 4096
    default = lib.w4a16_plan(M, N, K)
    forced = dict(kernel=lib.W4A16_KERNEL_SKINNY, cols=64, waves=8, kc=8, seg=4)
    try:
        lib.w4a16_set_plan(M, N, K, forced)
        got = lib.w4a16_plan(M, N, K)
        assert got == lib.w4a16_plan(M, N, K, **forced)          # stored complete
        assert got != default
        assert lib.w4a16_plan(M, N, K, group_size=64) == lib.w4a16_plan(M, N, K, group_size=64)
        assert lib.w4a16_plan(2, N, K) == lib.w4a16_plan(2, N, K)  # other shapes untouched
        # a forced plan still wins over the stored one
        assert lib.w4a16_plan(M, N, K, kernel=1, cols=16, waves=4, kc=32)["cols"] == 16
        lib.w4a16_set_plan(M, N, K, None)
        assert lib.w4a16_plan(M, N, K) == default
        lib.w4a16_set_plan(M, N, K, forced)
        lib.w4a16_clear_plans()
        assert lib.w4a16_plan(M, N, K) == default
    finally:
        lib.w4a16_clear_plans()


def test_set_plan_rejects_unusable_plans():
    so = B.load()
    try:
        for kw, code in [(dict(), lib.W4A16_ERR_INVALID_ARG), (dict(kernel=1, cols=48), lib.W4A16_ERR_INVALID_ARG),
                         (dict(kernel=1, kc=6), lib.W4A16_ERR_INVALID_ARG), (dict(kernel=9), lib.W4A16_ERR_INVALID_ARG)]:
            pl = B.w4a16_plan_t(**kw)
            assert so.w4a16_set_plan(1, 4096, 4096, 128, ctypes.byref(pl)) == code, kw
            assert so.w4a16_last_error_detail().decode()
        pl = B.w4a16_plan_t(kernel=1)
        assert so.w4a16_set_plan(1, 66, 4096, 128, ctypes.byref(pl)) == lib.W4A16_ERR_UNSUPPORTED
        assert so.w4a16_set_plan(0, 64, 4096, 128, ctypes.byref(pl)) == lib.W4A16_ERR_INVALID_ARG
        assert lib.w4a16_plan(1, 4096, 4096) == lib.w4a16_plan(1, 4096, 4096)
    finally:
        lib.w4a16_clear_plans()


def test_autotune_rejects_bad_arguments_before_any_hip_call():
    so = B.load()

    def tune(ptrs, M=1, N=64, K=128, g=128, layout=0):
        return so.w4a16_autotune(ptrs[0], ptrs[1], ptrs[2], ptrs[3], ptrs[4], M, N, K, g, layout, None, None, None)
    for i in range(5):
        ptrs = list(P)
        ptrs[i] = None
        assert tune(ptrs) == lib.W4A16_ERR_INVALID_ARG
        ptrs = list(P)
        ptrs[i] = ctypes.c_void_p(A + 8)
        assert tune(ptrs) == lib.W4A16_ERR_ALIGNMENT
    assert tune(P, layout=5) == lib.W4A16_ERR_INVALID_ARG
    assert tune(P, N=66) == lib.W4A16_ERR_UNSUPPORTED
    assert tune(P, M=0) == lib.W4A16_ERR_INVALID_ARG
    assert tune(P, g=96) == lib.W4A16_ERR_UNSUPPORTED
