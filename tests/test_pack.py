"""Host packer (w4a16_pack / w4a16_unpack in libw4a16.so) against the oracle, bit for bit.

CPU only: the packer is host code and no HIP call is made.
"""
import numpy as np
import pytest

import oracle
import synth
import weight_only_bit_gemv_amd as lib


def _same(a, b):
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def _check(W, group_size=128, symmetric=False, layout="linear"):
    qw, s, z = lib.w4a16_pack(W, group_size=group_size, symmetric=symmetric, layout=layout)
    qo, so, zo = oracle.quantize_pack(W, group_size, symmetric, layout)
    assert _same(qw, qo), "qweight differs"
    assert _same(s, so), "scales differ"
    assert _same(z, zo), "zeros differ"
    return qw, s, z


# reduced-N versions of every workload shape family (K unchanged)
SHAPES = [(4096, 256), (14336, 64), (4096, 448), (2048, 1408), (1408, 2048), (2048, 768),
          (768, 2048), (8192, 64), (28672, 32), (128, 8), (384, 5), (256, 1)]


@pytest.mark.parametrize("K,N", SHAPES)
def test_pack_matches_oracle_on_workload_draws(K, N):
    _check(synth.weight(K, N, wid=1))


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("std,mean", [(0.02, 0.0), (1.0, 0.0), (0.02, 1.0), (5.0, -3.0),
                                      (1e-3, 0.0), (3e-7, 0.0)])
def test_pack_matches_oracle_on_other_spreads(seed, std, mean):
    _check(synth.weight_custom(256, 40, seed=seed, std=std, mean=mean))


@pytest.mark.parametrize("symmetric", [False, True])
@pytest.mark.parametrize("g", [32, 64, 128, 256])
@pytest.mark.parametrize("K,N", [(4096, 96), (768, 200), (256, 7)])
def test_pack_group_sizes_and_modes_match_oracle(K, N, g, symmetric):
    qw, s, z = _check(synth.weight(K, N, wid=2), g, symmetric)
    assert s.shape == (K // g, N) and z.shape == (K // g, N)
    if symmetric:
        assert np.all(z == 8)


@pytest.mark.parametrize("g", [32, 64, 128, 256])
@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("std,mean", [(1.0, 0.0), (0.02, 1.0), (3e-7, 0.0)])
def test_pack_symmetric_other_spreads(g, seed, std, mean):
    _check(synth.weight_custom(512, 24, seed=seed, std=std, mean=mean), g, True)


def test_pack_symmetric_ties_and_extremes():
    """Symmetric mode: w/s = n + 0.5 ties go to even, +-max|w| map to codes 15 and 1."""
    s = 2.0 ** -5
    W = np.zeros((32, 4), dtype=np.float32)
    W[0, :] = 7 * s                                   # max|w| = 7 s -> scale s
    W[1, :] = -7 * s
    W[2:6, :] = np.array([0.5, 1.5, -0.5, -2.5], dtype=np.float32)[:, None] * s
    qw, sc, z = _check(W, 32, True)
    codes = lib.w4a16_unpack(qw)
    assert np.array_equal(codes[:6, 0], [15, 1, 8, 10, 8, 6])
    assert np.all(sc == np.float16(s)) and np.all(z == 8)


def test_pack_symmetric_zero_group_scale_one():
    W = np.zeros((64, 3), dtype=np.float32)
    W[:, 1] = -0.75
    qw, s, z = _check(W, 64, True)
    assert s[0, 0] == 1.0 and np.all(lib.w4a16_unpack(qw)[:, 0] == 8)
    assert np.all(lib.w4a16_unpack(qw)[:, 1] == 1)      # -0.75 / (0.75 / 7) = -7


def test_pack_exact_ties_round_half_even():
    """w/s = n + 0.5 exactly: half-to-even decides; packer and oracle must agree."""
    s = 2.0 ** -6
    W = np.zeros((128, 6), dtype=np.float32)
    W[1, :] = 15 * s                                  # group range 0 .. 15 s -> scale s, zero 0
    W[2:8, :] = np.array([0.5, 1.5, 2.5, 3.5, 12.5, 13.5], dtype=np.float32)[:, None] * s
    qw, sc, z = _check(W)
    codes = lib.w4a16_unpack(qw)
    assert np.array_equal(codes[2:8, 0], [0, 2, 2, 4, 12, 14])
    assert np.all(sc == np.float16(s)) and np.all(z == 0)


def test_pack_constant_and_zero_groups():
    W = np.zeros((256, 7), dtype=np.float32)
    W[:128, 1] = 3.7                                   # constant non-zero group -> scale 1.0
    W[128:, 2] = -0.25
    W[:, 3] = 1e-30                                    # scale underflows to 0 -> 1.0
    qw, s, z = _check(W)
    assert s[0, 1] == 1.0 and s[0, 3] == 1.0 and s[0, 0] == 1.0


def test_pack_special_words():
    """Groups that produce all-15 words (int32 -1) and words with the sign bit set."""
    W = np.zeros((128, 3), dtype=np.float32)
    W[:, 0] = 1.0
    W[0, 0] = 0.0                                      # codes 15 everywhere except row 0
    W[:, 1] = np.tile(np.array([0, 0, 0, 0, 0, 0, 0, 15], dtype=np.float32), 16)
    W[:, 2] = np.arange(128) % 16
    qw, s, z = _check(W)
    u = qw.view(np.uint32)
    assert u[1, 0] == 0xFFFFFFFF and qw[1, 0] == -1
    assert np.all(u[:, 1] == 0xF0000000)
    assert u[0, 2] == 0x76543210 and u[1, 2] == 0xFEDCBA98


def test_unpack_matches_oracle():
    codes = synth.uniform_codes(512, 37, seed=5)
    qw = oracle.pack(codes)
    assert np.array_equal(lib.w4a16_unpack(qw), oracle.unpack(qw))
    assert np.array_equal(lib.w4a16_unpack(qw), codes)


def test_pack_deterministic_across_calls():
    W = synth.weight(1024, 1000, wid=3)
    a = lib.w4a16_pack(W)
    b = lib.w4a16_pack(W)
    assert all(_same(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_pack_rejects_nonfinite(bad):
    W = synth.weight(256, 8)
    W[200, 3] = bad
    with pytest.raises(lib.W4A16Error) as e:
        lib.w4a16_pack(W)
    assert e.value.code == lib.W4A16_ERR_NONFINITE
    with pytest.raises(ValueError):
        oracle.quantize(W)


def test_pack_rejects_scale_overflow():
    W = np.zeros((128, 4), dtype=np.float32)
    W[0, 2] = -6e5
    W[1, 2] = 6e5                                      # (max - min) / 15 = 8e4 > 65504
    with pytest.raises(lib.W4A16Error) as e:
        lib.w4a16_pack(W)
    assert e.value.code == lib.W4A16_ERR_NONFINITE
    with pytest.raises(ValueError):
        oracle.quantize(W)


def test_pack_rejects_zero_out_of_domain():
    W = np.full((128, 4), 10.0, dtype=np.float32)
    W[0, :] = 10.001                                   # tiny spread far from 0: |zero| >> 1024
    with pytest.raises(lib.W4A16Error) as e:
        lib.w4a16_pack(W)
    assert e.value.code == lib.W4A16_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        oracle.quantize(W)


@pytest.mark.parametrize("K,N,g,code", [(100, 8, 128, lib.W4A16_ERR_UNSUPPORTED),
                                        (256, 8, 96, lib.W4A16_ERR_UNSUPPORTED),
                                        (256, 8, 16, lib.W4A16_ERR_UNSUPPORTED),
                                        (256, 8, 512, lib.W4A16_ERR_UNSUPPORTED),
                                        (96, 8, 64, lib.W4A16_ERR_UNSUPPORTED),
                                        (0, 8, 128, lib.W4A16_ERR_INVALID_ARG),
                                        (128, 0, 128, lib.W4A16_ERR_INVALID_ARG)])
def test_pack_rejects_bad_shapes(K, N, g, code):
    W = np.zeros((max(K, 1), max(N, 1)), dtype=np.float32)[:K, :N]
    with pytest.raises(lib.W4A16Error) as e:
        lib.w4a16_pack(W, group_size=g)
    assert e.value.code == code


def test_pack_ex_rejects_bad_symmetric_flag():
    W = np.zeros((128, 4), dtype=np.float32)
    out = [np.empty((16, 4), np.int32), np.empty((1, 4), np.float16), np.empty((1, 4), np.float16)]
    rc = lib.load().w4a16_pack_ex(W.ctypes.data, 128, 4, 128, 2, 0, *(a.ctypes.data for a in out))
    assert rc == lib.W4A16_ERR_INVALID_ARG
    rc = lib.load().w4a16_pack_ex(W.ctypes.data, 128, 4, 128, 0, 2, *(a.ctypes.data for a in out))
    assert rc == lib.W4A16_ERR_INVALID_ARG


@pytest.mark.parametrize("symmetric", [False, True])
@pytest.mark.parametrize("g", [32, 128])
@pytest.mark.parametrize("K,N", [(4096, 96), (768, 200), (256, 7)])
def test_pack_interleaved_layout_matches_oracle(K, N, g, symmetric):
    W = synth.weight(K, N, wid=4)
    qw, s, z = _check(W, g, symmetric, "interleaved")
    ql, sl, zl = lib.w4a16_pack(W, group_size=g, symmetric=symmetric)
    assert _same(s, sl) and _same(z, zl)                       # only the packing differs
    assert np.array_equal(lib.w4a16_unpack(qw, "interleaved"), lib.w4a16_unpack(ql))


def test_unpack_interleaved_matches_oracle():
    codes = synth.uniform_codes(512, 37, seed=8)
    qw = oracle.pack(codes, "interleaved")
    assert np.array_equal(lib.w4a16_unpack(qw, "interleaved"), codes)
    assert np.array_equal(lib.w4a16_unpack(qw, "interleaved"), oracle.unpack(qw, "interleaved"))


def test_unpack_ex_rejects_unknown_layout():
    qw = np.zeros((16, 4), np.int32)
    out = np.empty((128, 4), np.uint8)
    assert lib.load().w4a16_unpack_ex(qw.ctypes.data, 128, 4, 5, out.ctypes.data) == lib.W4A16_ERR_INVALID_ARG
