"""The library through its C ABI alone (needs an MI355X).

tests/capi/capi_driver.cpp (built by the build step into weight_only_bit_gemv_amd/lib/)
packs, dequantises and multiplies with plain host arrays, hipMalloc'd device buffers and a
hipStream_t, no Python or torch in its process. This test writes its inputs, runs it as a
child process and checks every output against the oracle: the packed format and the
dequantised weights bit for bit, the products at the oracle's bar.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

DRIVER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "weight_only_bit_gemv_amd", "lib",
                      "w4a16_capi_driver")


def _bar(y, ref):
    return np.all(np.abs(y - ref) <= 1e-2 + 5e-3 * np.abs(ref)), float(np.abs(y - ref).max())


@pytest.mark.parametrize("M,K,N,g", [(1, 4096, 4096, 128), (5, 2048, 1032, 64), (300, 1024, 520, 128),
                                     (16, 14336, 4096, 256)])
def test_c_abi_driver_matches_oracle(tmp_path, M, K, N, g):
    if not os.path.exists(DRIVER):
        pytest.fail(f"{DRIVER} is missing: run the build step")
    W = synth.weight_custom(K, N, seed=140 + M, std=0.02)
    x = synth.activations(M, K, wid=15)
    W.astype(np.float32).tofile(tmp_path / "w.f32")
    x.view(np.uint16).tofile(tmp_path / "x.f16")
    print(f"\n[capi] M={M} K={K} N={N} g={g}", flush=True)
    r = subprocess.run([DRIVER, str(tmp_path), str(M), str(K), str(N), str(g)], capture_output=True, text=True,
                       timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr

    def load(name, dtype, shape):
        return np.fromfile(tmp_path / name, dtype=dtype).reshape(shape)
    qw_ref, s_ref, z_ref = oracle.quantize_pack(W, g)
    qw = load("qweight.i32", np.int32, (K // 8, N))
    s = load("scales.f16", np.uint16, (K // g, N)).view(np.float16)
    z = load("zeros.f16", np.uint16, (K // g, N)).view(np.float16)
    assert np.array_equal(qw, qw_ref) and np.array_equal(s.view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(z.view(np.uint16), z_ref.view(np.uint16))
    assert np.array_equal(load("codes.u8", np.uint8, (K, N)), oracle.unpack(qw_ref))
    deq = load("deq.f16", np.uint16, (K, N))
    assert np.array_equal(deq, oracle.dequant_fp16(oracle.unpack(qw_ref), s_ref, z_ref, g).view(np.uint16))
    ref = oracle.matmul(x, qw_ref, s_ref, z_ref, g)
    for name in ("y.f16", "y_noalloc.f16", "y_grouped0.f16"):
        y = load(name, np.uint16, (M, N)).view(np.float16).astype(np.float64)
        ok, err = _bar(y, ref)
        assert ok, (name, err)
    y = load("y_grouped1.f16", np.uint16, (M, N)).view(np.float16).astype(np.float64)
    ok, err = _bar(y, oracle.matmul(-x, qw_ref, s_ref, z_ref, g))
    assert ok, ("y_grouped1.f16", err)
    # the decode and no-alloc entry points share kernels and plans: same bits
    assert np.array_equal(load("y.f16", np.uint16, (M, N)), load("y_noalloc.f16", np.uint16, (M, N)))
    if g in (128, 256):
        xq_ref, sx_ref = oracle.quantize_activations(x)
        assert np.array_equal(load("xq.u8", np.uint8, (M, K)), xq_ref)
        assert np.array_equal(load("sx.f32", np.float32, (M,)), sx_ref)
        y8 = load("y8.f16", np.uint16, (M, N)).view(np.float16).astype(np.float64)
        ok, err = _bar(y8, oracle.matmul_w4a8(xq_ref, sx_ref, qw_ref, s_ref, z_ref, g))
        assert ok, ("y8.f16", err)
