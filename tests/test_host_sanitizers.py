"""The host packer and the C ABI's validation / dispatch layer built with AddressSanitizer
and UndefinedBehaviorSanitizer (g++, CPU only), run on packing cases and on every error
path. The HIP runtime and the kernel launchers are stubs that abort, so the run also shows
that every rejected call is settled before any HIP call.

The packer's codes are compared bit for bit with the oracle's (and with the regular build
of the library): a packing mistake of the kind "Triton Kernel Matches bitsandbytes: Why Both
Lose to Math", section "Three Kernel Versions and Two Bugs", describes (a missing +8 zero
point) would show here as well as in test_pack.py.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weight_only_bit_gemv_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]

CASES = [  # K, N, group, symmetric, layout, weights
    (256, 40, 128, 0, 0, lambda: synth.weight(256, 40, wid=0)),
    (512, 13, 32, 1, 1, lambda: synth.weight_custom(512, 13, seed=31, std=0.02, mean=1.0)),
    (384, 24, 64, 0, 1, lambda: synth.weight_custom(384, 24, seed=32, std=5.0, mean=-3.0)),
    (1024, 300, 256, 1, 0, lambda: synth.weight_custom(1024, 300, seed=33, std=0.02)),
    (2048, 96, 128, 0, 0, lambda: synth.weight_custom(2048, 96, seed=34, std=3e-7)),
]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    out = tmp_path_factory.mktemp("san")
    exe = str(out / "host_driver")
    cmd = (["g++", "-std=c++17", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", os.path.join(ROCM, "include")] + SAN +
           [os.path.join(CSRC, "w4a16_pack.cpp"), os.path.join(CSRC, "w4a16_api.cpp"), DRIVER,
            "-o", exe, "-lpthread"])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe, out


def test_sanitized_packer_and_validation(driver):
    exe, out = driver
    with open(out / "cases.txt", "w") as f:
        for i, (K, N, g, sym, layout, make) in enumerate(CASES):
            make().astype(np.float32).tofile(out / f"w{i}.bin")
            f.write(f"{K} {N} {g} {sym} {layout}\n")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, str(out)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.startswith("checks ok"), r.stdout
    for i, (K, N, g, sym, layout, make) in enumerate(CASES):
        lay = ["linear", "interleaved"][layout]
        qw_ref, s_ref, z_ref = oracle.quantize_pack(make(), g, bool(sym), lay)
        qw = np.fromfile(out / f"q{i}.bin", dtype=np.int32).reshape(K // 8, N)
        s = np.fromfile(out / f"s{i}.bin", dtype=np.uint16).reshape(K // g, N)
        z = np.fromfile(out / f"z{i}.bin", dtype=np.uint16).reshape(K // g, N)
        c = np.fromfile(out / f"c{i}.bin", dtype=np.uint8).reshape(K, N)
        assert np.array_equal(qw, qw_ref), i
        assert np.array_equal(s, s_ref.view(np.uint16)) and np.array_equal(z, z_ref.view(np.uint16)), i
        assert np.array_equal(c, oracle.unpack(qw_ref, lay)), i
