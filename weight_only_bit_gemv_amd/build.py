"""Build libw4a16.so in-tree: HIP kernels for gfx950 with hipcc, host code with g++.

    python -m weight_only_bit_gemv_amd.build        (or __graft_entry__.build())

Output: weight_only_bit_gemv_amd/lib/libw4a16.so (and lib/w4a16_capi_driver, a test program
that calls the library through its C ABI only). Objects go to weight_only_bit_gemv_amd/_build/.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libw4a16.so")
# a test program that drives the library through the C ABI alone (tests/test_gpu_capi.py)
CAPI_DRIVER_SRC = os.path.join(ROOT, "tests", "capi", "capi_driver.cpp")
CAPI_DRIVER = os.path.join(LIBDIR, "w4a16_capi_driver")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_SOURCES = ["w4a16_skinny.hip", "w4a16_skinny_lw1.hip", "w4a16_skinny_lw2.hip", "w4a16_skinny_lw4.hip",
               "w4a16_prefill.hip", "w4a16_prefill_rb.hip", "w4a16_prefill_async.hip",
               "w4a16_dequant.hip", "w4a8_prefill.hip", "w4a16_noalloc.hip",
               "w4a16_readbw.hip"]
# The packer must round every fp32 step on its own: no contraction, no fast-math.
PACK_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math"]
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep packed-fp32 VALU instructions out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# MFMA accumulators in ordinary VGPRs for every kernel: in AGPRs the compiler copies
# accumulators between register files inside the prefill loops (accvgpr moves), which
# costs more than the registers it frees.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
PER_FILE_FLAGS = {}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that line
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False):
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        jobs.append([hipcc] + HIPCC_FLAGS + PER_FILE_FLAGS.get(src, VGPR_FORM) + inc +
                    ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    obj = os.path.join(BUILD, "w4a16_pack.o")
    jobs.append(["g++", "-std=c++17", "-fPIC"] + PACK_FLAGS + inc +
                ["-c", os.path.join(CSRC, "w4a16_pack.cpp"), "-o", obj])
    objs.append(obj)
    obj = os.path.join(BUILD, "w4a16_api.o")
    jobs.append(["g++", "-std=c++17", "-fPIC", "-O2", "-D__HIP_PLATFORM_AMD__",
                 "-I", os.path.join(ROCM, "include")] + inc +
                ["-c", os.path.join(CSRC, "w4a16_api.cpp"), "-o", obj])
    objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs +
         ["-lpthread"])
    os.replace(tmp, LIB)
    if os.path.exists(CAPI_DRIVER_SRC):
        tmp = CAPI_DRIVER + ".tmp"
        _run([hipcc, "-O2", "-std=c++17", "-I", INCLUDE, CAPI_DRIVER_SRC, "-o", tmp, "-L", LIBDIR, "-lw4a16",
              "-Wl,-rpath,$ORIGIN"])
        os.replace(tmp, CAPI_DRIVER)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
