"""GPU: w4a16_autotune times the plans of a shape on the device and the dispatcher then takes
the winner; results stay at the oracle's bar (|y - y_ref| <= 1e-2 + 5e-3 |y_ref|, y_ref in
fp64) and are bitwise equal to the same plan forced. w4a16_set_plan installs a plan the same
way."""
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
    L.w4a16_clear_plans()
    yield L
    L.w4a16_clear_plans()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def check_y(y_gpu, y_ref, what):
    y = y_gpu.detach().cpu().numpy().astype(np.float64)
    err = np.abs(y - y_ref)
    assert np.all(np.isfinite(y)), what
    assert np.all(err <= ATOL + RTOL * np.abs(y_ref)), f"{what}: max err {err.max():.3e}"


def inputs(M, K, N):
    wid = synth.WORKLOADS["decode_chain_7b"]["wid"]
    qw, s, z = oracle.quantize_pack(synth.weight(K, N, wid=wid, layer=7))
    x = synth.activations(M, K, wid=wid)
    return x, qw, s, z


# a narrow projection (the decode kernel only), a ragged strip count at K = 2560, and M = 32
# (decode-kernel plans and the prefill tile's split counts compete)
TUNE_CASES = [(1, 4096, 1024), (3, 2560, 1408), (32, 2048, 2048)]


@pytest.mark.parametrize("M,K,N", TUNE_CASES, ids=[f"M{m}-K{k}-N{n}" for m, k, n in TUNE_CASES])
def test_autotune_then_dispatch(lib, M, K, N):
    x, qw, s, z = inputs(M, K, N)
    d = [dev(a) for a in (x, qw, s, z)]
    y_ref = oracle.matmul(x, qw, s, z)
    default = lib.w4a16_plan(M, N, K)
    print(f"\n[autotune] M={M} K={K} N={N} default {default}", flush=True)
    try:
        y0 = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        plan, sec = lib.w4a16_autotune(*d, y=y0)
        print(f"[autotune] chose {plan} at {sec * 1e6:.2f} us per call", flush=True)
        assert 1e-7 < sec < 1e-2
        check_y(y0, y_ref, "y written by w4a16_autotune")
        assert lib.w4a16_plan(M, N, K) == plan
        y1 = lib.w4a16_matmul(*d)
        y2 = lib.w4a16_matmul(*d, plan=plan)
        torch.cuda.synchronize()
        check_y(y1, y_ref, "dispatcher after tuning")
        assert torch.equal(y1, y2)
        assert torch.equal(y0, y1)
        lib.w4a16_clear_plans()
        assert lib.w4a16_plan(M, N, K) == default
    finally:
        lib.w4a16_clear_plans()


def test_set_plan_is_taken_by_every_entry_point(lib):
    M, K, N = 2, 4096, 1024
    x, qw, s, z = inputs(M, K, N)
    d = [dev(a) for a in (x, qw, s, z)]
    y_ref = oracle.matmul(x, qw, s, z)
    plan = lib.w4a16_plan(M, N, K, kernel=lib.W4A16_KERNEL_SKINNY, cols=32, waves=8, kc=4, seg=4)
    assert plan["splits"] > 1 and plan != lib.w4a16_plan(M, N, K)
    try:
        lib.w4a16_set_plan(M, N, K, plan)
        forced = lib.w4a16_matmul(*d, plan=plan)
        auto = lib.w4a16_matmul(*d)
        noalloc = torch.empty_like(forced)
        lib.w4a16_matmul_noalloc(*d, noalloc)
        grouped = lib.w4a16_matmul_grouped(d[0], [tuple(d[1:])])[0]
        torch.cuda.synchronize()
        check_y(auto, y_ref, "set plan")
        for y, what in [(auto, "w4a16_matmul"), (noalloc, "w4a16_matmul_noalloc"), (grouped, "w4a16_matmul_grouped")]:
            assert torch.equal(y, forced), what
    finally:
        lib.w4a16_clear_plans()


def test_autotune_other_formats(lib):
    """The interleaved layout and 64-row groups: the tuned plan is kept per (M, N, K, group
    size) and the results stay at the bar."""
    M, K, N = 2, 2048, 1536
    wid = synth.WORKLOADS["decode_chain_7b"]["wid"]
    W = synth.weight(K, N, wid=wid, layer=9)
    try:
        for layout, g in (("interleaved", 128), ("linear", 64)):
            qw, s, z = oracle.quantize_pack(W, g, layout=layout)
            x = synth.activations(M, K, wid=wid)
            d = [dev(a) for a in (x, qw, s, z)]
            plan, sec = lib.w4a16_autotune(*d, group_size=g, layout=layout)
            print(f"\n[autotune] {layout} g={g}: {plan} at {sec * 1e6:.2f} us", flush=True)
            assert lib.w4a16_plan(M, N, K, group_size=g) == plan
            y = lib.w4a16_matmul(*d, group_size=g, layout=layout)
            torch.cuda.synchronize()
            check_y(y, oracle.matmul(x, qw, s, z, g, layout=layout), f"{layout} g={g}")
    finally:
        lib.w4a16_clear_plans()
