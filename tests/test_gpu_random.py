"""Seeded random shapes, formats and plans against the oracle (needs an MI355X).

Each case draws M, K, N, the group size, the layout and a plan (automatic, the decode
kernel, or one of the three prefill tiles with or without split-K) from a fixed seed, so
the set is reproducible; together they reach ragged M and N, every work-group tile height
and every kernel. Bar: |err| <= 1e-2 + 5e-3 |y_ref| against the fp64 oracle.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import weight_only_bit_gemv_amd as L
    return L


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def check_y(y_gpu, y_ref, what):
    y = y_gpu.detach().cpu().numpy().astype(np.float64)
    err = np.abs(y - y_ref)
    bound = 1e-2 + 5e-3 * np.abs(y_ref)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert np.all(err <= bound), f"{what}: max err {err.max():.3e}"


def _w4a16_cases(count=40, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        g = int(rng.choice([32, 64, 128, 256]))
        K = int(rng.integers(1, 13)) * max(g, 128)
        N = 4 * int(rng.integers(1, 520))
        M = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 130)), int(rng.integers(130, 300))]))
        layout = str(rng.choice(["linear", "interleaved"]))
        kind = str(rng.choice(["auto", "skinny", "async", "async_split", "lds", "register"]))
        if kind.startswith("async") and N % 8:
            N += 4
        plan = {"auto": None, "skinny": dict(kernel=1), "async": dict(kernel=2, tile=3),
                "async_split": dict(kernel=2, tile=3, splits=int(rng.integers(2, 5))),
                "lds": dict(kernel=2, tile=1), "register": dict(kernel=2, tile=2)}[kind]
        if kind == "async_split" and plan["splits"] > K // 128:
            plan["splits"] = K // 128
        cases.append((i, M, K, N, g, layout, kind, plan))
    return cases


W4A16_CASES = _w4a16_cases()


@pytest.mark.parametrize("case", W4A16_CASES, ids=[f"c{c[0]}-{c[6]}-M{c[1]}-K{c[2]}-N{c[3]}-g{c[4]}-{c[5][:3]}" for c in W4A16_CASES])
def test_random_w4a16(lib, case):
    i, M, K, N, g, layout, kind, plan = case
    print(f"\n[random w4a16] {case}", flush=True)
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=3000 + i, std=0.02), g, bool(i % 3 == 0), layout)
    x = synth.activations(M, K, wid=9)
    y = lib.w4a16_matmul(dev(x), dev(qw), dev(s), dev(z), plan=plan, group_size=g, layout=layout)
    check_y(y, oracle.matmul(x, qw, s, z, g, layout=layout), f"w4a16 {case}")


def _deep_cases(count=16, seed=2026):
    """Decode-sized M with K up to 16384 and N up to 6144, on the dispatcher's plan: the
    shapes outside its table that take the split-K branch of its rule (K > 4096)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        g = int(rng.choice([64, 128, 256]))
        K = 256 * int(rng.integers(17, 65))
        N = 4 * int(rng.integers(1, 1537))
        M = int(rng.integers(1, 17))
        layout = str(rng.choice(["linear", "interleaved"]))
        cases.append((i, M, K, N, g, layout))
    return cases


DEEP_CASES = _deep_cases()


@pytest.mark.parametrize("case", DEEP_CASES, ids=[f"c{c[0]}-M{c[1]}-K{c[2]}-N{c[3]}-g{c[4]}-{c[5][:3]}" for c in DEEP_CASES])
def test_random_deep_k_dispatcher_plan(lib, case):
    i, M, K, N, g, layout = case
    print(f"\n[random deep] {case} plan={lib.w4a16_plan(M, N, K, group_size=g)}", flush=True)
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=5000 + i, std=0.02), g, bool(i % 3 == 0), layout)
    x = synth.activations(M, K, wid=9)
    y = lib.w4a16_matmul(dev(x), dev(qw), dev(s), dev(z), group_size=g, layout=layout)
    rng = np.random.default_rng((6, i))
    cols = np.unique(np.concatenate([rng.choice(N, size=min(N, 96), replace=False), [0, N - 1]]))
    ref = oracle.matmul(x, qw[:, cols], s[:, cols], z[:, cols], g, layout=layout)
    check_y(y[:, torch.from_numpy(cols).to(DEV)], ref, f"deep {case}")


def _w4a8_cases(count=24, seed=2025):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        g = int(rng.choice([128, 256]))
        K = int(rng.integers(1, 13)) * g
        N = 8 * int(rng.integers(1, 260))
        M = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 65)), int(rng.integers(65, 300))]))
        layout = str(rng.choice(["linear", "interleaved"]))
        splits = int(rng.choice([0, 0, 1, 2, 3]))
        splits = min(splits, K // 128)
        cases.append((i, M, K, N, g, layout, splits))
    return cases


W4A8_CASES = _w4a8_cases()


@pytest.mark.parametrize("case", W4A8_CASES, ids=[f"c{c[0]}-M{c[1]}-K{c[2]}-N{c[3]}-g{c[4]}-{c[5][:3]}-S{c[6]}" for c in W4A8_CASES])
def test_random_w4a8(lib, case):
    i, M, K, N, g, layout, splits = case
    print(f"\n[random w4a8] {case}", flush=True)
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=4000 + i, std=0.02), g, bool(i % 3 == 0), layout)
    x = synth.activations(M, K, wid=9)
    xq, sx = oracle.quantize_activations(x)
    S = oracle.activation_block_sums(xq)
    xsum = np.zeros((S.shape[0], (M + 3) // 4 * 4), dtype=np.float32)
    xsum[:, :M] = S
    y = lib.w4a8_matmul(dev(xq), dev(sx), dev(xsum), dev(qw), dev(s), dev(z), group_size=g, layout=layout, splits=splits)
    check_y(y, oracle.matmul_w4a8(xq, sx, qw, s, z, g, layout), f"w4a8 {case}")
