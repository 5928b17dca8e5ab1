"""GPU parity of w4a16_matmul_grouped: several weight matrices in one launch, sharing x or each
with its own.

Each y_i must equal, bit for bit, a w4a16_matmul_fmt call on its own matrix under the plan
the grouped call used (same kernel, strip width, waves, K range per wavefront, splits), and
meet the oracle's bar (|y - y_ref| <= 1e-2 + 5e-3 |y_ref|).
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


CASES = [
    # (name, M, K, [N_i], group, layout, forced plan)
    ("qkv-4096", 1, 4096, [4096, 4096, 4096], 128, "linear", None),
    ("qkv-4096-M4", 4, 4096, [4096, 4096, 4096], 128, "interleaved", None),
    ("qkv-4096-M16", 16, 4096, [4096, 4096, 4096], 128, "linear", None),
    ("gate-up", 1, 4096, [14336, 14336], 128, "linear", None),
    ("gate-up-M8", 8, 4096, [14336, 14336], 128, "interleaved", None),
    ("ragged-c16", 5, 2048, [1408, 2052, 768, 4], 128, "linear", dict(kernel=1, cols=16)),
    ("ragged-c32-split", 5, 2048, [1408, 2052, 768, 4], 64, "linear", dict(kernel=1, cols=32, kc=4, waves=4)),
    ("ragged-c64-split", 37, 2048, [1412, 260, 68], 32, "interleaved", dict(kernel=1, cols=64, kc=8, waves=4)),
    ("deep-split", 2, 14336, [4096, 1024], 256, "linear", None),
    ("one-matrix", 3, 768, [2048], 128, "linear", None),
]


def _inputs(name, K, Ns, g, layout):
    mats = []
    for i, N in enumerate(Ns):
        W = synth.weight_custom(K, N, seed=70 + 7 * i + len(name), std=0.02)
        mats.append(oracle.quantize_pack(W, g, layout=layout))
    return mats


@pytest.mark.parametrize("name,M,K,Ns,g,layout,plan", CASES, ids=[c[0] for c in CASES])
def test_grouped_matches_single_calls_and_oracle(lib, name, M, K, Ns, g, layout, plan):
    mats = _inputs(name, K, Ns, g, layout)
    x = synth.activations(M, K, wid=12)
    pl = lib.w4a16_plan(M, sum(Ns), K, group_size=g, **(plan or {}))
    print(f"\n[grouped] {name} M={M} K={K} N={Ns} g={g} {layout} plan={pl}", flush=True)
    xd = dev(x)
    dmats = [(dev(q), dev(s), dev(z)) for q, s, z in mats]
    ys = lib.w4a16_matmul_grouped(xd, dmats, group_size=g, plan=plan, layout=layout)
    torch.cuda.synchronize()
    for i, ((q, s, z), (qd, sd, zd), y) in enumerate(zip(mats, dmats, ys)):
        single = lib.w4a16_matmul(xd, qd, sd, zd, group_size=g, layout=layout,
                                  plan={k: v for k, v in pl.items() if k != "tile"} if pl["kernel"] == 1 else None)
        torch.cuda.synchronize()
        if pl["kernel"] == 1:
            assert torch.equal(y.view(torch.int16), single.view(torch.int16)), (name, i)
        y_ref = oracle.matmul(x, q, s, z, g, layout=layout)
        err = np.abs(y.cpu().numpy().astype(np.float64) - y_ref)
        assert np.all(err <= 1e-2 + 5e-3 * np.abs(y_ref)), (name, i, err.max())


def test_grouped_prefill_sized_launches_per_matrix(lib):
    """Where the summed shape selects the prefill kernel, every matrix is launched on its own
    with its own plan; the results still meet the oracle's bar."""
    M, K, Ns = 200, 1024, [520, 1032, 264]
    mats = _inputs("prefill", K, Ns, 128, "linear")
    x = synth.activations(M, K, wid=12)
    assert lib.w4a16_plan(M, sum(Ns), K)["kernel"] == 2
    ys = lib.w4a16_matmul_grouped(dev(x), [(dev(q), dev(s), dev(z)) for q, s, z in mats])
    torch.cuda.synchronize()
    for (q, s, z), y in zip(mats, ys):
        y_ref = oracle.matmul(x, q, s, z)
        err = np.abs(y.cpu().numpy().astype(np.float64) - y_ref)
        assert np.all(err <= 1e-2 + 5e-3 * np.abs(y_ref)), err.max()


def test_grouped_repeated_calls_bitwise(lib):
    """Split-K arrival counters shared by all matrices of a launch return to zero: repeated
    grouped calls, alternating with single calls on the stream, give the same bits."""
    M, K, Ns = 4, 14336, [4096, 2048, 4096]
    mats = _inputs("repeat", K, Ns, 128, "linear")
    x = dev(synth.activations(M, K, wid=12))
    dmats = [(dev(q), dev(s), dev(z)) for q, s, z in mats]
    assert lib.w4a16_plan(M, sum(Ns), K)["splits"] > 1
    first = [y.clone() for y in lib.w4a16_matmul_grouped(x, dmats)]
    for _ in range(4):
        lib.w4a16_matmul(x, *dmats[1])
        ys = lib.w4a16_matmul_grouped(x, dmats)
        torch.cuda.synchronize()
        for a, b in zip(first, ys):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# mixture-of-experts layers at decode: the gate and up projections of the active experts read
# one token (shared x); each expert's down projection reads its own input
MOE_CASES = [
    # (name, M, K, N, experts, own x per matrix (True / False / "mixed"), group, layout, forced plan)
    ("moe-gate-up-16", 1, 2048, 768, 16, False, 128, "linear", None),
    ("moe-down-8-own-x", 1, 768, 2048, 8, True, 128, "linear", None),
    ("moe-down-4-own-x-M4", 4, 1408, 2048, 4, True, 64, "interleaved", None),
    ("moe-mixed-split", 3, 2048, 1408, 6, "mixed", 128, "linear", dict(kernel=1, cols=16, kc=8, waves=4)),
    ("own-x-row-blocks", 80, 1024, 264, 3, True, 128, "linear", None),
    ("own-x-prefill", 200, 1024, 264, 3, True, 128, "linear", None),
]


@pytest.mark.parametrize("name,M,K,N,E,own,g,layout,plan", MOE_CASES, ids=[c[0] for c in MOE_CASES])
def test_grouped_experts_with_their_own_inputs(lib, name, M, K, N, E, own, g, layout, plan):
    """Up to 16 matrices in one call, each with the call's x or its own: every y_i equals, bit
    for bit, a single call on (x_i, W_i) under the plan the grouped call used (decode kernel),
    and meets the oracle's bar against x_i."""
    mats = _inputs(name, K, [N] * E, g, layout)
    xs = [synth.activations(M, K, wid=20 + i) for i in range(E)]
    x0 = synth.activations(M, K, wid=12)
    use_own = [own is True or (own == "mixed" and i % 2 == 1) for i in range(E)]
    pl = lib.w4a16_plan(M, N * E, K, group_size=g, **(plan or {}))
    print(f"\n[grouped-own-x] {name} M={M} K={K} N={N} x{E} own={own} plan={pl}", flush=True)
    dx0 = dev(x0)
    dxs = [dev(x) for x in xs]
    dmats = [(dev(q), dev(s), dev(z)) + ((dxs[i],) if use_own[i] else ()) for i, (q, s, z) in enumerate(mats)]
    ys = lib.w4a16_matmul_grouped(dx0, dmats, group_size=g, plan=plan, layout=layout)
    torch.cuda.synchronize()
    for i, ((q, s, z), y) in enumerate(zip(mats, ys)):
        xi, dxi = (xs[i], dxs[i]) if use_own[i] else (x0, dx0)
        if pl["kernel"] == 1:
            single = lib.w4a16_matmul(dxi, *dmats[i][:3], group_size=g, layout=layout,
                                      plan={k: v for k, v in pl.items() if k != "tile"})
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), single.view(torch.int16)), (name, i)
        y_ref = oracle.matmul(xi, q, s, z, g, layout=layout)
        err = np.abs(y.cpu().numpy().astype(np.float64) - y_ref)
        assert np.all(err <= 1e-2 + 5e-3 * np.abs(y_ref)), (name, i, err.max())


# experts that each see their own number of tokens (a batch routed over the active experts)
ROW_CASES = [
    # (name, K, N, rows per matrix, group, layout, forced plan)
    ("tokens-16-over-8", 2048, 1408, [3, 1, 5, 2, 16, 1, 4, 2], 128, "linear", None),
    ("rows-split", 4096, 520, [40, 7, 17, 1, 33], 64, "interleaved", dict(kernel=1, cols=16, kc=8, waves=4)),
    ("rows-two-row-tiles", 1024, 264, [64, 20, 1, 47], 128, "linear", dict(kernel=1, cols=32, kc=8, waves=4,
                                                                            row_tiles=2)),
    ("rows-prefill", 1024, 264, [200, 64, 130], 128, "linear", None),
]


@pytest.mark.parametrize("name,K,N,rows,g,layout,plan", ROW_CASES, ids=[c[0] for c in ROW_CASES])
def test_grouped_matrices_with_their_own_row_counts(lib, name, K, N, rows, g, layout, plan):
    """Each matrix with its own x of M_i <= M rows (M = the largest): y_i has M_i rows, equal
    bit for bit to a single call on (x_i, W_i) under the grouped call's plan (decode kernel)
    and within the oracle's bar."""
    M = max(rows)
    mats = _inputs(name, K, [N] * len(rows), g, layout)
    xs = [synth.activations(m, K, wid=40 + i) for i, m in enumerate(rows)]
    big = [i for i, m in enumerate(rows) if m == M][0]
    pl = lib.w4a16_plan(M, N * len(rows), K, group_size=g, **(plan or {}))
    print(f"\n[grouped-rows] {name} rows={rows} K={K} N={N} plan={pl}", flush=True)
    dxs = [dev(x) for x in xs]
    dmats = [(dev(q), dev(s), dev(z), dxs[i]) for i, (q, s, z) in enumerate(mats)]
    ys = lib.w4a16_matmul_grouped(dxs[big], dmats, group_size=g, plan=plan, layout=layout)
    torch.cuda.synchronize()
    for i, ((q, s, z), y) in enumerate(zip(mats, ys)):
        assert tuple(y.shape) == (rows[i], N)
        if pl["kernel"] == 1:
            single = lib.w4a16_matmul(dxs[i], *dmats[i][:3], group_size=g, layout=layout,
                                      plan={k: v for k, v in pl.items() if k != "tile"})
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), single.view(torch.int16)), (name, i)
        y_ref = oracle.matmul(xs[i], q, s, z, g, layout=layout)
        err = np.abs(y.cpu().numpy().astype(np.float64) - y_ref)
        assert np.all(err <= 1e-2 + 5e-3 * np.abs(y_ref)), (name, i, err.max())
