"""w4a16_matmul_noalloc (split-K partials in the library's static scratch, no allocation)
against w4a16_matmul_fmt (the per-stream workspace) through the C ABI: two calls in a row
on one stream, the second with a smaller input, each bitwise equal to the existing entry
point's result and within the oracle's bar."""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"

PAIRS = [
    # decode kernel with split-K: auto plan of 14336x4096 (4 splits), then a smaller forced split
    ("decode-split", [(4, 14336, 4096, None, "linear"),
                      (1, 4096, 1408, dict(kernel=1, cols=16, kc=4, waves=4), "interleaved")]),
    # async prefill tile with split-K: 128-row work-groups, then 64-row ones
    ("prefill-split", [(130, 4096, 1032, dict(kernel=2, tile=3, splits=4), "linear"),
                       (40, 2048, 264, dict(kernel=2, tile=3, splits=2), "linear")]),
    # the dispatcher's own plans, with and without split-K
    ("auto", [(16, 14336, 4096, None, "interleaved"), (1, 4096, 4096, None, "linear")]),
]


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import weight_only_bit_gemv_amd as L
    return L


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("name,calls", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_matches_allocating_entry_point(lib, name, calls):
    data = []
    for i, (M, K, N, plan, layout) in enumerate(calls):
        qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=60 + i, std=0.02), layout=layout)
        x = synth.activations(M, K, wid=11)
        print(f"\n[noalloc] {name} call {i}: M={M} K={K} N={N} {layout} "
              f"plan={lib.w4a16_plan(M, N, K, **(plan or {}))}", flush=True)
        data.append((x, qw, s, z, [dev(x), dev(qw), dev(s), dev(z)], plan, layout))
    outs = []
    for x, qw, s, z, args, plan, layout in data:          # two no-alloc calls in a row
        y = torch.full((x.shape[0], qw.shape[1]), float("nan"), dtype=torch.float16, device=DEV)
        outs.append(lib.w4a16_matmul_noalloc(*args, y, plan=plan, layout=layout))
    torch.cuda.synchronize()
    for (x, qw, s, z, args, plan, layout), y in zip(data, outs):
        ref = lib.w4a16_matmul(*args, plan=plan, layout=layout)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), name
        y_ref = oracle.matmul(x, qw, s, z, layout=layout)
        err = np.abs(y.cpu().numpy().astype(np.float64) - y_ref)
        assert np.all(err <= 1e-2 + 5e-3 * np.abs(y_ref)), (name, err.max())
    # and once more in the other order: the counters the first pair left are back at zero
    for (x, qw, s, z, args, plan, layout), y in reversed(list(zip(data, outs))):
        y2 = torch.empty_like(y)
        lib.w4a16_matmul_noalloc(*args, y2, plan=plan, layout=layout)
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.int16), y.view(torch.int16)), name


def test_noalloc_under_graph_capture(lib):
    """The callers it is for: a split-K call captured in a HIP graph (the first call on the
    device, which takes the scratch address and clears its counters, happens eagerly before)
    and replayed four times, with eager no-alloc calls of other shapes (sharing the scratch)
    on the stream between the replays; every replay gives the eager call's bits."""
    M, K, N = 4, 14336, 4096
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=66, std=0.02))
    args = [dev(synth.activations(M, K, wid=11)), dev(qw), dev(s), dev(z)]
    assert lib.w4a16_plan(M, N, K)["splits"] > 1
    q2, s2, z2 = oracle.quantize_pack(synth.weight_custom(4096, 1032, seed=67, std=0.02))
    other = [dev(synth.activations(130, 4096, wid=11)), dev(q2), dev(s2), dev(z2)]
    print(f"\n[noalloc graph] M={M} K={K} N={N} plan={lib.w4a16_plan(M, N, K)}", flush=True)
    st = torch.cuda.Stream()
    ref = torch.empty((M, N), dtype=torch.float16, device=DEV)
    y_other = torch.empty((130, 1032), dtype=torch.float16, device=DEV)
    with torch.cuda.stream(st):
        lib.w4a16_matmul_noalloc(*args, ref)
    st.synchronize()
    y = torch.zeros_like(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        lib.w4a16_matmul_noalloc(*args, y)
    for rep in range(4):
        y.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        with torch.cuda.stream(st):
            lib.w4a16_matmul_noalloc(*other, y_other, plan=dict(kernel=2, tile=3, splits=2 + rep))
        st.synchronize()
