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
