"""Split-K calls on several streams at once (needs an MI355X).

The library keeps one split-K workspace (fp32 partials and arrival counters) per (device,
stream). Calls enqueued on two streams without synchronising between them run
concurrently; each must give the bits of the same call made alone, so neither stream's
partials or counters may be touched by the other's kernels.
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


# (M, K, N, plan): decode split-K (4 splits), async prefill split-K, a second decode split-K
CALLS = [(4, 14336, 4096, None), (130, 4096, 1032, dict(kernel=2, tile=3, splits=4)),
         (1, 8192, 2048, dict(kernel=1, cols=16, kc=8, waves=4))]


def test_concurrent_streams_match_lone_calls(lib):
    data = []
    for i, (M, K, N, plan) in enumerate(CALLS):
        qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=120 + i, std=0.02))
        x = synth.activations(M, K, wid=13)
        data.append((x, qw, s, z, [dev(x), dev(qw), dev(s), dev(z)], plan))
        print(f"\n[streams] call {i}: M={M} K={K} N={N} plan={lib.w4a16_plan(M, N, K, **(plan or {}))}", flush=True)
    alone = []
    for x, qw, s, z, args, plan in data:
        alone.append(lib.w4a16_matmul(*args, plan=plan).clone())
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    for st in streams:                                           # size each stream's workspace
        with torch.cuda.stream(st):
            for _, _, _, _, args, plan in data:
                lib.w4a16_matmul(*args, plan=plan)
    torch.cuda.synchronize()
    outs = [[torch.empty_like(a) for a in alone] for _ in streams]
    for rep in range(6):
        for j, st in enumerate(streams):                         # interleaved enqueues, no sync
            with torch.cuda.stream(st):
                for (_, _, _, _, args, plan), y in zip(data[::1 if (rep + j) % 2 == 0 else -1],
                                                       outs[j][::1 if (rep + j) % 2 == 0 else -1]):
                    lib.w4a16_matmul(*args, y=y, plan=plan)
        torch.cuda.synchronize()
        for j in range(len(streams)):
            for i, (y, a) in enumerate(zip(outs[j], alone)):
                assert torch.equal(y.view(torch.int16), a.view(torch.int16)), (rep, j, i)
    for (x, qw, s, z, _, _), a in zip(data, alone):
        ref = oracle.matmul(x, qw, s, z)
        assert np.all(np.abs(a.cpu().numpy().astype(np.float64) - ref) <= 1e-2 + 5e-3 * np.abs(ref))


def test_concurrent_streams_w4a8(lib):
    """The same for the W4A8 pair (quantiser and split-K product) on two streams."""
    M, K, N = 64, 4096, 520
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=130, std=0.02))
    w = [dev(qw), dev(s), dev(z)]
    xs = [dev(synth.activations(M, K, wid=14 + j)) for j in range(2)]
    alone = []
    for x in xs:
        q, sx, xsum = lib.w4a8_quantize(x)
        alone.append(lib.w4a8_matmul(q, sx, xsum, *w, splits=8).clone())
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    for rep in range(6):
        ys = []
        for x, st in zip(xs, streams):
            with torch.cuda.stream(st):
                q, sx, xsum = lib.w4a8_quantize(x)
                ys.append(lib.w4a8_matmul(q, sx, xsum, *w, splits=8))
        torch.cuda.synchronize()
        for j, (y, a) in enumerate(zip(ys, alone)):
            assert torch.equal(y.view(torch.int16), a.view(torch.int16)), (rep, j)
