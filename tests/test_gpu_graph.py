"""HIP graph capture of w4a16_matmul, grouped launches and the W4A8 pair (needs an MI355X).

A captured call is replayed several times, with eager calls of other shapes on the same
stream between the replays (they take and release the same split-K arrival counters, and
one of them grows the stream's workspace after the capture); every replay must give the
eager call's bits. A split-K call captured before any call of its shape on the stream must
fail cleanly and leave the capture usable.
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


def _problem(M, K, N, seed):
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=seed, std=0.02))
    x = synth.activations(M, K, wid=9)
    return x, qw, s, z, [dev(x), dev(qw), dev(s), dev(z)]


# (M, K, N, plan): the decode kernel with and without split-K, the async prefill tile with
# and without split-K
CASES = [(4, 14336, 4096, None), (1, 4096, 4096, None), (130, 2048, 520, dict(kernel=2, tile=3, splits=3)),
         (300, 1024, 1032, dict(kernel=2, tile=3, splits=1))]


@pytest.mark.parametrize("M,K,N,plan", CASES, ids=[f"M{m}-K{k}-N{n}" for m, k, n, _ in CASES])
def test_graph_replays_match_eager(lib, M, K, N, plan):
    print(f"\n[graph] M={M} K={K} N={N} plan={lib.w4a16_plan(M, N, K, **(plan or {}))}", flush=True)
    x, qw, s, z, args = _problem(M, K, N, seed=M + K)
    st = torch.cuda.Stream()
    y_ref = torch.empty((M, N), dtype=torch.float16, device=DEV)
    with torch.cuda.stream(st):
        lib.w4a16_matmul(*args, y=y_ref, plan=plan)           # eager; sizes the workspace
    st.synchronize()
    y_g = torch.zeros_like(y_ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        lib.w4a16_matmul(*args, y=y_g, plan=plan)
    # other calls on the same stream between replays: a decode split-K call, then a prefill
    # split-K call whose partials need a larger workspace than any made so far
    others = [(8, 14336, 4096, None), (256, 8192, 2048, dict(kernel=2, tile=3, splits=8))]
    other_data = [(_problem(m, k, n, seed=7 * m)[4], m, n, p) for m, k, n, p in others]
    for rep in range(4):
        y_g.fill_(7.0)                                           # a kernel, not a memset
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g.view(torch.int16), y_ref.view(torch.int16)), f"replay {rep}"
        a, m, n, p = other_data[rep % 2]
        with torch.cuda.stream(st):
            lib.w4a16_matmul(*a, plan=p)
        st.synchronize()
    y = y_ref.cpu().numpy().astype(np.float64)
    ref = oracle.matmul(x, qw, s, z)
    assert np.all(np.abs(y - ref) <= 1e-2 + 5e-3 * np.abs(ref))


def _fresh_stream():
    """A stream no call has used (torch.cuda.Stream() hands out pooled streams), created with
    the HIP runtime torch has loaded, at the default priority."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    h = ctypes.c_void_p()
    assert hip.hipStreamCreate(ctypes.byref(h)) == 0
    return hip, h, torch.cuda.ExternalStream(h.value, device=DEV)


def test_split_k_capture_without_workspace_fails_cleanly(lib):
    M, K, N = 64, 4096, 256
    plan = dict(kernel=2, tile=3, splits=4)
    print(f"\n[graph] capture without workspace plan={lib.w4a16_plan(M, N, K, **plan)}", flush=True)
    x, qw, s, z, args = _problem(M, K, N, seed=11)
    hip, handle, st = _fresh_stream()                             # no call on it yet
    y_bad = torch.zeros((M, N), dtype=torch.float16, device=DEV)
    y_ok = torch.zeros((M, N), dtype=torch.float16, device=DEV)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        with pytest.raises(lib.W4A16Error) as e:
            lib.w4a16_matmul(*args, y=y_bad, plan=plan)
        lib.w4a16_matmul(*args, y=y_ok, plan=dict(kernel=2, tile=3, splits=1))   # no workspace needed
    assert e.value.code == lib.W4A16_ERR_HIP and "capture" in str(e.value)
    g.replay()
    torch.cuda.synchronize()
    ref = oracle.matmul(x, qw, s, z)
    y = y_ok.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(y - ref) <= 1e-2 + 5e-3 * np.abs(ref))
    assert not torch.any(y_bad != 0)                              # the failed call enqueued nothing
    del g
    torch.cuda.synchronize()
    assert hip.hipStreamDestroy(handle) == 0


def _replay_against_eager(g, outs, refs, between):
    """Replay g four times, `between()` (eager calls on the capture stream) after each, and
    check every output against the eager result bit for bit."""
    for rep in range(4):
        for y in outs:
            y.fill_(7.0)                                         # a kernel, not a memset
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (y, r) in enumerate(zip(outs, refs)):
            assert torch.equal(y.view(torch.int16), r.view(torch.int16)), f"replay {rep} output {i}"
        between(rep)


@pytest.mark.parametrize("own_x,plan", [(False, None), (True, dict(kernel=1, cols=16, kc=8, waves=4)),
                                       (True, None)], ids=["shared-x", "own-x-split", "own-x"])
def test_grouped_graph_replays_match_eager(lib, own_x, plan):
    """A grouped launch (q/k/v-like with one x, or experts with their own) captured and
    replayed, with a single-matrix split-K call and a grouped call of the other kind on the
    stream between the replays."""
    M, K, Ns = 2, 2048, ([1408] * 6 if own_x else [2048, 512, 512])
    mats = [oracle.quantize_pack(synth.weight_custom(K, N, seed=90 + i, std=0.02)) for i, N in enumerate(Ns)]
    xs = [dev(synth.activations(M, K, wid=30 + i)) for i in range(len(Ns))]
    dmats = [(dev(q), dev(s), dev(z)) + ((xs[i],) if own_x else ()) for i, (q, s, z) in enumerate(mats)]
    print(f"\n[graph grouped] own_x={own_x} N={Ns} plan={lib.w4a16_plan(M, sum(Ns), K, **(plan or {}))}",
          flush=True)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        refs = [y.clone() for y in lib.w4a16_matmul_grouped(xs[0], dmats, plan=plan)]
    st.synchronize()
    outs = [torch.zeros_like(r) for r in refs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        lib.w4a16_matmul_grouped(xs[0], dmats, ys=outs, plan=plan)
    other = _problem(4, 14336, 4096, seed=5)[4]
    other_group = [d[:3] for d in dmats[:2]] if own_x else [d + (xs[1],) for d in dmats[:2]]

    def between(rep):
        with torch.cuda.stream(st):
            if rep % 2 == 0:
                lib.w4a16_matmul(*other)                             # decode split-K (4 splits)
            else:
                lib.w4a16_matmul_grouped(xs[0], other_group)
        st.synchronize()
    _replay_against_eager(g, outs, refs, between)


def test_w4a8_graph_replays_match_eager(lib):
    """The activation quantiser and a split-K W4A8 product captured together and replayed,
    with other W4A8 calls on the stream between the replays."""
    M, K, N = 100, 2048, 264
    qw, s, z = oracle.quantize_pack(synth.weight_custom(K, N, seed=44, std=0.02))
    w = [dev(qw), dev(s), dev(z)]
    x = dev(synth.activations(M, K, wid=8))
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        xq, sx, xsum = lib.w4a8_quantize(x)
        ref = lib.w4a8_matmul(xq, sx, xsum, *w, splits=4).clone()
    st.synchronize()
    y = torch.zeros_like(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        a, b, c = lib.w4a8_quantize(x)
        lib.w4a8_matmul(a, b, c, *w, y=y, splits=4)
    qw2, s2, z2 = oracle.quantize_pack(synth.weight_custom(4096, 1032, seed=45, std=0.02))
    w2 = [dev(qw2), dev(s2), dev(z2)]
    x2 = dev(synth.activations(7, 4096, wid=8))

    def between(rep):
        with torch.cuda.stream(st):
            q3, s3, c3 = lib.w4a8_quantize(x2)
            lib.w4a8_matmul(q3, s3, c3, *w2, splits=8 if rep % 2 else 1)
        st.synchronize()
    _replay_against_eager(g, [y], [ref], between)
    # the captured quantiser's outputs too
    assert torch.equal(a, xq) and torch.equal(b.view(torch.int32), sx.view(torch.int32))
    assert torch.equal(c.view(torch.int32), xsum.view(torch.int32))


def test_set_plan_is_captured(lib):
    """A plan installed with w4a16_set_plan (here one with split-K) is what a captured call of
    that shape takes: every replay gives the bits of the same plan forced in an eager call."""
    M, K, N = 3, 4096, 2048
    plan = lib.w4a16_plan(M, N, K, kernel=lib.W4A16_KERNEL_SKINNY, cols=64, waves=4, kc=8)
    assert plan["splits"] > 1
    x, qw, s, z, args = _problem(M, K, N, seed=77)
    st = torch.cuda.Stream()
    try:
        lib.w4a16_set_plan(M, N, K, plan)
        y_ref = torch.empty((M, N), dtype=torch.float16, device=DEV)
        with torch.cuda.stream(st):
            lib.w4a16_matmul(*args, y=y_ref, plan=plan)       # eager, forced; sizes the workspace
        st.synchronize()
        y_g = torch.zeros_like(y_ref)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            lib.w4a16_matmul(*args, y=y_g)                     # the dispatcher's (installed) plan
        for rep in range(3):
            y_g.fill_(7.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_g.view(torch.int16), y_ref.view(torch.int16)), f"replay {rep}"
    finally:
        lib.w4a16_clear_plans()
    y = y_ref.cpu().numpy().astype(np.float64)
    ref = oracle.matmul(x, qw, s, z)
    assert np.all(np.abs(y - ref) <= 1e-2 + 5e-3 * np.abs(ref))
