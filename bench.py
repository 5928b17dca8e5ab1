"""Benchmark of the W4A16 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload `decode_sweep` (the JSON line the headline metric is quoted on): one step
= y = x . dequant(Wq) for M in {1,2,4,8,16} on each of (K, N) = (4096, 14336),
(14336, 4096), (4096, 4096), group 128 (15 launches). Inputs are seeded synthetic data
(synth.py) resident in HBM before timing; the packed weights rotate over enough distinct
device copies (>= 1 GiB per shape family) that no launch finds its weights in the 256 MB
Infinity Cache. The K timed steps are replayed from one HIP graph on one stream and
bracketed by HIP events on that stream; every replay is checked bit for bit against an
eager run.

Other workloads (same JSON keys, config.workload names them):
  gemv_4096     one M=1, 4096 x 4096 GEMV
  gemv_lm_head  one M=1, 4096 x 128256 GEMV (the 7B-shaped chain's lm_head, 279 MB)
  moe_expert    M in {1,4,16} on (2048,1408), (1408,2048), (2048,768), (768,2048)
  shard_8       M in {1,4,16} on one GPU's column share (N / 8) of the 7B-shaped projections
                and lm_head: (4096,512), (4096,1792), (14336,512), (4096,16032)
  chain_7b      batch-1 decode weight stream of a 32-layer 7B-shaped model + lm_head:
                225 GEMVs per token in one graph (one layer's weights packed once and
                copied into 32 distinct device buffers); also reports tokens/s
  prefill       M-crossover against torch fp16 matmul (hipBLASLt) for M = 1..2048 on
                (8192,8192), (8192,28672), (28672,8192) and the decode shapes

Printed: one JSON line. `value` is the algorithmic byte rate (int4 weights + fp16
scales/zeros + fp16 x + fp16 y) of one step over the median of up to 5 timed batches (the
K steps split into batches of graph replays, each between HIP events; the minimum is
reported too), in GB/s. `roofline` is the dominant kernel's line (the decode-kernel instance
with the most time per step): algorithmic bytes per launch over its average launch time,
each of its calls graph-timed with HIP events on the launch stream, against the 8 TB/s HBM
peak (MFMA peak for prefill), its fraction of the measured read ceiling (w4a16_read_probe
at each call's byte count, same timing), its HBM traffic per launch from the committed
counter summary, and, from the committed kernel-trace summary of the same sources, its
kernel-only rate; `roofline.step` gives the same for the whole step (all kernels); `grouped` times q/k/v and gate/up as one
grouped launch against one launch per matrix (decode_sweep), or the active experts' gate/up
(one shared x) and down projections (each its own x) of mixture-of-experts layers
(moe_expert); `cpu_baseline` times the oracle (NumPy, fp64)
on the host cores over passes of the decode sweep (about 10 s). --record FILE also writes
the line with the command, the sources' hash and the machine.

Profiling support:
  --trace-pass             only the timed decode-sweep steps, for rocprofv3 --kernel-trace
  --summarize-kernel-trace DIR...  per-call and per-instance kernel durations of such a run
                           -> profiles/kernel_trace_skinny_decode_sweep.{json,md}
  --pmc-pass               a fixed copy calibration + a few eager sweep steps, for
                           rocprofv3 --pmc; prints no JSON (with --workload prefill:
                           eager prefill-kernel launches at M=2048, K=8192, N=28672)
  --summarize-pmc DIR...   read rocprofv3 counter CSVs of --pmc-pass runs and write the
                           per-launch HBM traffic summary to profiles/
  --summarize-prefill-pmc DIR...  the same for the prefill counter runs (MFMA busy, LDS)
"""
import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak (8 TB/s)
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA peak
GROUP = 128
SWEEP_KN = [(4096, 14336), (14336, 4096), (4096, 4096)]
# one GPU's column share (N / 8) of the 7B-shaped projections and lm_head: tensor parallelism
# over 8 GPUs without any exchange inside the product
SHARD8_KN = [(4096, 512), (4096, 1792), (14336, 512), (4096, 16032)]
SWEEP_M = [1, 2, 4, 8, 16]
ROTATE_BYTES = 1 << 30         # >= 4x the 256 MB Infinity Cache per shape family
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_skinny_decode_sweep.json")
# sources that decide what the decode kernel does (kernel, unpack helpers, plan table): the
# committed traffic counters stay valid while these are unchanged
KERNEL_SOURCES = sorted(os.path.relpath(f, ROOT) for f in
                        glob.glob(os.path.join(ROOT, "weight_only_bit_gemv_amd", "csrc", "w4a16_skinny*")) +
                        [os.path.join(ROOT, "weight_only_bit_gemv_amd", "csrc", "w4a16_device.hpp")])
PREFILL_SOURCES = sorted(os.path.relpath(f, ROOT) for f in
                         glob.glob(os.path.join(ROOT, "weight_only_bit_gemv_amd", "csrc", "w4a16_prefill*")) +
                         [os.path.join(ROOT, "weight_only_bit_gemv_amd", "csrc", "w4a16_device.hpp")])
COPY_CAL_BYTES = 256 << 20     # calibration copy for the PMC byte counters
KTRACE_FILE = os.path.join(ROOT, "profiles", "kernel_trace_skinny_decode_sweep.json")
METRIC = "W4A16 weight-stream HBM GB/s (% of peak) and us/call at M=1..16"


def alg_bytes(M, K, N, group=GROUP):
    """Algorithmic bytes of one call: int4 weights, fp16 scales + zeros, fp16 x and y."""
    return K * N // 2 + 2 * 2 * (K // group) * N + 2 * M * K + 2 * M * N


def kernel_source_hash(sources=None):
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_kernel_hash():
    """What the decode sweep's traffic depends on: the decode kernel's sources and the plan the
    dispatcher picks for each of the sweep's calls (not the rest of the dispatcher's code)."""
    import weight_only_bit_gemv_amd as lib
    h = hashlib.sha256(kernel_source_hash().encode())
    for (M, K, N, _) in workload_items("decode_sweep")[1]:
        h.update(json.dumps(lib.w4a16_plan(M, N, K), sort_keys=True).encode())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------------------

class Runner:
    """Device-resident inputs for a list of GEMM launches.

    families: key -> (K, N, wid, layer); every family gets its own packed weights, copied
    until its copies total `rotate_bytes` (1 copy when rotate_bytes is 0).
    items: list of (M, K, N, family key), launched in order by step().
    """

    def __init__(self, torch, lib, dev, stream, families, items, rotate_bytes, replicate=None,
                 group=GROUP, symmetric=False, layout="linear"):
        self.torch, self.lib, self.dev, self.stream = torch, lib, dev, stream
        self.group, self.symmetric, self.layout = group, symmetric, layout
        self.layout_id = lib._binding._layout_id(layout)
        self.weights, self.host = {}, {}
        packed = {}
        for key, (K, N, wid, layer) in families.items():
            src = (replicate or {}).get(key)
            if src is not None and src in self.weights:     # same values, distinct memory
                self.weights[key] = [[t.clone() for t in self.weights[src][0]]]
                self.host[key] = self.host[src]
                continue
            t0 = time.time()
            if (K, N, wid, layer) not in packed:
                W = synth.weight(K, N, wid=wid, layer=layer)
                packed[(K, N, wid, layer)] = lib.w4a16_pack(W, group_size=group, symmetric=symmetric,
                                                            layout=layout)
                del W
            qw, s, z = packed[(K, N, wid, layer)]
            self.host[key] = (qw, s, z)
            one = [torch.from_numpy(a).to(dev) for a in (qw, s, z)]
            per = sum(t.numel() * t.element_size() for t in one)
            copies = max(1, -(-rotate_bytes // per)) if rotate_bytes else 1
            self.weights[key] = [one] + [[t.clone() for t in one] for _ in range(copies - 1)]
            log(f"[bench] weights {key} K={K} N={N}: {copies} x {per / 1e6:.1f} MB ({time.time() - t0:.1f}s)")
        self.items = items
        wids = {key: fam[2] for key, fam in families.items()}
        self.x = {}
        for (M, K, N, key) in items:
            if (M, K, wids[key]) not in self.x:
                self.x[(M, K, wids[key])] = torch.from_numpy(synth.activations(M, K, wid=wids[key])).to(dev)
        self.xk = [self.x[(M, K, wids[key])] for (M, K, N, key) in items]
        self.y = [torch.empty((M, N), dtype=torch.float16, device=dev) for (M, K, N, key) in items]
        self.cursor = {key: 0 for key in families}
        self.step_bytes = sum(alg_bytes(M, K, N, group) for (M, K, N, key) in items)
        self.fn = lib.load().w4a16_matmul_fmt
        self.plans = {}
        self.sptr = stream.cuda_stream

    def launch(self, i, plan=None):
        """Enqueue item i (the dispatcher's plan, or a forced plan: a dict of plan fields)."""
        M, K, N, key = self.items[i]
        c = self.cursor[key]
        self.cursor[key] = (c + 1) % len(self.weights[key])
        qw, s, z = self.weights[key][c]
        args = (self.xk[i].data_ptr(), qw.data_ptr(), s.data_ptr(), z.data_ptr(),
                self.y[i].data_ptr(), M, N, K, self.group, self.layout_id, self.sptr)
        if plan is None:
            rc = self.fn(*args, None)
        else:
            key_p = tuple(sorted(plan.items()))
            if key_p not in self.plans:
                self.plans[key_p] = self.lib._binding._make_plan(plan)
            rc = self.fn(*args, ctypes.byref(self.plans[key_p]))
        if rc != 0:
            raise RuntimeError(f"w4a16_matmul failed ({rc}) for M={M} K={K} N={N}")

    def step(self):
        for i in range(len(self.items)):
            self.launch(i)

    def launch_w4a8(self, i, quantize=False):
        """Enqueue item i on the W4A8 path: the per-row E4M3 activation quantiser (when
        `quantize`, else once, up front) and the 8-bit product, same weights as launch()."""
        M, K, N, key = self.items[i]
        so = self.lib.load()
        if not hasattr(self, "xq"):
            self.xq, self.sx, self.xsum = {}, {}, {}
        if quantize or i not in self.xq:
            if i not in self.xq:
                self.xq[i] = self.torch.empty((M, K), dtype=self.torch.uint8, device=self.dev)
                self.sx[i] = self.torch.empty((M,), dtype=self.torch.float32, device=self.dev)
                self.xsum[i] = self.torch.empty((K // 128, self.lib.w4a8_sum_stride(M)), dtype=self.torch.float32,
                                                device=self.dev)
            rc = so.w4a8_quantize_activations(self.xk[i].data_ptr(), self.xq[i].data_ptr(), self.sx[i].data_ptr(),
                                              self.xsum[i].data_ptr(), M, K, self.sptr)
            if rc != 0:
                raise RuntimeError(f"w4a8_quantize_activations failed ({rc}) for M={M} K={K}")
        c = self.cursor[key]
        self.cursor[key] = (c + 1) % len(self.weights[key])
        qw, s, z = self.weights[key][c]
        rc = so.w4a8_matmul(self.xq[i].data_ptr(), self.sx[i].data_ptr(), self.xsum[i].data_ptr(), qw.data_ptr(),
                            s.data_ptr(), z.data_ptr(),
                            self.y[i].data_ptr(), M, N, K, self.group, self.layout_id, self.sptr)
        if rc != 0:
            raise RuntimeError(f"w4a8_matmul failed ({rc}) for M={M} K={K} N={N}")


def events(torch, stream):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


CLOCK_WARM_S = 0.3             # sustained load before a timed region (the GPU clock ramps up)


def replay(torch, g, stream, times=1):
    """Replay graph `g` on `stream` (CUDAGraph.replay launches on the current stream: a
    replay outside this context would run on the default stream, concurrently with work
    timed on `stream`)."""
    with torch.cuda.stream(stream):
        for _ in range(times):
            g.replay()


def keep_busy(torch, stream, g, seconds):
    """Replay graph `g` on `stream` until `seconds` of wall time have passed: the GPU raises
    its clock under sustained load, and a timed region that starts cold measures the ramp."""
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        replay(torch, g, stream)
        n += 1
        if n % 8 == 0:
            stream.synchronize()
    stream.synchronize()
    return n


def time_graph(torch, stream, body, reps, warm=2, busy_s=0.05, trials=3):
    """Capture `body` once into a HIP graph on `stream`; after `warm` replays and `busy_s`
    seconds of sustained replays, time `trials` runs of `reps` replays between HIP events
    recorded on the same stream. Returns (median seconds per replay, graph)."""
    with torch.cuda.stream(stream):      # eager call first: allocates any split-K workspace
        body()
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        body()
    replay(torch, g, stream, warm)
    keep_busy(torch, stream, g, busy_s)
    ts = []
    for _ in range(trials):
        e0, e1 = events(torch, stream)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3 / reps)
    return float(np.median(ts)), g


def batch_sizes(steps, batches=5):
    """Split `steps` into up to `batches` consecutive batches of near-equal size."""
    n = max(1, min(batches, steps))
    return [steps // n + (1 if i < steps % n else 0) for i in range(n)]


def timed_steps(torch, runner, steps, warmup):
    """Warm up eagerly (allocates this stream's split-K workspace), capture the steps of each
    batch size in a graph, check replays against the eager outputs, then time exactly `steps`
    steps as up to 5 batches, each replay between HIP events on the launch stream. Returns
    (total seconds, list of seconds per step of each batch)."""
    stream = runner.stream
    with torch.cuda.stream(stream):
        for _ in range(max(1, warmup)):
            runner.step()
    stream.synchronize()
    ref = [y.clone() for y in runner.y]
    sizes = batch_sizes(steps)
    graphs = {}
    for n in sorted(set(sizes)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(n):
                runner.step()
        graphs[n] = g
    for g in graphs.values():
        replay(torch, g, stream, 1)
    stream.synchronize()
    _check_same(torch, runner, ref, "graph warm-up replay")
    keep_busy(torch, stream, graphs[sizes[0]], CLOCK_WARM_S)
    torch.cuda.synchronize()
    marks = [events(torch, stream) for _ in sizes]
    with torch.cuda.stream(stream):
        for n, (e0, e1) in zip(sizes, marks):
            e0.record(stream)
            graphs[n].replay()
            e1.record(stream)
    marks[-1][1].synchronize()
    torch.cuda.synchronize()
    _check_same(torch, runner, ref, "timed replays")
    per_step = [e0.elapsed_time(e1) / 1e3 / n for n, (e0, e1) in zip(sizes, marks)]
    total = sum(e0.elapsed_time(e1) / 1e3 for e0, e1 in marks)
    del graphs
    return total, per_step


def _check_same(torch, runner, ref, what):
    for i, (y, r) in enumerate(zip(runner.y, ref)):
        if not torch.equal(y, r):
            raise RuntimeError(f"{what} differs from the eager result for item {runner.items[i][:3]}")


def per_item_times(torch, lib, runner, reps_per_copy=1):
    """Per-shape time: a graph of one launch per rotation copy of that shape's weights."""
    out = []
    seen = set()
    for i, (M, K, N, key) in enumerate(runner.items):
        if (M, K, N, key) in seen:
            continue
        seen.add((M, K, N, key))
        reps = len(runner.weights[key]) * reps_per_copy
        sec, _ = time_graph(torch, runner.stream, lambda: [runner.launch(i) for _ in range(reps)], 5)
        t = sec / reps
        b = alg_bytes(M, K, N, runner.group)
        out.append({"M": M, "K": K, "N": N, "us": round(t * 1e6, 3),
                    "GBps": round(b / t / 1e9, 1), "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 4),
                    "TFLOPs": round(2 * M * K * N / t / 1e12, 3),
                    "plan": lib.w4a16_plan(M, N, K, group_size=runner.group)})
    return out


def copy_bandwidth(torch, dev, stream):
    """Achievable HBM rate of a plain device copy (read + write bytes / time)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    with torch.cuda.stream(stream):
        for _ in range(3):
            b.copy_(a)
        e0, e1 = events(torch, stream)
        e0.record(stream)
        for _ in range(10):
            b.copy_(a)
        e1.record(stream)
    e1.synchronize()
    return 2 * n * 10 / (e0.elapsed_time(e1) / 1e3) / 1e9


def dense_time(torch, x, ws, y, stream, reps):
    """Seconds per torch fp16 matmul (hipBLASLt/rocBLAS), rotating over the weights `ws`.

    Timed eagerly, never inside a HIP graph: a library GEMM may reset its own split-K flags
    with a memset, which does not replay correctly from a captured graph. For these sizes
    the GPU stays ahead of the host, so back-to-back eager calls measure the kernels."""
    with torch.cuda.stream(stream):
        for i in range(len(ws)):                              # warm-up (library initialisation)
            torch.matmul(x, ws[i], out=y)
        stream.synchronize()
        t0, i = time.perf_counter(), 0
        while time.perf_counter() - t0 < 0.05:                # sustained load: clock ramp-up
            torch.matmul(x, ws[i % len(ws)], out=y)
            i += 1
            if i % 16 == 0:
                stream.synchronize()
        stream.synchronize()
        e0, e1 = events(torch, stream)
        e0.record(stream)
        for i in range(reps):
            torch.matmul(x, ws[i % len(ws)], out=y)
        e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps


def dequant_time(torch, lib, runner, key, stream, reps=4):
    """Seconds per w4a16_dequant call writing the fp16 weights [K, N] (the first half of a
    dequantise-then-dense-GEMM path), rotating over the weight copies."""
    K, N = runner.weights[key][0][0].shape[0] * 8, runner.weights[key][0][0].shape[1]
    w16 = torch.empty((K, N), dtype=torch.float16, device=runner.dev)
    so = lib.load()

    def call(i):
        qw, s, z = runner.weights[key][i % len(runner.weights[key])]
        rc = so.w4a16_dequant_fmt(qw.data_ptr(), s.data_ptr(), z.data_ptr(), None, w16.data_ptr(), N, K,
                                  runner.group, runner.layout_id, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"w4a16_dequant failed ({rc})")
    with torch.cuda.stream(stream):
        for i in range(2):
            call(i)
        stream.synchronize()
        e0, e1 = events(torch, stream)
        e0.record(stream)
        for i in range(reps):
            call(i)
        e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps


def dense_weights(torch, lib, runner, key):
    """fp16 weights [K, N] equal to the GPU's dequantised values, rotated like the int4 ones."""
    qw, s, z = runner.weights[key][0]
    _, w16 = lib.w4a16_dequant(qw, s, z, codes=False, group_size=runner.group, layout=runner.layout)
    copies = max(2, -(-ROTATE_BYTES // (w16.numel() * 2)))
    return [w16] + [w16.clone() for _ in range(copies - 1)]


def cpu_baseline(runner, wid, min_s=10.0, max_passes=40):
    """The oracle as it stands (unpack + exact dequant + fp64 BLAS matmul) on whole passes over
    the step's GEMMs, repeated until at least `min_s` seconds of CPU work (a bounded sample)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = None
    xs = {(M, K): synth.activations(M, K, wid=wid) for (M, K, N, key) in runner.items}
    total_bytes, passes = 0, 0
    t0 = time.perf_counter()
    while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_s):
        for (M, K, N, key) in runner.items:
            qw, s, z = runner.host[key]
            oracle.matmul(xs[(M, K)], qw, s, z, runner.group, layout=runner.layout)
            total_bytes += alg_bytes(M, K, N, runner.group)
        passes += 1
    dt = time.perf_counter() - t0
    return {"value": round(total_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": blas_threads,
            "kind": "oracle",
            "sample": (f"{passes} passes over the {len(runner.items)} GEMMs of one step (same shapes and "
                       f"data), {dt:.1f} s; NumPy elementwise unpack/dequant on 1 thread, fp64 BLAS matmul "
                       f"on {blas_threads} threads of {len(os.sched_getaffinity(0))} available")}


def load_traffic(kernel=None):
    """Measured HBM bytes per launch from the committed PMC summary (of one decode-kernel
    instance, or the mean over the sweep's launches), if it was taken on the current kernel
    sources and plans (else None)."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha") != decode_kernel_hash():
        return None
    if kernel is not None:
        return d.get("per_kernel", {}).get(kernel, {}).get("traffic_bytes_per_launch")
    return d.get("traffic_bytes_per_launch")


# ---- workloads ----------------------------------------------------------------------------

def workload_items(name):
    """(families, items, description, replicate) of a decode-type workload."""
    if name == "decode_sweep":
        wid = synth.WORKLOADS[name]["wid"]
        fam = {(K, N): (K, N, wid, 0) for (K, N) in SWEEP_KN}
        items = [(M, K, N, (K, N)) for (K, N) in SWEEP_KN for M in SWEEP_M]
        desc = ("decode_sweep: M in {1,2,4,8,16} x (K,N) in {(4096,14336),(14336,4096),"
                "(4096,4096)}, int4 weights packed 8/int32 along K, fp16 scale+zero per 128-row group")
        return fam, items, desc, None
    if name == "gemv_4096":
        fam = {(4096, 4096): (4096, 4096, 0, 0)}
        return fam, [(1, 4096, 4096, (4096, 4096))], "gemv_4096: M=1, K=N=4096, group 128", None
    if name == "gemv_lm_head":
        _, K, N = synth.CHAIN_7B_LM_HEAD
        fam = {(K, N): (K, N, synth.WORKLOADS["decode_chain_7b"]["wid"], 100)}
        return fam, [(1, K, N, (K, N))], ("gemv_lm_head: M=1, K=4096, N=128256 (the lm_head of the 7B-shaped "
                                          "chain, 279 MB per call), group 128"), None
    if name == "moe_expert":
        wid = synth.WORKLOADS[name]["wid"]
        kns = [(2048, 1408), (1408, 2048), (2048, 768), (768, 2048)]
        fam = {(K, N): (K, N, wid, 0) for (K, N) in kns}
        items = [(M, K, N, (K, N)) for (K, N) in kns for M in (1, 4, 16)]
        return fam, items, "moe_expert: M in {1,4,16} x (2048,1408),(1408,2048),(2048,768),(768,2048)", None
    if name == "shard_8":
        wid = synth.WORKLOADS["decode_sweep"]["wid"]
        fam = {(K, N): (K, N, wid, 8) for (K, N) in SHARD8_KN}
        items = [(M, K, N, (K, N)) for (K, N) in SHARD8_KN for M in (1, 4, 16)]
        desc = ("shard_8: one GPU's share of the 7B-shaped decode projections split by output columns "
                "over 8 GPUs: (K,N) in {(4096,512) q/k/v/o, (4096,1792) gate/up, (14336,512) down, "
                "(4096,16032) lm_head}, M in {1,4,16}, group 128")
        return fam, items, desc, None
    if name == "chain_7b":
        wid = synth.WORKLOADS["decode_chain_7b"]["wid"]
        fam, items, replicate = {}, [], {}
        for layer in range(synth.CHAIN_7B_LAYERS):
            for p, (pname, K, N) in enumerate(synth.CHAIN_7B_LAYER):
                key = (layer, pname)
                # one layer's seven matrices are drawn (distinct seeds per projection);
                # the other 31 layers are device copies of them (distinct memory)
                fam[key] = (K, N, wid, p)
                if layer > 0:
                    replicate[key] = (0, pname)
                items.append((1, K, N, key))
        _, K, N = synth.CHAIN_7B_LM_HEAD
        fam[("lm_head",)] = (K, N, wid, 100)
        items.append((1, K, N, ("lm_head",)))
        desc = ("chain_7b: batch-1 decode of a 32-layer 7B-shaped model, per layer q,k,v,o "
                "4096x4096, gate,up 4096x14336, down 14336x4096, plus lm_head 4096x128256; "
                "225 GEMVs per token")
        return fam, items, desc, replicate
    raise SystemExit(f"unknown workload {name}")


def read_ceiling(torch, lib, dev, stream, sizes):
    """Seconds per plain read (w4a16_read_probe: 16-byte non-temporal loads, nothing else) of
    each byte count in `sizes`, through windows rotated over 1 GiB and timed like the decode
    calls (a graph of one read per window). The measured ceiling for a call that moves that
    many bytes."""
    so = lib.load()
    buf = torch.empty(ROTATE_BYTES + (64 << 20), dtype=torch.uint8, device=dev)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    out = {}
    for b in sorted(set(sizes)):
        n16 = -(-b // 16) * 16
        stride = -(-n16 // 4096) * 4096
        n = max(1, ROTATE_BYTES // stride)

        def body():
            for i in range(n):
                rc = so.w4a16_read_probe(buf.data_ptr() + i * stride, n16, sink.data_ptr(), stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"w4a16_read_probe failed ({rc})")
        sec, _ = time_graph(torch, stream, body, 5)
        out[b] = sec / n
    del buf
    return out


CHAIN_GROUPS = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]


class GroupedChain:
    """The chain_7b token with the projections that share an input launched together
    (w4a16_matmul_grouped): per layer q/k/v in one launch, o, gate/up in one launch, down;
    then lm_head: 129 launches instead of 225, on the same weights as `runner`."""

    def __init__(self, torch, lib, runner):
        B = lib._binding
        self.torch, self.stream, self.so = torch, runner.stream, lib.load()
        self.sptr = runner.stream.cuda_stream
        self.layout_id, self.group = runner.layout_id, runner.group
        self.calls, self.y, self.items = [], [], []     # one y and one item per matrix
        self.step_bytes = runner.step_bytes
        x = runner.x[(1, 4096, synth.WORKLOADS["decode_chain_7b"]["wid"])]
        for layer in range(synth.CHAIN_7B_LAYERS):
            for names in CHAIN_GROUPS:
                keys = [(layer, nm) for nm in names]
                arr = (B.w4a16_matrix_t * len(keys))()
                K = None
                for i, key in enumerate(keys):
                    qw, s, z = runner.weights[key][0]
                    K, N = qw.shape[0] * 8, qw.shape[1]
                    y = torch.empty((1, N), dtype=torch.float16, device=runner.dev)
                    self.y.append(y)
                    self.items.append((1, K, N, key))
                    arr[i] = B.w4a16_matrix_t(qw.data_ptr(), s.data_ptr(), z.data_ptr(), y.data_ptr(), N)
                xk = x if K == 4096 else runner.x[(1, K, synth.WORKLOADS["decode_chain_7b"]["wid"])]
                self.calls.append((xk, arr, len(keys), K))
        lm = [i for i, it in enumerate(runner.items) if it[3] == ("lm_head",)][0]
        self.lm = (runner, lm)
        self.y.append(runner.y[lm])
        self.items.append(runner.items[lm])

    def step(self):
        for xk, arr, n, K in self.calls:
            rc = self.so.w4a16_matmul_grouped(xk.data_ptr(), arr, n, 1, K, self.group, self.layout_id, self.sptr, None)
            if rc != 0:
                raise RuntimeError(f"w4a16_matmul_grouped failed ({rc})")
        self.lm[0].launch(self.lm[1])


def grouped_timing(torch, lib, dev, stream, label, mats, own_x, ms, wid, group=GROUP, layout="linear", rows=None):
    """One grouped launch (w4a16_matmul_grouped) over the matrices `mats` = [(K, N, seed), ...]
    (same K) against one launch per matrix, at each M in `ms`, weights rotated over 1 GiB.
    own_x: every matrix reads its own activations (x_i) instead of one shared x. rows: each
    matrix's own row count M_i (then ms is (max rows,), and x_i has M_i rows)."""
    B = lib._binding
    so = lib.load()
    lay = B._layout_id(layout)
    K = mats[0][0]
    Ns = [N for _, N, _ in mats]
    one = []
    for K_, N, seed in mats:
        qw, s, z = lib.w4a16_pack(synth.weight(K_, N, wid=wid, layer=seed), group_size=group, layout=layout)
        one.append([torch.from_numpy(a).to(dev) for a in (qw, s, z)])
    per = sum(t.numel() * t.element_size() for m in one for t in m)
    ring = [one] + [[[t.clone() for t in m] for m in one] for _ in range(max(1, -(-ROTATE_BYTES // per)) - 1)]
    out = []
    for M in ms:
        Ms = rows or [M] * len(mats)
        x = torch.from_numpy(synth.activations(M, K, wid=wid)).to(dev)
        xs = [torch.from_numpy(synth.activations(Ms[i], K, wid=wid + 1 + i)).to(dev) if own_x else x
              for i in range(len(mats))]
        ys = [torch.empty((m, N), dtype=torch.float16, device=dev) for m, N in zip(Ms, Ns)]
        arrs = []
        for ms_ in ring:
            arr = (B.w4a16_matrix_t * len(mats))()
            for i, ((q, s_, z_), y) in enumerate(zip(ms_, ys)):
                arr[i] = B.w4a16_matrix_t(q.data_ptr(), s_.data_ptr(), z_.data_ptr(), y.data_ptr(), Ns[i],
                                          xs[i].data_ptr() if own_x else None, Ms[i])
            arrs.append(arr)

        def grouped():
            for arr in arrs:
                if so.w4a16_matmul_grouped(x.data_ptr(), arr, len(mats), M, K, group, lay, stream.cuda_stream, None):
                    raise RuntimeError("w4a16_matmul_grouped failed")

        def separate():
            for ms_ in ring:
                for (q, s_, z_), y, xi, m in zip(ms_, ys, xs, Ms):
                    if so.w4a16_matmul_fmt(xi.data_ptr(), q.data_ptr(), s_.data_ptr(), z_.data_ptr(), y.data_ptr(),
                                           m, q.shape[1], K, group, lay, stream.cuda_stream, None):
                        raise RuntimeError("w4a16_matmul_fmt failed")
        tg = time_graph(torch, stream, grouped, 5)[0] / len(ring)
        ts = time_graph(torch, stream, separate, 5)[0] / len(ring)
        b = sum(alg_bytes(m, K, N, group) for m, N in zip(Ms, Ns))
        out.append({"matrices": label, "M": M if rows is None else Ms, "K": K, "N": Ns, "own_x": own_x, "bytes": b,
                    "grouped_us": round(tg * 1e6, 3), "grouped_GBps": round(b / tg / 1e9, 1),
                    "grouped_frac_hbm": round(b / tg / 1e9 / HBM_PEAK_GBS, 4),
                    "separate_launches_us": round(ts * 1e6, 3), "speedup": round(ts / tg, 3),
                    "plan": lib.w4a16_plan(M, sum(Ns), K, group_size=group)})
    del ring
    return out


def grouped_decode(torch, lib, dev, stream, group=GROUP, layout="linear", ms=(1, 16)):
    """The projections of the 7B-shaped layer that share an input, at M = 1 and 16: q/k/v
    (3 x 4096 x 4096) and gate/up (2 x 4096 x 14336), as one grouped launch against one
    launch per matrix."""
    wid = synth.WORKLOADS["decode_chain_7b"]["wid"]
    names = [nm for nm, _, _ in synth.CHAIN_7B_LAYER]
    shapes = dict((nm, (K, N)) for nm, K, N in synth.CHAIN_7B_LAYER)
    out = []
    for group_names in (("q", "k", "v"), ("gate", "up")):
        mats = [shapes[nm] + (names.index(nm),) for nm in group_names]
        out += grouped_timing(torch, lib, dev, stream, "+".join(group_names), mats, False, ms, wid, group, layout)
    return out


def grouped_experts(torch, lib, dev, stream, group=GROUP, layout="linear"):
    """Batch-1 decode of mixture-of-experts layers built from the expert shapes: the gate and
    up projections of the active experts read the token (one shared x), and each expert's
    down projection reads its own input. E active experts of hidden 2048 and expert width F:
    2E matrices 2048 x F with one x, then E matrices F x 2048 with their own x, each set as
    one grouped launch against one launch per matrix."""
    wid = synth.WORKLOADS["moe_expert"]["wid"]
    out = []
    for E, F in ((4, 1408), (8, 768)):
        up = [(2048, F, 100 + e) for e in range(2 * E)]
        down = [(F, 2048, 200 + e) for e in range(E)]
        out += grouped_timing(torch, lib, dev, stream, f"{E} experts gate+up ({2 * E} x 2048x{F})", up, False, (1,),
                              wid, group, layout)
        out += grouped_timing(torch, lib, dev, stream, f"{E} experts down ({E} x {F}x2048, own x)", down, True, (1,),
                              wid, group, layout)
    # a batch of 16 tokens, each routed to 2 of 8 experts (seeded): the down projections of
    # the experts, each over its own tokens (M_e rows), in one launch
    rng = np.random.default_rng((7, 16, 8))
    picks = np.array([rng.choice(8, size=2, replace=False) for _ in range(16)])
    counts = [int(c) for c in np.bincount(picks.ravel(), minlength=8)]
    active = [e for e in range(8) if counts[e] > 0]
    down = [(1408, 2048, 300 + e) for e in active]
    out += grouped_timing(torch, lib, dev, stream, f"16 tokens top-2 of 8 experts, down ({len(active)} x 1408x2048, "
                          f"tokens per expert {[counts[e] for e in active]})", down, True,
                          (max(counts),), wid, group, layout, rows=[counts[e] for e in active])
    return out


def load_kernel_trace():
    """Per-kernel durations from the committed kernel-trace summary of the decode sweep, if it
    was taken on the current decode kernel sources and plans (else None)."""
    try:
        d = json.load(open(KTRACE_FILE))
    except (OSError, ValueError):
        return None
    return d if d.get("kernel_source_sha") == decode_kernel_hash() else None


def run_decode(args):
    import torch
    import weight_only_bit_gemv_amd as lib

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)
    fam, items, desc, replicate = workload_items(args.workload)
    chain = args.workload == "chain_7b"
    rotate = 0 if chain else ROTATE_BYTES
    runner = Runner(torch, lib, dev, stream, fam, items, rotate, replicate, args.group_size,
                    args.symmetric, args.layout)
    if args.group_size != GROUP or args.symmetric or args.layout != "linear":
        desc = (desc.replace("per 128-row group", "").rstrip(", ") +
                f"; weight format: {'symmetric (zero 8)' if args.symmetric else 'asymmetric'}, "
                f"group {args.group_size}, {args.layout} layout")
    launches = len(items)
    steps = args.steps if not chain else max(1, args.steps // 10)
    elapsed, per_step = timed_steps(torch, runner, steps, args.warmup)
    t_med, t_min = float(np.median(per_step)), float(np.min(per_step))
    value = runner.step_bytes / t_med / 1e9
    avg_launch_s = t_med / launches
    if args.trace_pass:
        log(f"[trace] {steps} timed steps done")
        return

    with torch.cuda.stream(stream):                 # eager rate, for reference
        e0, e1 = events(torch, stream)
        e0.record(stream)
        for _ in range(steps):
            runner.step()
        e1.record(stream)
    e1.synchronize()
    eager_elapsed = e0.elapsed_time(e1) / 1e3

    per = per_item_times(torch, lib, runner) if not chain else []
    if not args.no_dense and not chain:
        dw = {}
        for r in per:
            key = next(k for (M, K, N, k) in items if (K, N) == (r["K"], r["N"]))
            if key not in dw:
                dw[key] = dense_weights(torch, lib, runner, key)
            x = runner.x[(r["M"], r["K"], fam[key][2])]
            y = torch.empty((r["M"], r["N"]), dtype=torch.float16, device=dev)
            d = dense_time(torch, x, dw[key], y, stream, 4 * len(dw[key]))
            r["dense_fp16_us"] = round(d * 1e6, 3)
            r["speedup_vs_dense_fp16"] = round(d / (r["us"] / 1e6), 3)
        del dw
    copy_gbs = copy_bandwidth(torch, dev, stream)
    ceil_s = {}
    if not chain:
        ceil_s = read_ceiling(torch, lib, dev, stream, [alg_bytes(M, K, N, args.group_size) for (M, K, N, _) in items])
        for r in per:
            b = alg_bytes(r["M"], r["K"], r["N"], args.group_size)
            r["read_ceiling_us"] = round(ceil_s[b] * 1e6, 3)
            r["frac_of_read_ceiling"] = round(ceil_s[b] / (r["us"] / 1e6), 4)
    achieved = runner.step_bytes / launches / avg_launch_s / 1e9
    measured_plans = args.workload == "decode_sweep" and args.group_size == GROUP and not args.symmetric \
        and args.layout == "linear"
    # the dominant kernel: the decode-kernel instance with the most time per step, from the
    # per-shape graph-timed calls (HIP events on the launch stream; every shape appears once
    # per step)
    inst = {}
    for r in per:
        if r["plan"]["kernel"] != lib.W4A16_KERNEL_SKINNY:
            continue
        name = kernel_instance(r["plan"], args.group_size, args.layout == "interleaved")
        g = inst.setdefault(name, {"calls": 0, "us": 0.0, "bytes": 0})
        g["calls"] += 1
        g["us"] += r["us"]
        g["bytes"] += alg_bytes(r["M"], r["K"], r["N"], args.group_size)
    if inst:
        dom_name, dom = max(inst.items(), key=lambda kv: kv[1]["us"])
        dom_gbs = dom["bytes"] / (dom["us"] * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(dom_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                "traffic": load_traffic(dom_name) if measured_plans else None,
                "kernel": dom_name,
                "achieved_is": (f"the dominant kernel ({dom['calls']} of {launches} calls per step, "
                                f"{round(dom['us'] / sum(g['us'] for g in inst.values()), 3)} of the calls' time): "
                                "algorithmic bytes per launch / its average launch time, each call graph-timed "
                                "with HIP events on the launch stream (the gap between graph nodes included)"),
                "avg_launch_us": round(dom["us"] / dom["calls"], 3),
                "alg_bytes_per_launch": round(dom["bytes"] / dom["calls"]),
                "step": {"achieved": round(achieved, 2), "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "avg_launch_us": round(avg_launch_s * 1e6, 3),
                         "traffic": load_traffic() if measured_plans else None,
                         "is": "algorithmic bytes per launch / (median step time / launches), all kernels"}}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "skinny_kernel (decode weight stream, MFMA, split-K when K is deep)",
                "achieved_is": ("algorithmic bytes per launch / (median step time / launches): whole-step rate, "
                                "the gap between graph nodes included"),
                "avg_launch_us": round(avg_launch_s * 1e6, 3)}
    if ceil_s:
        read_step = sum(ceil_s[alg_bytes(M, K, N, args.group_size)] for (M, K, N, _) in items)
        step = roof.get("step", roof)
        step["read_ceiling_GBps"] = round(runner.step_bytes / read_step / 1e9, 1)
        step["frac_of_read_ceiling"] = round(read_step / t_med, 4)
        if inst:   # the dominant kernel's calls against plain reads of the same byte counts
            rows = [r for r in per if r["plan"]["kernel"] == lib.W4A16_KERNEL_SKINNY and
                    kernel_instance(r["plan"], args.group_size, args.layout == "interleaved") == roof["kernel"]]
            roof["frac_of_read_ceiling"] = round(sum(r["read_ceiling_us"] for r in rows) /
                                                 sum(r["us"] for r in rows), 4)
    kt = load_kernel_trace() if (args.workload == "decode_sweep" and args.group_size == GROUP and
                                 not args.symmetric and args.layout == "linear") else None
    if kt:
        dom = kt["dominant"]
        roof["dominant_kernel"] = {
            "name": dom["name"], "avg_ns": dom["avg_ns"], "alg_bytes_per_launch": dom["alg_bytes_per_launch"],
            "GBps": dom["GBps"], "frac": dom["frac_hbm"], "share_of_kernel_time": dom["share"],
            "source": os.path.relpath(KTRACE_FILE, ROOT),
            "is": ("kernel-trace durations (rocprofv3) of the same sources and plans, no graph gap; the "
                   "profiler lengthens kernels a little, so this is a lower bound of the unprofiled rate")}
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(t_med * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": desc, "group_size": args.group_size, "symmetric": args.symmetric,
                   "layout": args.layout,
                   "launches_per_step": launches, "bytes_per_step": runner.step_bytes,
                   "timing": (f"{len(per_step)} batches of HIP-graph replays ({'+'.join(map(str, batch_sizes(steps)))} "
                              f"steps), events on the launch stream; value and ms_per_step from the median batch"),
                   "weight_copies_rotated": {str(k): len(v) for k, v in runner.weights.items() if not chain}},
        "roofline": roof,
        "step_ms_median": round(t_med * 1e3, 4), "step_ms_min": round(t_min * 1e3, 4),
        "value_at_min": round(runner.step_bytes / t_min / 1e9, 2),
        "timed_total_ms": round(elapsed * 1e3, 4),
        "measured_copy_GBps": round(copy_gbs, 1),
        "frac_of_measured_copy": round(value / copy_gbs, 4),
        "eager_ms_per_step": round(eager_elapsed / steps * 1e3, 4),
        "per_shape": per,
    }
    if args.workload == "decode_sweep" and not args.no_grouped:
        result["grouped"] = grouped_decode(torch, lib, dev, stream, args.group_size, args.layout)
    if args.workload == "moe_expert" and not args.no_grouped:
        result["grouped"] = grouped_experts(torch, lib, dev, stream, args.group_size, args.layout)
    if chain:
        result["tokens_per_s"] = round(1.0 / t_med, 2)
        result["us_per_token"] = round(t_med * 1e6, 2)
        result["ceiling_tokens_per_s_at_8TBps"] = round(HBM_PEAK_GBS * 1e9 / runner.step_bytes, 1)
        result["ceiling_tokens_per_s_at_measured_copy"] = round(copy_gbs * 1e9 / runner.step_bytes, 1)
        gc = GroupedChain(torch, lib, runner)
        g_elapsed, g_per = timed_steps(torch, gc, steps, args.warmup)
        g_med = float(np.median(g_per))
        result["grouped_chain"] = {"launches_per_token": len(gc.calls) + 1, "us_per_token": round(g_med * 1e6, 2),
                                   "tokens_per_s": round(1.0 / g_med, 2),
                                   "GBps": round(runner.step_bytes / g_med / 1e9, 1),
                                   "frac_hbm": round(runner.step_bytes / g_med / 1e9 / HBM_PEAK_GBS, 4),
                                   "groups": "per layer q+k+v, o, gate+up, down; then lm_head"}
    if not args.no_cpu and args.workload == "decode_sweep":
        result["cpu_baseline"] = cpu_baseline(runner, synth.WORKLOADS["decode_sweep"]["wid"])
    emit(result, args)


def emit(result, args):
    """Print the JSON line; with --record, also write it with the command, the sources' hash
    and the machine to a file."""
    print(json.dumps(result), flush=True)
    if args.record:
        import platform
        import torch
        rec = {"command": "python " + " ".join(sys.argv), "sources_sha": all_sources_hash(),
               "host": platform.node(), "gpu": torch.cuda.get_device_name(0),
               "date_utc": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime()), "result": result}
        os.makedirs(os.path.dirname(os.path.abspath(args.record)), exist_ok=True)
        with open(args.record, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")


def all_sources_hash():
    """Hash of every source that decides a measured number: the kernels, the dispatcher, the
    binding, synth.py and bench.py."""
    files = sorted(glob.glob(os.path.join(ROOT, "weight_only_bit_gemv_amd", "csrc", "*")) +
                   [os.path.join(ROOT, "weight_only_bit_gemv_amd", "_binding.py"), os.path.join(ROOT, "synth.py"),
                    os.path.abspath(__file__), os.path.join(ROOT, "include", "w4a16.h")])
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def run_prefill(args):
    """M-crossover of the W4A16 path (dispatcher's choice) against torch fp16 matmul."""
    import torch
    import weight_only_bit_gemv_amd as lib
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    wid = synth.WORKLOADS["prefill"]["wid"]
    kns = [(8192, 8192), (8192, 28672), (28672, 8192)] + SWEEP_KN
    ms = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048]
    rows, best_gbs = [], None
    for (K, N) in kns:
        fam = {(K, N): (K, N, wid, 0)}
        items = [(M, K, N, (K, N)) for M in ms]
        runner = Runner(torch, lib, dev, stream, fam, items, ROTATE_BYTES // 2, None, args.group_size,
                        args.symmetric, args.layout)
        with torch.cuda.stream(stream):
            runner.step()
        stream.synchronize()
        ws = dense_weights(torch, lib, runner, (K, N))
        dq = dequant_time(torch, lib, runner, (K, N), stream)
        cross = None
        for i, M in enumerate(ms):
            log(f"[prefill] K={K} N={N} M={M}")
            reps = len(runner.weights[(K, N)])
            sec, _ = time_graph(torch, stream, lambda: [runner.launch(i) for _ in range(reps)], 2, warm=1)
            t = sec / reps
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            d = dense_time(torch, runner.xk[i], ws, y, stream, 2 * len(ws))
            fl = 2 * M * K * N
            row = {"M": M, "K": K, "N": N, "w4a16_us": round(t * 1e6, 2),
                   "w4a16_TFLOPs": round(fl / t / 1e12, 2), "w4a16_GBps": round(alg_bytes(M, K, N, args.group_size) / t / 1e9, 1),
                   "dense_fp16_us": round(d * 1e6, 2), "dense_TFLOPs": round(fl / d / 1e12, 2),
                   "speedup_vs_dense": round(d / t, 3),
                   # dequantise to fp16 with the library's kernel, then the dense GEMM
                   "dequant_then_dense_us": round((dq + d) * 1e6, 2),
                   "plan": lib.w4a16_plan(M, N, K, group_size=args.group_size)}
            forced = []
            if 32 <= M <= 512:           # both kernels, where the dispatcher's threshold lies
                forced.append(("skinny_us", dict(kernel=lib.W4A16_KERNEL_SKINNY)))
            if M >= 32:                  # both prefill tiles
                forced += [("prefill_lds_tile_us", dict(kernel=lib.W4A16_KERNEL_PREFILL, tile=lib.W4A16_TILE_LDS)),
                           ("prefill_register_tile_us",
                            dict(kernel=lib.W4A16_KERNEL_PREFILL, tile=lib.W4A16_TILE_REGISTER_B)),
                           ("prefill_async_tile_us",
                            dict(kernel=lib.W4A16_KERNEL_PREFILL, tile=lib.W4A16_TILE_ASYNC, splits=1)),
                           ("prefill_async_split_us",
                            dict(kernel=lib.W4A16_KERNEL_PREFILL, tile=lib.W4A16_TILE_ASYNC))]
            for name, plan in forced:
                sec, _ = time_graph(torch, stream, lambda: [runner.launch(i, plan) for _ in range(reps)],
                                    2, warm=1)
                row[name] = round(sec / reps * 1e6, 2)
            if M >= 32 and N % 8 == 0 and args.group_size in (128, 256):
                # W4A8 (E4M3 activations): the 8-bit product alone, and with the per-row
                # activation quantiser in front of it
                with torch.cuda.stream(stream):
                    runner.launch_w4a8(i)
                stream.synchronize()
                sec, _ = time_graph(torch, stream, lambda: [runner.launch_w4a8(i) for _ in range(reps)], 2, warm=1)
                row["w4a8_us"] = round(sec / reps * 1e6, 2)
                row["w4a8_TFLOPs"] = round(fl / (sec / reps) / 1e12, 2)
                sec, _ = time_graph(torch, stream, lambda: [runner.launch_w4a8(i, quantize=True) for _ in range(reps)],
                                    2, warm=1)
                row["w4a8_with_quantize_us"] = round(sec / reps * 1e6, 2)
            rows.append(row)
            if cross is None and d < t:
                cross = M
        rows.append({"K": K, "N": N, "crossover_M_dense_faster_from": cross})
        del ws, runner
        torch.cuda.empty_cache()
    big = [r for r in rows if "w4a16_TFLOPs" in r and r["M"] >= 512]
    best = max(big, key=lambda r: r["w4a16_TFLOPs"])
    result = {"metric": "W4A16 prefill TFLOP/s and M-crossover against dense fp16",
              "value": best["w4a16_TFLOPs"], "unit": "TFLOP/s", "n_gpus": 1, "steps": 1,
              "warmup": 1, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "f16", "data": "synthetic",
              "config": {"workload": "prefill crossover: M in 1..2048 on (8192,8192),(8192,28672),"
                                     "(28672,8192) and the decode-sweep shapes",
                         "group_size": args.group_size, "symmetric": args.symmetric, "layout": args.layout},
              "roofline": {"bound": "mfma", "achieved": best["w4a16_TFLOPs"],
                           "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(best["w4a16_TFLOPs"] / MFMA_F16_PEAK_TFLOPS, 4),
                           "traffic": None, "kernel": PREFILL_KERNEL_NAMES.get(best["plan"]["tile"], "prefill"),
                           "shape": [best["M"], best["K"], best["N"]]},
              "rows": rows}
    emit(result, args)


PREFILL_PMC_SHAPE = (2048, 8192, 28672)      # M, K, N of the prefill counter pass
PREFILL_KERNEL_NAMES = {1: "prefill_kernel (128x128 LDS tile)", 2: "prefill_rb_kernel (128x256 register tile)",
                        3: "prefill_async_kernel (128x256, direct-to-LDS ring)"}
PREFILL_PMC_FILE = os.path.join(ROOT, "profiles", "prefill_counters_M2048_K8192_N28672.json")
W4A8_PMC_FILE = os.path.join(ROOT, "profiles", "w4a8_counters_M2048_K8192_N28672.json")
W4A8_SOURCES = [os.path.join("weight_only_bit_gemv_amd", "csrc", n) for n in ("w4a8_prefill.hip", "w4a16_device.hpp")]
SIMDS = 1024                                  # 256 compute units x 4 SIMDs
SCLK_GHZ = 2.4


def run_prefill_pmc_pass(args):
    """Eager launches of the prefill kernel on one large shape, for rocprofv3 --pmc."""
    import torch
    import weight_only_bit_gemv_amd as lib
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    M, K, N = PREFILL_PMC_SHAPE
    wid = synth.WORKLOADS["prefill"]["wid"]
    runner = Runner(torch, lib, dev, stream, {(K, N): (K, N, wid, 0)}, [(M, K, N, (K, N))], 0)
    with torch.cuda.stream(stream):
        if args.w4a8:
            runner.launch_w4a8(0)                   # quantise once, outside the counted launches
        for _ in range(args.steps):
            if args.w4a8:
                runner.launch_w4a8(0)
            else:
                runner.launch(0, dict(kernel=lib.W4A16_KERNEL_PREFILL))
    stream.synchronize()
    log(f"[pmc] {args.steps} {'W4A8' if args.w4a8 else 'prefill'} launches done")


def summarize_prefill_pmc(dirs, w4a8=False):
    """MFMA and LDS counters of the prefill kernel, or of the W4A8 product kernel (runs with
    --kernel-trace and --pmc)."""
    import csv
    tag = "w4a8_kernel" if w4a8 else "prefill"
    vals, durs, names = {}, [], set()
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(path)):
                if tag in row["Kernel_Name"]:
                    vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
                    names.add(row["Kernel_Name"])
        for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
            for row in csv.DictReader(open(path)):
                if tag in row["Kernel_Name"]:
                    durs.append(int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
    mean = {k: float(np.mean(v)) for k, v in vals.items()}
    M, K, N = PREFILL_PMC_SHAPE
    dur_ns = float(np.median(durs)) if durs else None
    out = {"kernel_source_sha": kernel_source_hash(W4A8_SOURCES if w4a8 else PREFILL_SOURCES), "shape_MKN": [M, K, N],
           "kernels": sorted(names), "counters_mean_per_dispatch": mean, "kernel_ns_median": dur_ns,
           "TFLOPs": round(2 * M * K * N / dur_ns / 1e3, 1) if dur_ns else None}
    if dur_ns and "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
        # busy cycles summed over SIMDs against every SIMD busy for the whole kernel at the
        # nominal clock
        out["mfma_busy_fraction"] = round(mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (dur_ns * SCLK_GHZ * SIMDS), 4)
    if "SQ_LDS_BANK_CONFLICT" in mean and "SQ_LDS_IDX_ACTIVE" in mean:
        out["lds_bank_conflict_over_active"] = round(mean["SQ_LDS_BANK_CONFLICT"] / mean["SQ_LDS_IDX_ACTIVE"], 4)
    with open(W4A8_PMC_FILE if w4a8 else PREFILL_PMC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def run_pmc_pass(args):
    """Eager launches for rocprofv3 --pmc: a calibration copy of known size, then sweeps."""
    import torch
    import weight_only_bit_gemv_amd as lib
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    a = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    with torch.cuda.stream(stream):
        for _ in range(3):
            b.copy_(a)
    stream.synchronize()
    log("[pmc] calibration copies done")
    fam, items, _, replicate = workload_items("decode_sweep")
    runner = Runner(torch, lib, dev, stream, fam, items, ROTATE_BYTES, replicate)
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            runner.step()
    stream.synchronize()
    log(f"[pmc] {args.steps} sweep steps done")


def summarize_pmc(dirs):
    """Combine FETCH_SIZE and WRITE_SIZE counter CSVs into profiles/traffic_*.json."""
    import csv
    vals = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(path)):
                name = row.get("Counter_Name") or row.get("Counter-Name")
                kname = row.get("Kernel_Name") or row.get("Kernel-Name") or ""
                v = float(row.get("Counter_Value") or row.get("Counter-Value"))
                disp = row.get("Dispatch_Id") or row.get("Dispatch-Id")
                vals.setdefault(name, []).append((int(disp), kname, v))
    out = {}
    for name in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = sorted(vals.get(name, []))
        copy = [v for _, k, v in rows if "skinny" not in k and "w4a16" not in k]
        kern = [v for _, k, v in rows if "skinny_kernel" in k]
        if not copy or not kern:
            raise SystemExit(f"no {name} rows for both the copy and the kernel")
        # counters are KiB per dispatch; the copy reads and writes COPY_CAL_BYTES each
        cal = COPY_CAL_BYTES / (np.median(copy[:3]) * 1024)
        out[name] = {"kernel_kib_mean": float(np.mean(kern)), "copy_kib_median": float(np.median(copy[:3])),
                     "scale": cal, "kernel_bytes_mean": float(np.mean(kern)) * 1024 * cal,
                     "dispatches": len(kern)}
    launches = len(SWEEP_M) * len(SWEEP_KN)
    alg = sum(alg_bytes(M, K, N) for (K, N) in SWEEP_KN for M in SWEEP_M) / launches
    traffic = out["FETCH_SIZE"]["kernel_bytes_mean"] + out["WRITE_SIZE"]["kernel_bytes_mean"]
    # per decode-kernel instance: the mean per dispatch over its own calls (every sweep call
    # is launched equally often), against the mean algorithmic bytes of those calls
    import weight_only_bit_gemv_amd as lib
    per_kernel = {}
    for (K, N) in SWEEP_KN:
        for M in SWEEP_M:
            inst = kernel_instance(lib.w4a16_plan(M, N, K))
            per_kernel.setdefault(inst, {"alg": []})["alg"].append(alg_bytes(M, K, N))
    for inst, d in per_kernel.items():
        t = 0.0
        for name in ("FETCH_SIZE", "WRITE_SIZE"):
            ks = [v for _, k, v in vals[name] if inst in k]
            t += float(np.mean(ks)) * 1024 * out[name]["scale"]
        a = float(np.mean(d.pop("alg")))
        d.update({"traffic_bytes_per_launch": round(t), "algorithmic_bytes_per_launch": round(a),
                  "traffic_over_algorithmic": round(t / a, 4)})
    summary = {"kernel_source_sha": decode_kernel_hash(),
               "workload": "decode_sweep (15 shapes), mean over dispatches",
               "traffic_bytes_per_launch": round(traffic),
               "algorithmic_bytes_per_launch": round(alg),
               "traffic_over_algorithmic": round(traffic / alg, 4),
               "per_kernel": per_kernel,
               "counters": out}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(summary, f, indent=1)
        f.write("\n")
    print(json.dumps(summary, indent=1))


def kernel_instance(plan, group=GROUP, nat=False):
    """Name of the decode-kernel instance a skinny plan launches (its template arguments)."""
    sg = min(plan["seg"], group // 32)
    return (f"skinny_kernel<{plan['row_tiles']}, {plan['cols'] // 16}, {plan['seg']}, {sg}, {plan['waves']}, "
            f"{'true' if nat else 'false'}, 1>")


def summarize_kernel_trace(dirs):
    """Per-call and per-instance kernel durations of a `--trace-pass` run under rocprofv3
    --kernel-trace: the decode sweep's skinny dispatches in launch order, dispatch j being
    call j mod 15 of the step. Writes profiles/kernel_trace_skinny_decode_sweep.{json,md}."""
    import csv
    import weight_only_bit_gemv_amd as lib
    rows = []
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                if "skinny_kernel" in r["Kernel_Name"]:
                    rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                                 r["Kernel_Name"]))
    rows.sort()
    stats = []
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                if "skinny_kernel" in r["Name"]:
                    stats.append({"name": r["Name"], "calls": int(r["Calls"]), "avg_ns": round(float(r["AverageNs"]), 1),
                                  "min_ns": int(float(r["MinNs"])), "max_ns": int(float(r["MaxNs"])),
                                  "share": float(r["Percentage"])})
    items = workload_items("decode_sweep")[1]
    L = len(items)
    if not rows or len(rows) % L:
        raise SystemExit(f"{len(rows)} skinny dispatches: not whole steps of {L}")
    rows = rows[2 * L:]                                   # drop the first two (eager) steps
    per_item = []
    for i, (M, K, N, _) in enumerate(items):
        durs = [r[1] for j, r in enumerate(rows) if j % L == i]
        pl = lib.w4a16_plan(M, N, K)
        b = alg_bytes(M, K, N)
        avg = float(np.mean(durs))
        per_item.append({"M": M, "K": K, "N": N, "kernel": kernel_instance(pl), "dispatches": len(durs),
                         "avg_ns": round(avg, 1), "median_ns": float(np.median(durs)), "alg_bytes": b,
                         "GBps": round(b / avg, 1), "frac_hbm": round(b / avg / HBM_PEAK_GBS, 4),
                         "trace_name_sample": [r[2] for j, r in enumerate(rows) if j % L == i][0][:120]})
    kern = {}
    for it in per_item:
        k = kern.setdefault(it["kernel"], {"calls_per_step": 0, "ns": 0.0, "bytes": 0})
        k["calls_per_step"] += 1
        k["ns"] += it["avg_ns"]
        k["bytes"] += it["alg_bytes"]
    total_ns = sum(k["ns"] for k in kern.values())
    per_kernel = []
    for name, k in kern.items():
        avg = k["ns"] / k["calls_per_step"]
        bpl = k["bytes"] / k["calls_per_step"]
        per_kernel.append({"name": name, "calls_per_step": k["calls_per_step"], "avg_ns": round(avg, 1),
                           "alg_bytes_per_launch": round(bpl), "GBps": round(bpl / avg, 1),
                           "frac_hbm": round(bpl / avg / HBM_PEAK_GBS, 4), "share": round(k["ns"] / total_ns, 4)})
    per_kernel.sort(key=lambda k: -k["share"])
    step_bytes = sum(it["alg_bytes"] for it in per_item)
    out = {"kernel_source_sha": decode_kernel_hash(),
           "command": "rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- "
                      "python -u bench.py --trace-pass --steps 20; python bench.py --summarize-kernel-trace <dir>",
           "dispatches_used": len(rows), "per_call": per_item, "per_kernel": per_kernel, "dominant": per_kernel[0],
           "rocprof_kernel_stats": stats,
           "kernel_only_step_us": round(total_ns / 1e3, 3),
           "kernel_only_step_GBps": round(step_bytes / total_ns, 1)}
    base = os.path.splitext(KTRACE_FILE)[0]
    with open(KTRACE_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    lines = ["# skinny_kernel on the decode sweep: kernel-trace durations per call", "",
             "Command (repository root, MI355X):", "", "```", out["command"], "```", "",
             f"Sources: decode kernel + plans sha `{out['kernel_source_sha']}`; {len(rows)} dispatches after the two "
             "eager warm-up steps (graph replays of the timed steps; no per-shape loops). Durations exclude "
             "the gap between graph nodes.", "",
             "| M | K | N | kernel | avg ns | GB/s | of 8 TB/s |", "|---|---|---|---|---|---|---|"]
    for it in per_item:
        lines.append(f"| {it['M']} | {it['K']} | {it['N']} | `{it['kernel']}` | {it['avg_ns']:.0f} | "
                     f"{it['GBps']:.0f} | {it['frac_hbm']:.3f} |")
    lines += ["", "| kernel | calls per step | avg ns | bytes per launch | GB/s | of 8 TB/s | share of kernel time |",
              "|---|---|---|---|---|---|---|"]
    for k in per_kernel:
        lines.append(f"| `{k['name']}` | {k['calls_per_step']} | {k['avg_ns']:.0f} | {k['alg_bytes_per_launch']} | "
                     f"{k['GBps']:.0f} | {k['frac_hbm']:.3f} | {k['share']:.3f} |")
    lines += ["", f"Kernel time per step {out['kernel_only_step_us']} us: {out['kernel_only_step_GBps']} GB/s of "
              "algorithmic bytes with the gaps between launches removed.", "",
              "`run_kernel_stats.csv` of the same run (all dispatches, warm-up steps included):", "",
              "| kernel | calls | average ns | min ns | max ns | share % |", "|---|---|---|---|---|---|"]
    for k in stats:
        lines.append(f"| `{k['name']}` | {k['calls']} | {k['avg_ns']:.0f} | {k['min_ns']} | {k['max_ns']} | "
                     f"{k['share']:.2f} |")
    with open(base + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(out, indent=1))


RECORD_KEEP_ROW = ("M", "K", "N", "w4a16_us", "w4a16_TFLOPs", "dense_fp16_us", "speedup_vs_dense",
                   "dequant_then_dense_us", "w4a8_us", "w4a8_TFLOPs", "w4a8_with_quantize_us",
                   "crossover_M_dense_faster_from")


def summarize_records(paths):
    """Trimmed copies of --record files in profiles/ (bench_<workload>.json) and one table of
    the figures they hold (profiles/bench_records.md)."""
    recs = []
    for path in paths:
        rec = json.load(open(path))
        res = rec["result"]
        wl = res["config"]["workload"].split(":")[0].split()[0]
        if "rows" in res:                                   # prefill crossover
            wl = "prefill"
            rows = []
            for r in res["rows"]:
                t = {k: r[k] for k in RECORD_KEEP_ROW if k in r}
                if "plan" in r:
                    t["plan"] = f"k{r['plan']['kernel']}t{r['plan']['tile']}s{r['plan']['splits']}"
                rows.append(t)
            res = dict(res, rows=rows)
        out = dict(rec, result=res)
        with open(os.path.join(ROOT, "profiles", f"bench_{wl}.json"), "w") as f:
            json.dump(out, f, separators=(",", ":"))
            f.write("\n")
        recs.append((wl, rec, res))
    lines = ["# bench.py records (one MI355X)", "",
             "Each `bench_<workload>.json` here is the record `python bench.py --workload <w> --record FILE` wrote on "
             "the GPU box (command, hash of every measured source, host, date), trimmed by "
             "`python bench.py --summarize-records FILE...`.", ""]
    for wl, rec, res in recs:
        lines += [f"## {wl}", "", f"`{rec['command']}`; sources `{rec['sources_sha']}`; {rec['gpu']} on host "
                  f"`{rec['host']}`; {rec['date_utc']}.", ""]
        if wl == "prefill":
            lines += ["| K | N | M | W4A16 us | TFLOP/s | dense fp16 us | speedup | dequant+dense us | W4A8 us | plan |",
                      "|---|---|---|---|---|---|---|---|---|---|"]
            for r in res["rows"]:
                if "crossover_M_dense_faster_from" in r:
                    lines.append(f"| {r['K']} | {r['N']} | crossover: dense faster from M = "
                                 f"{r['crossover_M_dense_faster_from']} | | | | | | | |")
                elif r["M"] in (1, 16, 32, 64, 128, 256, 512, 1024, 2048):
                    lines.append(f"| {r['K']} | {r['N']} | {r['M']} | {r['w4a16_us']} | {r['w4a16_TFLOPs']} | "
                                 f"{r['dense_fp16_us']} | {r['speedup_vs_dense']} | {r['dequant_then_dense_us']} | "
                                 f"{r.get('w4a8_us', '')} | {r.get('plan', '')} |")
            lines.append("")
            continue
        roof = res["roofline"]
        step = roof.get("step", roof)
        lines.append(f"value {res['value']} GB/s ({step['frac']} of 8 TB/s), median step {res['ms_per_step']} ms, "
                     f"min {res.get('step_ms_min')} ms; read ceiling {step.get('read_ceiling_GBps')} GB/s "
                     f"(fraction {step.get('frac_of_read_ceiling')}); device copy {res['measured_copy_GBps']} GB/s.")
        if "step" in roof:
            lines.append(f"Roofline line (dominant kernel `{roof['kernel']}`, graph-timed calls): "
                         f"{roof['achieved']} GB/s = {roof['frac']} of 8 TB/s, {roof['avg_launch_us']} us per launch "
                         f"on {roof['alg_bytes_per_launch']} B; {roof.get('frac_of_read_ceiling')} of the read ceiling; "
                         f"HBM traffic {roof.get('traffic')} B per launch (counters).")
        if "dominant_kernel" in roof:
            dk = roof["dominant_kernel"]
            lines.append(f"Dominant kernel `{dk['name']}`: {dk['avg_ns']} ns per launch on {dk['alg_bytes_per_launch']} B, "
                         f"{dk['GBps']} GB/s, {dk['frac']} of 8 TB/s (kernel trace).")
        if "tokens_per_s" in res:
            gc = res["grouped_chain"]
            lines.append(f"chain: {res['tokens_per_s']} tok/s (225 launches, {res['us_per_token']} us/token); grouped "
                         f"{gc['tokens_per_s']} tok/s ({gc['launches_per_token']} launches, {gc['frac_hbm']} of 8 TB/s); "
                         f"ceiling {res['ceiling_tokens_per_s_at_8TBps']} tok/s at 8 TB/s.")
        if res.get("per_shape"):
            lines += ["", "| M | K | N | us | GB/s | of 8 TB/s | read ceiling us | of read ceiling | dense fp16 us |",
                      "|---|---|---|---|---|---|---|---|---|"]
            for r in res["per_shape"]:
                lines.append(f"| {r['M']} | {r['K']} | {r['N']} | {r['us']} | {r['GBps']} | {r['frac_hbm']} | "
                             f"{r.get('read_ceiling_us', '')} | {r.get('frac_of_read_ceiling', '')} | "
                             f"{r.get('dense_fp16_us', '')} |")
        if res.get("grouped"):
            lines += ["", "| grouped | M | us | GB/s | of 8 TB/s | one launch per matrix us | speedup |",
                      "|---|---|---|---|---|---|---|"]
            for g in res["grouped"]:
                lines.append(f"| {g['matrices']} | {g['M']} | {g['grouped_us']} | {g['grouped_GBps']} | "
                             f"{g['grouped_frac_hbm']} | {g['separate_launches_us']} | {g['speedup']} |")
        if res.get("cpu_baseline"):
            cb = res["cpu_baseline"]
            lines.append(f"\nOracle on the host: {cb['value']} GB/s ({cb['sample']}).")
        lines.append("")
    with open(os.path.join(ROOT, "profiles", "bench_records.md"), "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_sweep",
                    choices=["decode_sweep", "gemv_4096", "gemv_lm_head", "moe_expert", "shard_8", "chain_7b",
                             "prefill"])
    ap.add_argument("--group-size", type=int, default=GROUP, choices=[32, 64, 128, 256],
                    help="K rows per scale/zero group (decode workloads)")
    ap.add_argument("--symmetric", action="store_true",
                    help="symmetric quantiser (zero point 8) instead of min/max (decode workloads)")
    ap.add_argument("--layout", default="linear", choices=["linear", "interleaved"],
                    help="packing of the 4-bit codes in each int32 word")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense fp16 baseline")
    ap.add_argument("--no-grouped", action="store_true", help="skip the grouped-projection timings")
    ap.add_argument("--record", metavar="FILE", help="also write the JSON line with command, source hash and host")
    ap.add_argument("--trace-pass", action="store_true",
                    help="only the timed steps (for rocprofv3 --kernel-trace); prints no JSON")
    ap.add_argument("--summarize-kernel-trace", nargs="+", metavar="DIR")
    ap.add_argument("--summarize-records", nargs="+", metavar="FILE")
    ap.add_argument("--pmc-pass", action="store_true")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR")
    ap.add_argument("--summarize-prefill-pmc", nargs="+", metavar="DIR")
    ap.add_argument("--w4a8", action="store_true",
                    help="with --pmc-pass/--summarize-prefill-pmc: the W4A8 product kernel instead")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return 0
    if args.summarize_prefill_pmc:
        summarize_prefill_pmc(args.summarize_prefill_pmc, args.w4a8)
        return 0
    if args.summarize_kernel_trace:
        summarize_kernel_trace(args.summarize_kernel_trace)
        return 0
    if args.summarize_records:
        summarize_records(args.summarize_records)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the W4A16 path is built and timed on a single "
              "MI355X (no sharding or collectives); run it with --gpus 1.", file=sys.stderr)
        return 2
    if args.pmc_pass and args.workload == "prefill":
        run_prefill_pmc_pass(args)
    elif args.pmc_pass:
        run_pmc_pass(args)
    elif args.workload == "prefill":
        run_prefill(args)
    else:
        run_decode(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
