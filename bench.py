"""Benchmark of the W4A16 decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = the decode batch sweep: y = x . dequant(Wq) for M in {1,2,4,8,16} on each of
(K, N) = (4096, 14336), (14336, 4096), (4096, 4096), group 128 (15 launches). Inputs are
seeded synthetic data (synth.py) resident in HBM before timing; the packed weights rotate
over enough distinct device copies (>= 1 GiB per shape family) that no launch finds its
weights in the 256 MB Infinity Cache. The K timed steps are replayed from one HIP graph on
one stream and bracketed by HIP events on that stream.

Printed: one JSON line. `value` is the weight-stream rate over the whole timed region:
algorithmic bytes (int4 weights + fp16 scales/zeros + fp16 x + fp16 y) / time, in GB/s.
`roofline` relates the decode kernel's average launch to the 8 TB/s HBM peak;
`cpu_baseline` times the oracle (NumPy, fp64) on the host cores on one sweep.

Extra modes (profiling support):
  --pmc-pass               run a fixed copy calibration + a few sweep steps, eagerly, for
                           rocprofv3 --pmc; prints no JSON
  --summarize-pmc DIR...   read rocprofv3 counter CSVs of --pmc-pass runs and write the
                           per-launch HBM traffic summary to profiles/
"""
import argparse
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
GROUP = 128
SWEEP_KN = [(4096, 14336), (14336, 4096), (4096, 4096)]
SWEEP_M = [1, 2, 4, 8, 16]
WID = synth.WORKLOADS["decode_sweep"]["wid"]
ROTATE_BYTES = 1 << 30         # >= 4x the 256 MB Infinity Cache per shape family
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_skinny_decode_sweep.json")
KERNEL_SOURCES = ["weight_only_bit_gemv_amd/csrc/w4a16_skinny.hip",
                  "weight_only_bit_gemv_amd/csrc/w4a16_device.hpp",
                  "weight_only_bit_gemv_amd/csrc/w4a16_internal.h",
                  "weight_only_bit_gemv_amd/csrc/w4a16_api.cpp"]
COPY_CAL_BYTES = 256 << 20     # calibration copy for the PMC byte counters


def alg_bytes(M, K, N):
    """Algorithmic bytes of one call: int4 weights, fp16 scales + zeros, fp16 x and y."""
    return K * N // 2 + 2 * 2 * (K // GROUP) * N + 2 * M * K + 2 * M * N


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------------------

class Sweep:
    """Device-resident inputs of the decode sweep with rotating weight copies."""

    def __init__(self, torch, lib, dev, stream):
        self.torch, self.lib, self.dev, self.stream = torch, lib, dev, stream
        self.weights = {}       # (K, N) -> list of (qw, s, z) device copies
        self.host = {}          # (K, N) -> host (qw, s, z)
        for (K, N) in SWEEP_KN:
            t0 = time.time()
            W = synth.weight(K, N, wid=WID)
            qw, s, z = lib.w4a16_pack(W)
            del W
            self.host[(K, N)] = (qw, s, z)
            one = [torch.from_numpy(a).to(dev) for a in (qw, s, z)]
            per = sum(t.numel() * t.element_size() for t in one)
            copies = max(2, -(-ROTATE_BYTES // per))
            self.weights[(K, N)] = [one] + [[t.clone() for t in one] for _ in range(copies - 1)]
            log(f"[bench] weights K={K} N={N}: {copies} copies x {per / 1e6:.1f} MB "
                f"({time.time() - t0:.1f}s)")
        self.shapes = [(M, K, N) for (K, N) in SWEEP_KN for M in SWEEP_M]
        self.x = {(M, K): torch.from_numpy(synth.activations(M, K, wid=WID)).to(dev)
                  for (M, K, N) in self.shapes}
        self.y = {(M, K, N): torch.empty((M, N), dtype=torch.float16, device=dev)
                  for (M, K, N) in self.shapes}
        self.cursor = {kn: 0 for kn in SWEEP_KN}
        self.step_bytes = sum(alg_bytes(M, K, N) for (M, K, N) in self.shapes)
        so = lib.load()
        self.fn = so.w4a16_matmul
        self.sptr = stream.cuda_stream

    def launch(self, M, K, N):
        kn = (K, N)
        i = self.cursor[kn]
        self.cursor[kn] = (i + 1) % len(self.weights[kn])
        qw, s, z = self.weights[kn][i]
        rc = self.fn(self.x[(M, K)].data_ptr(), qw.data_ptr(), s.data_ptr(), z.data_ptr(),
                     self.y[(M, K, N)].data_ptr(), M, N, K, GROUP, self.sptr)
        if rc != 0:
            raise RuntimeError(f"w4a16_matmul failed ({rc}) for M={M} K={K} N={N}")

    def step(self):
        for (M, K, N) in self.shapes:
            self.launch(M, K, N)


def time_graph(torch, stream, body, reps, warm=2):
    """Capture `body` once into a HIP graph on `stream`; replay `reps` times between HIP
    events recorded on the same stream. Returns seconds per replay."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        body()
    for _ in range(warm):
        g.replay()
    stream.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps, g


def copy_bandwidth(torch, dev, stream):
    """Achievable HBM rate of a plain device copy (read + write bytes / time)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    with torch.cuda.stream(stream):
        for _ in range(3):
            b.copy_(a)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            b.copy_(a)
        e1.record(stream)
    e1.synchronize()
    return 2 * n * 10 / (e0.elapsed_time(e1) / 1e3) / 1e9


def dense_baseline(torch, lib, sw, dev, stream):
    """torch fp16 matmul (hipBLASLt/rocBLAS) on the same shapes with fp16 weights that are
    the GPU's dequantised values, rotated the same way. Returns per-shape seconds.

    Timed eagerly, never inside a HIP graph: a library GEMM may reset its own split-K flags
    with a memset, which does not replay correctly from a captured graph. The GPU stays
    ahead of the host for these sizes, so back-to-back eager calls measure the kernels."""
    out = {}
    for (K, N) in SWEEP_KN:
        qw, s, z = sw.weights[(K, N)][0]
        _, w16 = lib.w4a16_dequant(qw, s, z, codes=False)
        per = w16.numel() * 2
        copies = max(2, -(-ROTATE_BYTES // per))
        ws = [w16] + [w16.clone() for _ in range(copies - 1)]
        for M in SWEEP_M:
            x = sw.x[(M, K)]
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            reps = 4 * len(ws)
            with torch.cuda.stream(stream):
                for i in range(len(ws)):                       # warm-up (library initialisation)
                    torch.matmul(x, ws[i], out=y)
                stream.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(reps):
                    torch.matmul(x, ws[i % len(ws)], out=y)
                e1.record(stream)
            e1.synchronize()
            out[(M, K, N)] = e0.elapsed_time(e1) / 1e3 / reps
        del ws
    return out


def cpu_baseline(sw):
    """The oracle as it stands (unpack + exact dequant + fp64 BLAS matmul) on one sweep."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = None
    total_bytes = 0
    t0 = time.perf_counter()
    for (M, K, N) in sw.shapes:
        qw, s, z = sw.host[(K, N)]
        x = synth.activations(M, K, wid=WID)
        oracle.matmul(x, qw, s, z)
        total_bytes += alg_bytes(M, K, N)
    dt = time.perf_counter() - t0
    return {"value": round(total_bytes / dt / 1e9, 4), "unit": "GB/s",
            "cores": blas_threads,
            "kind": "oracle",
            "sample": (f"one pass over the 15 decode-sweep GEMMs (same shapes and data), "
                       f"{dt:.1f} s; NumPy elementwise unpack/dequant on 1 thread, fp64 BLAS "
                       f"matmul on {blas_threads} threads of "
                       f"{len(os.sched_getaffinity(0))} available")}


def load_traffic(launches_per_step):
    """Measured HBM bytes per launch from the committed PMC summary, if it was taken on the
    current kernel source (else None)."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha") != kernel_source_hash():
        return None
    return d.get("traffic_bytes_per_launch")


# ---------------------------------------------------------------------------------------

def run_bench(args):
    import torch
    import weight_only_bit_gemv_amd as lib

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)
    sw = Sweep(torch, lib, dev, stream)
    launches = len(sw.shapes)

    # eager warm-up on the bench stream (allocates the split-K workspace for this stream)
    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup)):
            sw.step()
    stream.synchronize()
    eager_ref = {k: v.clone() for k, v in sw.y.items()}

    # timed region: K steps replayed from one graph
    steps = args.steps

    def body():
        for _ in range(steps):
            sw.step()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        body()
    for _ in range(max(0, args.warmup)):
        g.replay()
    stream.synchronize()
    for k, v in sw.y.items():        # every replay must reproduce the eager results
        if not torch.equal(v, eager_ref[k]):
            raise RuntimeError(f"graph replay differs from eager result for {k}")
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        g.replay()
        e1.record(stream)
    e1.synchronize()
    torch.cuda.synchronize()
    elapsed = e0.elapsed_time(e1) / 1e3
    total_bytes = sw.step_bytes * steps
    value = total_bytes / elapsed / 1e9
    avg_launch_s = elapsed / (steps * launches)
    for k, v in sw.y.items():
        if not torch.equal(v, eager_ref[k]):
            raise RuntimeError(f"timed replay differs from eager result for {k}")

    # eager (no graph) rate for reference: includes host launch cost
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(steps):
            sw.step()
        e1.record(stream)
    e1.synchronize()
    eager_elapsed = e0.elapsed_time(e1) / 1e3

    # per-shape timing (graph of one launch per rotation copy)
    per_shape = []
    for (M, K, N) in sw.shapes:
        reps = len(sw.weights[(K, N)])
        sec, _ = time_graph(torch, stream, lambda: [sw.launch(M, K, N) for _ in range(reps)], 5)
        t = sec / reps
        b = alg_bytes(M, K, N)
        per_shape.append({"M": M, "K": K, "N": N, "us": round(t * 1e6, 3),
                          "GBps": round(b / t / 1e9, 1),
                          "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 4),
                          "TFLOPs": round(2 * M * K * N / t / 1e12, 3),
                          "plan": lib.w4a16_plan(M, N, K)})
    del g

    copy_gbs = copy_bandwidth(torch, dev, stream)
    dense = {} if args.no_dense else dense_baseline(torch, lib, sw, dev, stream)
    for r in per_shape:
        d = dense.get((r["M"], r["K"], r["N"]))
        if d:
            r["dense_fp16_us"] = round(d * 1e6, 3)
            r["speedup_vs_dense_fp16"] = round(d / (r["us"] / 1e6), 3)

    traffic = load_traffic(launches)
    achieved = sw.step_bytes / launches / avg_launch_s / 1e9
    result = {
        "metric": "W4A16 weight-stream HBM GB/s (% of peak) and us/call at M=1..16",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode_sweep: M in {1,2,4,8,16} x (K,N) in {(4096,14336),"
                               "(14336,4096),(4096,4096)}, int4 weights packed 8/int32 along K, "
                               "fp16 scale+zero per 128-row group",
                   "launches_per_step": launches,
                   "bytes_per_step": sw.step_bytes,
                   "timing": "HIP graph of all steps, events on the launch stream",
                   "weight_copies_rotated": {f"{k}x{n}": len(v) for (k, n), v in sw.weights.items()}},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "skinny_kernel (decode split-K MFMA)",
                     "avg_launch_us": round(avg_launch_s * 1e6, 3)},
        "measured_copy_GBps": round(copy_gbs, 1),
        "frac_of_measured_copy": round(value / copy_gbs, 4),
        "eager_ms_per_step": round(eager_elapsed / steps * 1e3, 4),
        "per_shape": per_shape,
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(sw)
    print(json.dumps(result), flush=True)


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
    sw = Sweep(torch, lib, dev, stream)
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            sw.step()
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
    summary = {"kernel_source_sha": kernel_source_hash(),
               "workload": "decode_sweep (15 shapes), mean over dispatches",
               "traffic_bytes_per_launch": round(traffic),
               "algorithmic_bytes_per_launch": round(alg),
               "traffic_over_algorithmic": round(traffic / alg, 4),
               "counters": out}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(summary, f, indent=1)
        f.write("\n")
    print(json.dumps(summary, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense fp16 baseline")
    ap.add_argument("--pmc-pass", action="store_true")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the W4A16 path is built and timed on a single "
              "MI355X (no sharding or collectives); run it with --gpus 1.", file=sys.stderr)
        return 2
    if args.pmc_pass:
        run_pmc_pass(args)
        return 0
    run_bench(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
