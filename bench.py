"""Benchmark of the DVM hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input: for
the LayerNorm stream (the metric's workload) that is 64 LayerNorm calls, each
with a new row count R = B*S (B ~ U{1..32}, S ~ U{1..4096}) over H = 5120,
each captured through the C ABI as a fused group, shape-tiled, encoded to
bytecode on the host and run by the resident VM kernel.  The timed region
includes capture, fusion decisions, encoding and launches; inputs are already
in HBM.  Throughput counts algorithmic bytes: x read and y written (bf16) plus
gamma/beta (fp32) per call.

The default run (--config all) prints one JSON line whose headline fields are
the LayerNorm stream's, plus a "configs" object with the other workloads,
each measured in the same run: sqrt(a + b) (warm and cold kernel time),
if-else-add (reduce-all and host-resolved branch: device-only and end to
end), MatMul+bias+SiLU (MIX kernel, against the matrix-core roofline) and the
transformer op stream (10,000 motifs per step through the streaming fuser, T
and T_kv drawn per step).  --config NAME runs one workload alone and prints
its own line with the same fields.

Device time is measured with HIP events recorded on the launch stream around
the timed region; encode latency and fuser cost are read from the library's
own clock (steady_clock inside dvm_flush and the fuser calls), not timed
around the Python binding.  The CPU baseline (the oracle, numpy fp64) runs
before the GPU is touched, on one core and on all the host cores this process
may use.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "VM-interpreted fused-op HBM GB/s (% of peak) + bytecode encode µs per graph"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0    # MI355X dense bf16
CONFIGS = ["all", "layernorm", "sqrt_add", "ifelse", "matmul", "stream"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="all", choices=CONFIGS)
    ap.add_argument("--calls", type=int, default=0, help="calls per step for ifelse / matmul (0: default)")
    ap.add_argument("--motifs", type=int, default=10000, help="motifs per step for the op stream")
    ap.add_argument("--stream-steps", type=int, default=2, help="timed op-stream steps (seeds 0, 1, ...)")
    ap.add_argument("--stacking", type=int, default=7,
                    help="independent graphs packed into one launch (1: every graph launches alone)")
    ap.add_argument("--stack-order", default="spatial", choices=["spatial", "temporal"],
                    help="stacked segments on their own workgroups, or in sequence on every workgroup")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=6.0, help="CPU work per baseline leg")
    ap.add_argument("--no-decode-split", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain device copy of known size (counter calibration)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="derive the VM kernel's HBM bytes per launch from rocprofv3 counter files and store them")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# counter-measured traffic (stored by --traffic-from, read while the sources
# that decide it -- kernels and encoder -- are unchanged)
# ---------------------------------------------------------------------------
COPY_BYTES = 512 << 20          # bytes read (and written) by the calibration copy
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_dvm_vm_vector_layernorm_stream.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "device_bytecode_vm_amd", "csrc", f)
                  for f in ("vm_vector.hip", "vm_vector_wide.hip", "bytecode.h", "dvm_host.cpp")]


def kernel_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per launch measured by counters for the current sources, or
    None when the kernel or the encoder changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.loads(fh.read().split("\n", 1)[1])
    except (OSError, ValueError, IndexError):
        return None
    if rec.get("kernel_sha256_16") != kernel_hash():
        return None
    return rec


def counter_per_dispatch(path, kernel):
    import csv
    per = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if kernel in r["Kernel_Name"]:
                per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return per


def traffic_from(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the VM kernel over one
    bench step, each scaled by what the counter reads for a plain copy of
    COPY_BYTES; averaged per launch."""
    cf = counter_per_dispatch(copy_fetch_csv, "")
    cw = counter_per_dispatch(copy_write_csv, "")
    f_scale = COPY_BYTES / (max(cf.values()) * 1024.0)   # the calibration copy is the largest dispatch
    w_scale = COPY_BYTES / (max(cw.values()) * 1024.0)
    vf = {k: v for k, v in counter_per_dispatch(fetch_csv, "dvm_vm_vector").items() if k not in
          counter_per_dispatch(fetch_csv, "_prof")}
    vw = {k: v for k, v in counter_per_dispatch(write_csv, "dvm_vm_vector").items() if k not in
          counter_per_dispatch(write_csv, "_prof")}
    n = min(len(vf), len(vw))
    fetch = sum(vf.values()) / len(vf) * 1024.0 * f_scale
    write = sum(vw.values()) / len(vw) * 1024.0 * w_scale
    rec = {"kernel_sha256_16": kernel_hash(), "dispatches": n, "fetch_bytes_per_launch": round(fetch),
           "write_bytes_per_launch": round(write), "traffic_bytes_per_launch": round(fetch + write),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("# HBM traffic of the VECTOR VM (dvm_vm_vector, dvm_vm_vector_wide) on the LayerNorm stream "
                 "(see the counter commands in profiles/README.md)\n" + json.dumps(rec) + "\n")
    return rec


def calibrate_copy():
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": COPY_BYTES}), flush=True)


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------
def pctl(xs, q):
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q)) if len(xs) else 0.0


def encode_stats(log):
    """p50 / p99 / max of the library's own encode times (µs per graph)."""
    us = [e[2] for e in log]
    return {"p50": round(pctl(us, 50), 2), "p99": round(pctl(us, 99), 2), "max": round(max(us) if us else 0.0, 2),
            "graphs": len(us), "clock": "steady_clock inside dvm_flush (tiling + bytecode)"}


class Span:
    """Device time between two events recorded on `stream` (ms)."""

    def __init__(self, stream):
        import torch
        self.stream = stream
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.a.record(self.stream)
        return self

    def __exit__(self, *exc):
        self.b.record(self.stream)

    def ms(self):
        import torch
        torch.cuda.synchronize()
        return self.a.elapsed_time(self.b)


def _event_time(stream, fn, reps):
    """Device time per call of fn (seconds) after one untimed call."""
    import torch
    fn()
    torch.cuda.synchronize()
    with Span(stream) as sp:
        for _ in range(reps):
            fn()
    return sp.ms() / reps * 1e-3


# ---------------------------------------------------------------------------
# CPU baseline: the oracle (numpy fp64), before any GPU work
# ---------------------------------------------------------------------------
def host_cores():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))       # the share of a one-GPU machine's host cores


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _parallel(fn, items, n):
    """fn over items on n threads (numpy releases the GIL inside its array
    loops); returns the wall time of the parallel phase."""
    chunks = [items[i::n] for i in range(n)]
    bar = threading.Barrier(n + 1)
    t = [0.0, 0.0]

    def work(ch):
        bar.wait()
        for it in ch:
            fn(it)
        bar.wait()

    th = [threading.Thread(target=work, args=(c,)) for c in chunks]
    for x in th:
        x.start()
    bar.wait()
    t[0] = time.perf_counter()
    bar.wait()
    t[1] = time.perf_counter()
    for x in th:
        x.join()
    return t[1] - t[0]


def cpu_baselines(budget_s):
    """Oracle throughput on bounded samples of each workload: one core, and
    (LayerNorm, the headline) all cores.  Inputs are drawn before timing."""
    from threadpoolctl import threadpool_limits
    from oracle import ops as O
    import workloads as W
    cores = host_cores()
    res = {"cpu_model": cpu_model(), "cores_available": cores}
    H = W.H_LN
    gam, bet = W.layernorm_params()
    # LayerNorm: blocks of 512 rows from the stream's calls
    shapes = W.layernorm_shapes(0, 64)
    blocks = [W.layernorm_x(0, i, min(r, 512), H) for i, (r, _) in enumerate(shapes[:16])]
    with threadpool_limits(1):
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            for x in blocks:
                O.layer_norm(x, gam, bet, W.LN_EPS)
                done += x.shape[0]
        t1 = time.perf_counter() - t0
        one = done * H * 4 / t1 / 1e9
        reps = max(1, int(done / sum(b.shape[0] for b in blocks)))
        items = [b for _ in range(reps) for b in blocks]      # the same work, split over the threads
        wall = _parallel(lambda x: O.layer_norm(x, gam, bet, W.LN_EPS), items, cores)
        allc = sum(b.shape[0] for b in items) * H * 4 / wall / 1e9
    res["layernorm"] = {
        "value": round(allc, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
        "value_1core": round(one, 4),
        "sample": f"16 calls of the LayerNorm stream, first min(R, 512) rows each ({sum(b.shape[0] for b in blocks)} "
                  f"rows x 5120), repeated; numpy fp64; 1 core {t1:.1f} s, {cores} threads {wall:.1f} s; "
                  f"CPU {res['cpu_model']}"}
    # sqrt(a + b), if-else-add, op stream: one core
    with threadpool_limits(1):
        a, b = W.vv_sqrt_add(0, (513, 1031))
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < budget_s / 4:
            O.sqrt(O.add(a, b))
            n += 1
        res["sqrt_add"] = {"value": round(n * a.size * 12 / (time.perf_counter() - t0) / 1e9, 4), "unit": "GB/s",
                           "cores": 1, "kind": "oracle", "sample": f"{n} evaluations of the full (513, 1031) graph"}
        xs = [W.ifelse_inputs(0, i, (min(r, 512), c))[:2] for i, (r, c) in enumerate(W.ifelse_shapes(0)[:8])]
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < budget_s / 4:
            for x, y in xs:
                O.if_else_add(x, y)
                n += x.size
        res["if_else_add"] = {"value": round(n * 16 / (time.perf_counter() - t0) / 1e9, 4), "unit": "GB/s",
                              "cores": 1, "kind": "oracle",
                              "sample": "8 calls, first min(N, 512) rows of 4096 each, repeated"}
        rg = W.rng(0)
        T, TKV = 64, 6484
        ins = {"add": (rg.normal(size=(T, H)), rg.normal(size=(T, H))),
               "rmsnorm": (rg.normal(size=(T, H)),), "swiglu": (rg.normal(size=(T, W.N_FFN)),
                                                            rg.normal(size=(T, W.N_FFN))),
               "softmax": (rg.normal(size=(T, TKV)),)}
        mb = {"add": 3 * T * H * 2, "rmsnorm": 2 * T * H * 2, "swiglu": 3 * T * W.N_FFN * 2,
              "softmax": 2 * T * TKV * 2}
        w1 = np.ones(H)
        done, t0, k = 0, time.perf_counter(), 0
        motifs = W.stream_step(0, 400)[2]
        while time.perf_counter() - t0 < budget_s / 4:
            kind = motifs[k % len(motifs)][0]
            if kind == "add":
                O.add(*ins["add"])
            elif kind == "rmsnorm":
                O.rms_norm(ins["rmsnorm"][0], w1, W.RMS_EPS)
            elif kind == "swiglu":
                O.swiglu(*ins["swiglu"])
            else:
                O.softmax(ins["softmax"][0])
            done += mb[kind]
            k += 1
        res["op_stream"] = {"value": round(done / (time.perf_counter() - t0) / 1e9, 4), "unit": "GB/s",
                            "cores": 1, "kind": "oracle",
                            "sample": f"{k} motifs of the stream on 64-row slices (softmax rows of 6484)"}
    # MatMul+bias+SiLU: 64 rows at a time; BLAS on all cores (B drawn in
    # fp32 directly: the timing does not depend on the values)
    g1 = W.rng(1)
    b_ = g1.standard_normal((W.K_MM, W.N_FFN), dtype=np.float32) * np.float32(0.02)
    bias = g1.standard_normal(W.N_FFN) * 0.02
    a_ = W.matmul_a(0, 0, 64)
    with threadpool_limits(cores):
        rows, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < budget_s / 4:
            O.matmul_bias_silu(a_, b_, bias)
            rows += 64
        dt = time.perf_counter() - t0
    res["matmul_bias_silu"] = {"value": round(rows * 2.0 * W.K_MM * W.N_FFN / dt / 1e12, 6), "unit": "TFLOP/s",
                               "cores": cores, "kind": "oracle",
                               "sample": f"{rows} rows in 64-row blocks at K=5120, N=17408, numpy fp64 (BLAS)"}
    return res


# ---------------------------------------------------------------------------
# LayerNorm stream (the headline)
# ---------------------------------------------------------------------------
def layernorm_bench(args):
    import torch
    import device_bytecode_vm_amd as dvm
    from device_bytecode_vm_amd import composites as CP
    import workloads as W

    shapes = W.layernorm_shapes(0, 64)
    H = W.H_LN
    ctx = dvm.Context(0)
    stream = torch.cuda.current_stream()
    xs = [W.device_normal((r, H), seed=1000 + i, dtype="bf16") for i, (r, _) in enumerate(shapes)]
    gam = W.device_normal((H,), seed=1, mu=1.0, sd=0.1)
    bet = W.device_normal((H,), seed=2, mu=0.0, sd=0.1)
    # every call writes its own output (independent calls, as in a model's
    # layers), so the stream's graphs may share launches
    ys = [torch.empty((r, H), dtype=torch.bfloat16, device="cuda") for r, _ in shapes]
    call_bytes = [r * H * 2 * 2 + 2 * H * 4 for r, _ in shapes]
    step_bytes = float(sum(call_bytes))
    torch.cuda.synchronize()

    def one_step(g):
        for x, y in zip(xs, ys):
            CP.layer_norm(g, g.input(x), g.input(gam), g.input(bet), W.LN_EPS, out=y)
        g.flush_launch()

    g = dvm.Graph(ctx, stream)
    g.set_stacking(args.stacking, args.stack_order == "temporal")
    for _ in range(args.warmup):
        one_step(g)
    torch.cuda.synchronize()
    s0 = g.stats()
    n_log0 = len(g.flush_log())
    t0 = time.perf_counter()
    with Span(stream) as sp:
        for _ in range(args.steps):
            one_step(g)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dev_ms = sp.ms()
    s1 = g.stats()
    log = g.flush_log(detail=True)[n_log0:]
    ms_step = (t1 - t0) * 1e3 / args.steps
    e2e_gbs = step_bytes * args.steps / (t1 - t0) / 1e9
    launches = s1["launches"] - s0["launches"]
    avg_launch_s = dev_ms * 1e-3 / max(launches, 1)
    kern_gbs = step_bytes * args.steps / (dev_ms * 1e-3) / 1e9      # = bytes per launch / launch time
    fuse_us = (s1["fuse_us_total"] - s0["fuse_us_total"]) / max(s1["ops"] - s0["ops"], 1)

    progs = []
    for x, y in zip(xs, ys):
        gp = dvm.Graph(ctx, stream)
        CP.layer_norm(gp, gp.input(x), gp.input(gam), gp.input(bet), W.LN_EPS, out=y)
        progs.append(gp.flush())
    hdr = progs[int(np.argmax([r for r, _ in shapes]))].header()
    tr = stored_traffic()
    traffic = tr["traffic_bytes_per_launch"] if tr else None
    decode = None if args.no_decode_split else decode_split(progs, stream)

    out = {
        "metric": METRIC, "value": round(e2e_gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "layernorm_stream", "calls_per_step": 64, "hidden": H,
                   "rows": "R=B*S, B~U{1..32}, S~U{1..4096}, seed 0",
                   "rows_total_per_step": int(sum(r for r, _ in shapes)), "eps": W.LN_EPS,
                   "x_dtype": "bf16", "gamma_beta_dtype": "f32", "y_dtype": "bf16"},
        "encode_us": encode_stats(log),
        "fuse_us_per_op": round(fuse_us, 3),
        "device_ms_per_step": round(dev_ms / args.steps, 4),
        "graphs_per_step": (s1["graphs"] - s0["graphs"]) / args.steps,
        "roofline": {"bound": "hbm", "achieved": round(kern_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kern_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "dvm_vm_vector_wide + dvm_vm_vector", "launches_per_step": launches / args.steps,
                     "graphs_stacked_per_step": (s1["stacked"] - s0["stacked"]) / args.steps,
                     "stacking": args.stacking, "stack_order": args.stack_order,
                     "launches_by_kernel": {
                         "dvm_vm_vector_wide": sum(1 for p in progs if p.header()["kernel_type"] == 2),
                         "dvm_vm_vector": sum(1 for p in progs if p.header()["kernel_type"] == 0)},
                     "avg_launch_us": round(avg_launch_s * 1e6, 3),
                     "timing": "HIP events on the launch stream around the timed steps; avg launch = device span / "
                               "launches (gaps between back-to-back launches included)",
                     "bytes_per_launch_avg": round(step_bytes * args.steps / max(launches, 1), 1)},
        "largest_call_header": {k: hdr[k] for k in ("block_dim", "body_tile", "grid", "tr", "tc", "g", "nv",
                                                    "n_instr")},
        "decode_split": decode,
    }
    return out


def decode_split(progs, stream):
    """One pass of the programs through the VM's profiling twin (outside the
    timed region): the share of each workgroup's cycles spent decoding
    (instruction fetch, field decode, dispatch), executing handlers and
    changing tiles, summed over workgroups and programs."""
    import torch
    tot = np.zeros(5)
    for p in progs:
        n = p.PROF_COUNTERS * p.header()["grid"]
        c = torch.zeros(max(n, 1), dtype=torch.int64, device="cuda")
        p.launch_profiled(c, stream)
        torch.cuda.synchronize()
        tot += c.view(-1, p.PROF_COUNTERS).sum(0).cpu().numpy().astype(np.float64)
    total = max(tot[0], 1.0)
    return {"decode_frac": round(tot[1] / total, 4), "execute_frac": round(tot[2] / total, 4),
            "tile_change_frac": round(tot[3] / total, 4),
            "decode_cycles_per_dispatch": round(tot[1] / max(tot[4], 1.0), 1),
            "execute_cycles_per_dispatch": round(tot[2] / max(tot[4], 1.0), 1),
            "dispatches": int(tot[4]), "counter": "s_memtime, wave 0 of each workgroup, profiling twin kernel"}


# ---------------------------------------------------------------------------
# sqrt(a + b): one 6.3 MB graph
# ---------------------------------------------------------------------------
def sqrt_add_bench(args):
    import torch
    import device_bytecode_vm_amd as dvm
    import workloads as W
    ctx = dvm.Context(0)
    stream = torch.cuda.current_stream()
    a = W.device_uniform((513, 1031), 1)
    b = W.device_uniform((513, 1031), 2)
    c = torch.empty_like(a)
    nbytes = 3 * a.numel() * 4
    g = dvm.Graph(ctx, stream)

    def one():
        t = g.op("add", g.input(a), g.input(b))
        g.op("sqrt", t, out=c, live=True)
        g.release(t)
        g.flush_launch()

    for _ in range(max(args.warmup, 1)):
        one()
    torch.cuda.synchronize()
    n = 200
    n_log0 = len(g.flush_log())
    t0 = time.perf_counter()
    for _ in range(n):
        one()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / n
    log = g.flush_log(detail=True)[n_log0:]
    gp = dvm.Graph(ctx, stream)
    t = gp.op("add", gp.input(a), gp.input(b))
    gp.op("sqrt", t, out=c, live=True)
    gp.release(t)
    p = gp.flush()
    kus = _event_time(stream, lambda: p.launch(stream), 200) * 1e6
    # cold: a 512 MiB write between launches evicts the operands from L2 and
    # the MALL; median over the launches
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    for i in range(30):
        scratch.fill_(i & 0xff)
        with Span(stream) as sp:
            p.launch(stream)
        cold.append(sp.ms() * 1e3)
    del scratch
    kus_cold = sorted(cold)[len(cold) // 2]
    return {"metric": METRIC, "value": round(nbytes / dt / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
            "steps": n, "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "sqrt_add", "shape": [513, 1031]},
            "encode_us": encode_stats(log),
            "device_only_gbs": round(nbytes / (kus * 1e-6) / 1e9, 2), "kernel_us_warm": round(kus, 3),
            "kernel_us_cold": round(kus_cold, 3),
            "device_only_gbs_cold": round(nbytes / (kus_cold * 1e-6) / 1e9, 2),
            "roofline": {"bound": "hbm", "achieved": round(nbytes / (kus_cold * 1e-6) / 1e9, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(nbytes / (kus_cold * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": None, "kernel": "dvm_vm_vector", "timing": "cold launches (caches evicted)"},
            "note": "one 6.3 MB graph is launch-latency bound: 70% of the HBM roofline is out of reach",
            "header": {k: p.header()[k] for k in ("block_dim", "body_tile", "grid", "tr", "tc", "nv")}}


# ---------------------------------------------------------------------------
# MatMul + bias + SiLU (MIX kernel)
# ---------------------------------------------------------------------------
def matmul_bench(args):
    import torch
    import device_bytecode_vm_amd as dvm
    from device_bytecode_vm_amd import composites as CP
    import workloads as W
    calls = args.calls or 32
    ms = W.matmul_ms(0)[:calls]
    K, N = W.K_MM, W.N_FFN
    ctx = dvm.Context(0)
    stream = torch.cuda.current_stream()
    b = W.device_normal((K, N), seed=1, sd=0.02, dtype="bf16")
    bias = W.device_normal((N,), seed=2, sd=0.02)
    mmax = max(ms)
    a = W.device_normal((mmax, K), seed=3, sd=0.02, dtype="bf16")
    y = torch.empty((mmax, N), dtype=torch.bfloat16, device="cuda")
    flops = float(sum(2.0 * m * K * N for m in ms))
    nbytes = float(sum(2 * m * K + 2 * K * N + 4 * N + 2 * m * N for m in ms))
    g = dvm.Graph(ctx, stream)
    steps = max(1, min(args.steps, 5))

    def one_step():
        for m in ms:
            CP.matmul_bias_silu(g, g.input(a[:m]), g.input(b), g.input(bias), out=y[:m])
        g.flush_launch()

    for _ in range(max(1, min(args.warmup, 2))):
        one_step()
    torch.cuda.synchronize()
    n_log0 = len(g.flush_log())
    t0 = time.perf_counter()
    with Span(stream) as sp:
        for _ in range(steps):
            one_step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    kt = sp.ms() * 1e-3 / steps
    log = g.flush_log(detail=True)[n_log0:]
    tt = _event_time(stream, lambda: [torch.matmul(a[:m], b) for m in ms], 2)
    kern = flops / kt / 1e12
    # per-call bound: min(matrix peak, arithmetic intensity x HBM peak)
    bound_s = sum(max(2.0 * m * K * N / (MFMA_PEAK_TFLOPS * 1e12), (2 * m * K + 2 * K * N + 2 * m * N) / 8e12)
                  for m in ms)
    return {"metric": "MatMul+bias+SiLU TFLOP/s (MIX VM kernel)", "value": round(flops / dt / 1e12, 2),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
            "ms_per_step": round(dt * 1e3, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "matmul_bias_silu", "calls_per_step": len(ms), "K": K, "N": N,
                       "M": "distinct M ~ U{1..8192}, seed 0", "rows_total": int(sum(ms))},
            "encode_us": encode_stats(log),
            "device_only_tflops": round(kern, 2),
            "roofline": {"bound": "mfma", "achieved": round(kern, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(kern / MFMA_PEAK_TFLOPS, 4), "traffic": None, "kernel": "dvm_vm_mix",
                         "launches_per_step": len(ms), "avg_launch_us": round(kt / len(ms) * 1e6, 2),
                         "frac_of_per_call_bound": round(bound_s / kt, 4),
                         "algorithmic_bytes_per_step": nbytes},
            "context": {"torch_matmul_tflops_same_shapes": round(flops / tt / 1e12, 2)}}


# ---------------------------------------------------------------------------
# if (sum(x) > 0) x + y else x - y: reduce-all, host-resolved branch
# ---------------------------------------------------------------------------
def ifelse_bench(args):
    import torch
    import device_bytecode_vm_amd as dvm
    import workloads as W
    calls = args.calls or 256
    shapes = W.ifelse_shapes(0)[:calls]
    coin = W.rng(0).random(calls) < 0.5
    nmax = max(r for r, _ in shapes)
    C = shapes[0][1]
    ctx = dvm.Context(0)
    stream = torch.cuda.current_stream()
    # mean 0.125 puts sum(x) at least 8 standard deviations from zero for every size
    xp = W.device_normal((nmax, C), seed=11, mu=0.125)
    xn = W.device_normal((nmax, C), seed=12, mu=-0.125)
    yy = W.device_normal((nmax, C), seed=13)
    out = torch.empty_like(yy)
    s = torch.empty((), dtype=torch.float32, device="cuda")
    # the host reads the sum through pinned memory: the copy is queued behind
    # the reduce-all and the graph's sync waits for both (one round trip)
    s_host = torch.empty((), dtype=torch.float32, pin_memory=True)
    nbytes = float(sum(16.0 * r * C for r, _ in shapes))
    g = dvm.Graph(ctx, stream)
    taken = []
    steps = max(1, min(args.steps, 3))

    def one_step():
        taken.clear()
        for (r, _), c in zip(shapes, coin):
            x = (xp if c else xn)[:r]
            vx, vy = g.input(x), g.input(yy[:r])
            g.op("reduce_sum", vx, out=s, live=True, axis=0x7FFFFFFF)
            s_host.copy_(s, non_blocking=True)
            g.sync()
            sv = float(s_host)
            taken.append(sv > 0)
            g.op("add" if sv > 0 else "sub", vx, vy, out=out[:r], live=True)
            g.flush_launch()
        torch.cuda.synchronize()

    one_step()
    t0 = time.perf_counter()
    for _ in range(steps):
        one_step()
    dt_host = (time.perf_counter() - t0) / steps
    assert taken == [bool(c) for c in coin], "branch differs from the sign the input was drawn with"

    # device-side branch: a branch program per call reads the reduce-all's
    # result on the device, so calls queue back to back (one sync per step)
    gd = dvm.Graph(ctx, stream)

    # (begin_branch_reduce: the branch program folds the reduce-all's
    # workgroup partials itself, so each call is two launches, not three)
    def dev_queue():
        for (r, _), c in zip(shapes, coin):
            vx, vy = gd.input((xp if c else xn)[:r]), gd.input(yy[:r])
            gd.begin_branch_reduce(vx, s, 0.0)
            gd.op("add", vx, vy, out=out[:r], live=True)
            gd.else_branch()
            gd.op("sub", vx, vy, out=out[:r], live=True)
            gd.end_branch()

    def dev_step():
        dev_queue()
        torch.cuda.synchronize()

    dev_step()
    n_log0 = len(gd.flush_log())
    t0 = time.perf_counter()
    for _ in range(steps):
        dev_step()
    dt = (time.perf_counter() - t0) / steps
    log = gd.flush_log(detail=True)[n_log0:]
    # device-only: the branch is known from the input's sign, so every call's
    # reduce-all (launched when it closes its graph) and branch program are
    # queued back to back with no host sync
    progs = []
    for (r, _), c in zip(shapes, coin):
        gp = dvm.Graph(ctx, stream)
        gp.op("add" if c else "sub", gp.input((xp if c else xn)[:r]), gp.input(yy[:r]), out=out[:r], live=True)
        progs.append(gp.flush())
    gk = dvm.Graph(ctx, stream)

    def queued():
        for (r, _), c, p in zip(shapes, coin, progs):
            gk.op("reduce_sum", gk.input((xp if c else xn)[:r]), out=s, live=True, axis=0x7FFFFFFF)
            p.launch(stream)

    kq = _event_time(stream, queued, steps)
    # the device-branch path on the device: events on the stream around the
    # queued calls (sum, then the branch program), no host sync inside
    kt = _event_time(stream, dev_queue, steps)
    kern = nbytes / kt / 1e9
    return {"metric": METRIC, "value": round(nbytes / dt / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
            "steps": steps, "warmup": 1, "ms_per_step": round(dt * 1e3, 3),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "if_else_add", "calls_per_step": len(shapes), "cols": C,
                       "rows": "N ~ U{1..16384}, seed 0",
                       "branch": "device-side: a branch program reads the reduce-all's result on the GPU",
                       "add_branch_calls": int(sum(coin))},
            "encode_us": encode_stats(log),
            "e2e_host_branch_gbs": round(nbytes / dt_host / 1e9, 2),
            "device_only_gbs": round(kern, 2),
            "device_only_known_branch_gbs": round(nbytes / kq / 1e9, 2),
            "roofline": {"bound": "hbm", "achieved": round(kern, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(kern / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "dvm_vm_vector",
                         "launches_per_step": 2 * len(shapes),
                         "bytes_per_call": "16 B/element (sum pass 4, branch 12)"}}


# ---------------------------------------------------------------------------
# Transformer op stream (streaming fusion of add / RMSNorm / SwiGLU / softmax)
# ---------------------------------------------------------------------------
def stream_bench(args):
    """Steps with seeds 0, 1, ...: each draws its own T, T_kv and 10,000
    motifs.  Value = physical bytes of the flushed graphs (each graph's
    operand tensors read once and stored outputs written once, from the
    library) per second of wall time, capture to final stream sync; motif
    bytes (each motif's own inputs and output) are reported as effective."""
    import torch
    import device_bytecode_vm_amd as dvm
    from device_bytecode_vm_amd import composites as CP
    import workloads as W
    H, F, NH = W.H_LN, W.N_FFN, W.HEADS
    ctx = dvm.Context(0)
    stream = torch.cuda.current_stream()
    bf = dict(dtype="bf16")
    w = W.device_normal((H,), seed=25, mu=1.0, sd=0.1)
    g = dvm.Graph(ctx, stream)
    g.set_stacking(args.stacking, args.stack_order == "temporal")

    def run_step(seed):
        T, TKV, motifs = W.stream_step(seed, args.motifs)
        hs = [W.device_normal((T, H), seed=20, **bf), torch.empty((T, H), dtype=torch.bfloat16, device="cuda")]
        rs = [W.device_normal((T, H), seed=21 + j, **bf) for j in range(4)]
        gs = [W.device_normal((T, F), seed=26 + j, **bf) for j in range(2)]
        us = [W.device_normal((T, F), seed=28 + j, **bf) for j in range(2)]
        ss = [W.device_normal((NH, T, TKV), seed=30 + j, **bf) for j in range(2)]
        n_out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        o_out = torch.empty((T, F), dtype=torch.bfloat16, device="cuda")
        p_out = torch.empty((NH, T, TKV), dtype=torch.bfloat16, device="cuda")
        mb = {"add": 3 * T * H * 2, "rmsnorm": 2 * T * H * 2 + H * 4, "swiglu": 3 * T * F * 2,
              "softmax": 2 * NH * T * TKV * 2}
        torch.cuda.synchronize()
        s0 = g.stats()
        n_log0 = len(g.flush_log())
        t0 = time.perf_counter()
        cur = 0
        vh = g.input(hs[0])
        for kind, j in motifs:
            if kind == "add":
                nxt = 1 - cur
                vh = g.op("add", vh, g.input(rs[j]), out=hs[nxt])
                cur = nxt
            elif kind == "rmsnorm":
                CP.rms_norm(g, vh, g.input(w), W.RMS_EPS, out=n_out)
            elif kind == "swiglu":
                CP.swiglu(g, g.input(gs[j]), g.input(us[j]), out=o_out)
            else:
                CP.softmax(g, g.input(ss[j]), out=p_out)
        g.sync()
        dt = time.perf_counter() - t0
        s1 = g.stats()
        log = g.flush_log(detail=True)[n_log0:]
        return {"T": T, "T_kv": TKV, "dt": dt, "phys": s1["bytes"] - s0["bytes"],
                "motif_bytes": float(sum(mb[k] for k, _ in motifs)), "graphs": s1["graphs"] - s0["graphs"],
                "launches": s1["launches"] - s0["launches"], "ops": s1["ops"] - s0["ops"],
                "stacked": s1["stacked"] - s0["stacked"],
                "fuse_us": s1["fuse_us_total"] - s0["fuse_us_total"],
                "reasons": {k: s1["flush_reason"][k] - s0["flush_reason"][k] for k in s1["flush_reason"]},
                "log": log, "n_motifs": len(motifs)}

    run_step(0)                     # warmup (untimed): library set-up, allocator growth
    runs = [run_step(sd) for sd in range(max(1, args.stream_steps))]
    dt = sum(r["dt"] for r in runs)
    phys = sum(r["phys"] for r in runs)
    eff = sum(r["motif_bytes"] for r in runs)
    log = [e for r in runs for e in r["log"]]
    gbs = phys / dt / 1e9
    n = len(runs)
    return {"metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": n,
            "warmup": 1, "ms_per_step": round(dt / n * 1e3, 3), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "transformer_op_stream", "motifs_per_step": args.motifs,
                       "steps": [{"seed": i, "T": r["T"], "T_kv": r["T_kv"]} for i, r in enumerate(runs)],
                       "hidden": H, "ffn": F, "heads": NH,
                       "bytes": "physical: per flushed graph, its operand tensors read once and its stored "
                                "outputs written once",
                       "timed": "capture, fusion, encode, launch, final stream sync"},
            "effective_gbs": round(eff / dt / 1e9, 2),
            "graphs_per_step": sum(r["graphs"] for r in runs) / n,
            "launches_per_step": sum(r["launches"] for r in runs) / n,
            "graphs_stacked_per_step": sum(r["stacked"] for r in runs) / n, "stacking": args.stacking,
            "stack_order": args.stack_order,
            "ops_per_step": sum(r["ops"] for r in runs) / n,
            "flush_reasons_per_step": {k: sum(r["reasons"][k] for r in runs) / n for k in runs[0]["reasons"]},
            "encode_us": encode_stats(log),
            "fuse_us_per_op": round(sum(r["fuse_us"] for r in runs) / max(sum(r["ops"] for r in runs), 1), 3),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": "dvm_vm_vector + dvm_vm_vector_wide",
                         "timing": "end to end (wall), physical bytes"}}


def brief(res):
    """The fields of a workload's line that the combined line carries."""
    keep = ("value", "unit", "ms_per_step", "steps", "config", "encode_us", "roofline", "device_only_gbs",
            "device_only_known_branch_gbs",
            "device_only_tflops", "kernel_us_warm", "kernel_us_cold", "device_only_gbs_cold", "effective_gbs",
            "graphs_per_step", "launches_per_step", "graphs_stacked_per_step", "stacking", "ops_per_step", "flush_reasons_per_step", "fuse_us_per_op",
            "context", "note", "e2e_host_branch_gbs", "cpu_baseline")
    return {k: res[k] for k in keep if k in res}


def main():
    args = parse()
    if args.traffic_from:
        print(json.dumps(traffic_from(*args.traffic_from)))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build has no multi-GPU "
              "path; the scaling design is described in DESIGN.md", file=sys.stderr)
        sys.exit(2)
    # the CPU baseline runs first, before anything touches the GPU
    cpu = None
    if not args.no_cpu_baseline and not args.calibrate_copy and args.config in ("all", "layernorm"):
        cpu = cpu_baselines(args.cpu_seconds)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    runners = {"layernorm": layernorm_bench, "sqrt_add": sqrt_add_bench, "ifelse": ifelse_bench,
               "matmul": matmul_bench, "stream": stream_bench}
    cpu_key = {"sqrt_add": "sqrt_add", "ifelse": "if_else_add", "matmul": "matmul_bias_silu",
               "stream": "op_stream", "layernorm": "layernorm"}
    if args.config == "all":
        out = layernorm_bench(args)
        out["configs"] = {}
        for name in ("sqrt_add", "ifelse", "matmul", "stream"):
            r = runners[name](args)
            if cpu:
                r["cpu_baseline"] = cpu[cpu_key[name]]
            out["configs"][r["config"]["workload"]] = brief(r)
            torch.cuda.empty_cache()
    else:
        out = runners[args.config](args)
    if cpu and args.config in ("all", "layernorm"):
        out["cpu_baseline"] = dict(cpu["layernorm"], cpu_model=cpu["cpu_model"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
