"""Benchmark of the DVM hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input: for
the LayerNorm stream (the metric's workload) that is 64 LayerNorm calls, each
with a new row count R = B*S (B ~ U{1..32}, S ~ U{1..4096}) over H = 5120,
each captured through the C ABI as a fused group, shape-tiled, encoded to
bytecode on the host and run by the resident VM kernel.  The timed region
includes capture, fusion decisions, encoding and launches; inputs are already
in HBM.  Throughput counts algorithmic bytes: x read and y written (bf16) plus
gamma/beta (fp32) per call.

Prints one JSON line.  --config selects another workload for a separate run
(sqrt_add; ifelse: the reduce-all and host-resolved branch; matmul: the MIX
kernel's MatMul+bias+SiLU, against the matrix-core roofline; stream: the
transformer op stream through the streaming fuser); those lines use the same
fields.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "VM-interpreted fused-op HBM GB/s (% of peak) + bytecode encode µs per graph"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="layernorm", choices=["layernorm", "sqrt_add", "ifelse", "stream", "matmul"])
    ap.add_argument("--calls", type=int, default=0, help="calls per step for ifelse / matmul (0: default)")
    ap.add_argument("--motifs", type=int, default=2000, help="motifs per step for the op stream")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain device copy of known size (counter calibration)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="derive the VM kernel's HBM bytes per launch from rocprofv3 counter files and store them")
    return ap.parse_args()


COPY_BYTES = 512 << 20          # bytes read (and written) by the calibration copy
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_dvm_vm_vector_layernorm_stream.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "device_bytecode_vm_amd", "csrc", f)
                  for f in ("vm_vector.hip", "vm_vector_wide.hip", "bytecode.h")]


def kernel_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per launch measured by counters for the current kernel
    sources, or None when the kernel changed since they were taken."""
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
    big_f = max(cf.values())          # the calibration copy is the largest dispatch
    big_w = max(cw.values())
    f_scale = COPY_BYTES / (big_f * 1024.0)
    w_scale = COPY_BYTES / (big_w * 1024.0)
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
                 "(see the counter commands in "
                 "profiles/README.md)\n" + json.dumps(rec) + "\n")
    return rec


def calibrate_copy():
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": COPY_BYTES}), flush=True)


def pctl(xs, q):
    return float(np.percentile(np.asarray(xs), q)) if len(xs) else 0.0


# ---------------------------------------------------------------------------
# LayerNorm stream
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
    rmax = max(r for r, _ in shapes)
    ybuf = torch.empty((rmax, H), dtype=torch.bfloat16, device="cuda")
    ys = [ybuf[:r] for r, _ in shapes]
    call_bytes = [r * H * 2 * 2 + 2 * H * 4 for r, _ in shapes]
    step_bytes = float(sum(call_bytes))
    torch.cuda.synchronize()

    def one_step(g):
        for x, y in zip(xs, ys):
            CP.layer_norm(g, g.input(x), g.input(gam), g.input(bet), W.LN_EPS, out=y)
        g.flush_launch()

    g = dvm.Graph(ctx, stream)
    for _ in range(args.warmup):
        one_step(g)
    torch.cuda.synchronize()
    s0 = g.stats()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step(g)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    s1 = g.stats()
    ms_step = (t1 - t0) * 1e3 / args.steps
    e2e_gbs = step_bytes * args.steps / (t1 - t0) / 1e9
    graphs = s1["graphs"] - s0["graphs"]
    enc_mean = (s1["encode_us_total"] - s0["encode_us_total"]) / max(graphs, 1)

    # encode latency distribution: encode-only passes (no launch)
    ectx = dvm.Context(-1)
    enc_us = []
    for rep in range(3):
        for x, y in zip(xs, ys):
            ge = dvm.Graph(ectx)
            CP.layer_norm(ge, ge.input(x), ge.input(gam), ge.input(bet), W.LN_EPS, out=y)
            tt0 = time.perf_counter()
            p = ge.flush()
            enc_us.append((time.perf_counter() - tt0) * 1e6)
            del p

    # kernel-only: pre-encoded programs, HIP events on the launch stream
    progs = []
    for x, y in zip(xs, ys):
        gp = dvm.Graph(ctx, stream)
        CP.layer_norm(gp, gp.input(x), gp.input(gam), gp.input(bet), W.LN_EPS, out=y)
        progs.append(gp.flush())
    for p in progs:
        p.launch(stream)
    torch.cuda.synchronize()
    reps = max(1, min(args.steps, 5))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in progs]
    kern_ms = np.zeros(len(progs))
    for _ in range(reps):
        for p, (a, b) in zip(progs, ev):
            a.record(stream)
            p.launch(stream)
            b.record(stream)
        torch.cuda.synchronize()
        kern_ms += np.array([a.elapsed_time(b) for a, b in ev])
    kern_ms /= reps
    kern_gbs = step_bytes / (kern_ms.sum() * 1e-3) / 1e9
    hdr = progs[int(np.argmax([r for r, _ in shapes]))].header()
    tr = stored_traffic()
    traffic = tr["traffic_bytes_per_launch"] if tr else None
    decode = decode_split(progs, stream)

    out = {
        "metric": METRIC, "value": round(e2e_gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "layernorm_stream", "calls_per_step": 64, "hidden": H,
                   "rows": "R=B*S, B~U{1..32}, S~U{1..4096}, seed 0",
                   "rows_total_per_step": int(sum(r for r, _ in shapes)), "eps": W.LN_EPS,
                   "x_dtype": "bf16", "gamma_beta_dtype": "f32", "y_dtype": "bf16"},
        "encode_us": {"p50": round(pctl(enc_us, 50), 2), "p99": round(pctl(enc_us, 99), 2),
                      "max": round(max(enc_us), 2), "mean_in_stream": round(enc_mean, 2)},
        "device_only_gbs": round(kern_gbs, 2),
        "graphs_per_step": graphs / args.steps,
        "roofline": {"bound": "hbm", "achieved": round(kern_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kern_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "dvm_vm_vector_wide + dvm_vm_vector", "launches_per_step": len(progs),
                     "launches_by_kernel": {
                         "dvm_vm_vector_wide": sum(1 for p in progs if p.header()["kernel_type"] == 2),
                         "dvm_vm_vector": sum(1 for p in progs if p.header()["kernel_type"] == 0)},
                     "avg_launch_us": round(float(kern_ms.mean()) * 1e3, 3),
                     "bytes_per_launch_avg": round(step_bytes / len(progs), 1)},
        "largest_call_header": {k: hdr[k] for k in ("block_dim", "body_tile", "grid", "tr", "tc", "g", "nv",
                                                    "n_instr")},
        "decode_split": decode,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = layernorm_cpu_baseline(args.cpu_seconds)
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


def layernorm_cpu_baseline(budget_s):
    """The oracle's LayerNorm (numpy fp64) on a bounded sample of the same
    workload: the first calls of the stream, row-sampled to fit the budget."""
    from oracle import ops as O
    import workloads as W
    shapes = W.layernorm_shapes(0, 64)
    gam, bet = W.layernorm_params()
    H = W.H_LN
    done_rows, t_total, calls = 0, 0.0, 0
    for i, (r, _) in enumerate(shapes):
        rows = min(r, 4096)
        x = W.layernorm_x(0, i, rows, H)
        t0 = time.perf_counter()
        O.layer_norm(x, gam, bet, W.LN_EPS)
        t_total += time.perf_counter() - t0
        done_rows += rows
        calls += 1
        if t_total >= budget_s:
            break
    gbs = done_rows * H * 4 / t_total / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} calls of the LayerNorm stream, first min(R, 4096) rows each "
                      f"({done_rows} rows x 5120), numpy fp64, {t_total:.1f} s"}


# ---------------------------------------------------------------------------
# other workloads (separate runs)
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

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    n = max(args.steps, 1) * 50
    t0 = time.perf_counter()
    for _ in range(n):
        one()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / n
    gp = dvm.Graph(ctx, stream)
    t = gp.op("add", gp.input(a), gp.input(b))
    gp.op("sqrt", t, out=c, live=True)
    gp.release(t)
    p = gp.flush()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(10):
        p.launch(stream)
    e0.record(stream)
    for _ in range(200):
        p.launch(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    kus = e0.elapsed_time(e1) / 200 * 1e3
    # cold: a 512 MiB write between launches evicts the operands from L2 and
    # the MALL; median over the launches
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    for i in range(30):
        scratch.fill_(i & 0xff)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        p.launch(stream)
        c1.record(stream)
        torch.cuda.synchronize()
        cold.append(c0.elapsed_time(c1) * 1e3)
    del scratch
    kus_cold = sorted(cold)[len(cold) // 2]
    return {"metric": METRIC, "value": round(nbytes / dt / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
            "steps": n, "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "sqrt_add", "shape": [513, 1031]},
            "device_only_gbs": round(nbytes / (kus * 1e-6) / 1e9, 2), "kernel_us_warm": round(kus, 3),
            "kernel_us_cold": round(kus_cold, 3),
            "device_only_gbs_cold": round(nbytes / (kus_cold * 1e-6) / 1e9, 2),
            "note": "one 6.3 MB graph is launch-latency bound: 70% of the HBM roofline is out of reach",
            "header": p.header()}


MFMA_PEAK_TFLOPS = 2500.0


def _event_time(stream, fn, reps):
    """Device time per call of fn (seconds), HIP events on `stream`, after one
    untimed call (library set-up, allocator growth)."""
    import torch
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps * 1e-3


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
    g = dvm.Graph(ctx, stream)

    def one_step():
        for m in ms:
            CP.matmul_bias_silu(g, g.input(a[:m]), g.input(b), g.input(bias), out=y[:m])
        g.flush_launch()

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    progs = []
    for m in ms:
        gp = dvm.Graph(ctx, stream)
        CP.matmul_bias_silu(gp, gp.input(a[:m]), gp.input(b), gp.input(bias), out=y[:m])
        progs.append(gp.flush())
    kt = _event_time(stream, lambda: [p.launch(stream) for p in progs], max(1, min(args.steps, 3)))
    tt = _event_time(stream, lambda: [torch.matmul(a[:m], b) for m in ms], max(1, min(args.steps, 3)))
    kern = flops / kt / 1e12
    out = {"metric": "MatMul+bias+SiLU TFLOP/s (MIX VM kernel)", "value": round(flops / dt / 1e12, 2),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(dt * 1e3, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "matmul_bias_silu", "calls_per_step": len(ms), "K": K, "N": N,
                      "M": "distinct M ~ U{1..8192}, seed 0", "rows_total": int(sum(ms))},
           "device_only_tflops": round(kern, 2),
           "roofline": {"bound": "mfma", "achieved": round(kern, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(kern / MFMA_PEAK_TFLOPS, 4), "traffic": None, "kernel": "dvm_vm_mix_128",
                        "launches_per_step": len(ms), "avg_launch_us": round(kt / len(ms) * 1e6, 2)},
           "context": {"torch_matmul_tflops_same_shapes": round(flops / tt / 1e12, 2)}}
    if not args.no_cpu_baseline:
        from oracle import ops as O
        ah = a[:64].float().cpu().numpy().astype(np.float64)
        bh = b.float().cpu().numpy().astype(np.float64)
        biash = bias.cpu().numpy().astype(np.float64)
        rows, t_total = 0, 0.0
        while t_total < args.cpu_seconds and rows < 4096:
            t1 = time.perf_counter()
            O.matmul_bias_silu(ah, bh, biash)
            t_total += time.perf_counter() - t1
            rows += 64
        out["cpu_baseline"] = {"value": round(rows * 2.0 * K * N / t_total / 1e12, 6), "unit": "TFLOP/s",
                               "cores": os.cpu_count(), "kind": "oracle",
                               "sample": f"{rows} rows (64-row blocks) of MatMul+bias+SiLU at K={K}, N={N}, "
                                         f"numpy fp64 (BLAS threads), {t_total:.1f} s"}
    return out


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

    def one_step():
        taken.clear()
        for (r, _), c in zip(shapes, coin):
            x = (xp if c else xn)[:r]
            vx, vy = g.input(x), g.input(yy[:r])
            g.op("reduce_sum", vx, out=s, live=True, axis=0x7FFFFFFF)
            g.flush_launch()
            s_host.copy_(s, non_blocking=True)
            g.sync()
            sv = float(s_host)
            taken.append(sv > 0)
            g.op("add" if sv > 0 else "sub", vx, vy, out=out[:r], live=True)
            g.flush_launch()
        torch.cuda.synchronize()

    for _ in range(args.warmup):
        one_step()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step()
    dt = (time.perf_counter() - t0) / args.steps
    assert taken == [bool(c) for c in coin], "branch differs from the sign the input was drawn with"
    # device-only: the branch is known from the input's sign, so every call's
    # reduce-all (launched when it closes its graph) and branch program are
    # queued back to back with no host sync; one event pair spans them all
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

    kt = _event_time(stream, queued, max(1, min(args.steps, 3)))
    kern = nbytes / kt / 1e9
    res = {"metric": METRIC, "value": round(nbytes / dt / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 3),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": "if_else_add", "calls_per_step": len(shapes), "cols": C,
                      "rows": "N ~ U{1..16384}, seed 0", "branch": "host-resolved after a reduce-all",
                      "add_branch_calls": int(sum(coin))},
           "device_only_gbs": round(kern, 2),
           "roofline": {"bound": "hbm", "achieved": round(kern, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(kern / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "dvm_vm_vector",
                        "launches_per_step": 2 * len(progs), "bytes_per_call": "16 B/element (sum pass 4, branch 12)"}}
    if not args.no_cpu_baseline:
        from oracle import ops as O
        done, t_total = 0, 0.0
        for i, (r, c) in enumerate(shapes):
            rows = min(r, 1024)
            x, y, _ = W.ifelse_inputs(0, i, (rows, c))
            t1 = time.perf_counter()
            O.if_else_add(x, y)
            t_total += time.perf_counter() - t1
            done += rows * c
            if t_total >= args.cpu_seconds:
                break
        res["cpu_baseline"] = {"value": round(done * 16.0 / t_total / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "sample": f"{i + 1} calls, first min(N, 1024) rows each, "
                                                          f"numpy fp64, {t_total:.1f} s"}
    return res


# ---------------------------------------------------------------------------
# Transformer op stream (streaming fusion of add / RMSNorm / SwiGLU / softmax)
# ---------------------------------------------------------------------------
def stream_bench(args):
    import torch
    import device_bytecode_vm_amd as dvm
    from device_bytecode_vm_amd import composites as CP
    import workloads as W
    T, TKV, motifs = W.stream_step(0, args.motifs)
    H, F, NH = W.H_LN, W.N_FFN, 40
    ctx = dvm.Context(0)
    stream = torch.cuda.current_stream()
    bf = dict(dtype="bf16")
    hs = [W.device_normal((T, H), seed=20, **bf), torch.empty((T, H), dtype=torch.bfloat16, device="cuda")]
    rs = [W.device_normal((T, H), seed=21 + j, **bf) for j in range(4)]
    w = W.device_normal((H,), seed=25, mu=1.0, sd=0.1)
    gs = [W.device_normal((T, F), seed=26 + j, **bf) for j in range(2)]
    us = [W.device_normal((T, F), seed=28 + j, **bf) for j in range(2)]
    ss = [W.device_normal((NH, T, TKV), seed=30 + j, **bf) for j in range(2)]
    n_out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    o_out = torch.empty((T, F), dtype=torch.bfloat16, device="cuda")
    p_out = torch.empty((NH, T, TKV), dtype=torch.bfloat16, device="cuda")
    mb = {"add": 3 * T * H * 2, "rmsnorm": 2 * T * H * 2 + H * 4, "swiglu": 3 * T * F * 2,
          "softmax": 2 * NH * T * TKV * 2}
    nbytes = float(sum(mb[k] for k, _ in motifs))
    g = dvm.Graph(ctx, stream)
    state = {"cur": 0}

    def one_step():
        state["cur"] = 0
        vh = g.input(hs[0])
        for kind, j in motifs:
            if kind == "add":
                nxt = 1 - state["cur"]
                vh = g.op("add", vh, g.input(rs[j]), out=hs[nxt])
                state["cur"] = nxt
            elif kind == "rmsnorm":
                CP.rms_norm(g, vh, g.input(w), W.RMS_EPS, out=n_out)
            elif kind == "swiglu":
                CP.swiglu(g, g.input(gs[j]), g.input(us[j]), out=o_out)
            else:
                CP.softmax(g, g.input(ss[j]), out=p_out)
        g.sync()

    for _ in range(args.warmup):
        one_step()
    s0 = g.stats()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    s1 = g.stats()
    graphs = (s1["graphs"] - s0["graphs"]) / args.steps
    reasons = {k: (s1["flush_reason"][k] - s0["flush_reason"][k]) / args.steps for k in s1["flush_reason"]}
    enc = (s1["encode_us_total"] - s0["encode_us_total"]) / max(s1["graphs"] - s0["graphs"], 1)
    gbs = nbytes / dt / 1e9
    res = {"metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 3), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "transformer_op_stream", "motifs_per_step": len(motifs), "T": T, "T_kv": TKV,
                      "hidden": H, "ffn": F, "heads": NH, "bytes": "motif-level: each motif's inputs + output",
                      "timed": "capture, fusion, encode, launch, final stream sync"},
           "graphs_per_step": graphs, "flush_reasons_per_step": reasons, "encode_us_mean": round(enc, 2),
           "encode_us_max": round(s1["encode_us_max"], 2),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "dvm_vm_vector",
                        "note": "end-to-end, motif-level bytes"}}
    if not args.no_cpu_baseline:
        from oracle import ops as O
        rg = W.rng(0)
        done, t_total, k = 0.0, 0.0, 0
        for kind, _ in motifs:
            rows = 64
            t1 = time.perf_counter()
            if kind == "add":
                a1, a2 = rg.normal(size=(rows, H)), rg.normal(size=(rows, H))
                _ = a1 + a2
                done += 3 * rows * H * 2
            elif kind == "rmsnorm":
                O.rms_norm(rg.normal(size=(rows, H)), np.ones(H), W.RMS_EPS)
                done += 2 * rows * H * 2
            elif kind == "swiglu":
                O.swiglu(rg.normal(size=(rows, F)), rg.normal(size=(rows, F)))
                done += 3 * rows * F * 2
            else:
                O.softmax(rg.normal(size=(rows, TKV)))
                done += 2 * rows * TKV * 2
            t_total += time.perf_counter() - t1
            k += 1
            if t_total >= args.cpu_seconds:
                break
        res["cpu_baseline"] = {"value": round(done / t_total / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "sample": f"{k} motifs of the stream on 64-row slices, "
                                                          f"numpy fp64, {t_total:.1f} s"}
    return res


def main():
    args = parse()
    if args.traffic_from:
        print(json.dumps(traffic_from(*args.traffic_from)))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.config == "layernorm":
        out = layernorm_bench(args)
    elif args.config == "sqrt_add":
        out = sqrt_add_bench(args)
    elif args.config == "matmul":
        out = matmul_bench(args)
    elif args.config == "ifelse":
        out = ifelse_bench(args)
    else:
        out = stream_bench(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
