#!/usr/bin/env python3
"""Throughput benchmark of the pipelined GEMM on one MI355X.

Default workload: fp16 GEMM M = N = K = 4096 with fp16 output, 8 rotating
(A, B, C) buffer sets so that consecutive calls do not hit each other's data
in the caches; inputs uniform in [-1, 1) without zeros, seeded.  One "step"
is one GEMM call (the whole hot path) on the next buffer set.

Protocol (the "Xe2 ESIMD GEMM" page, "Performance testing" and "Workflow"):
W untimed warm-up steps, a pause, untimed steps until the clock has come
back from idle (time_steps), then exactly K timed steps (default 1000)
between two device synchronisations.  The kernel time is measured with HIP
events recorded on the stream the kernels are launched on.

The JSON line also carries
* roofline: algorithmic flops (or bytes, for the memory-bound shape) per
  launch over the average launch duration, against MI355X's dense peak;
* cpu_baseline: the CPU oracle timed on a bounded sample (leading rows of
  the same product) on the host cores, scaled to the same unit;
* clocks: amd-smi readings of the shader clock (mean over the XCDs), the
  memory clock and the socket power before the warm-up, while the same
  steps run again after the timed block, and after them (none of it inside
  the timed block; `--no-clocks` skips it).
"""
from __future__ import annotations

import argparse
import json
import os
import shutil
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_F16_TFLOPS = 2516.6     # 256 CU x 2048 fp16 FMA/clk/CU x 2 x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
NOMINAL_GFX_MHZ = 2400           # the shader clock the dense peak above is quoted at

METRIC = "fp16 GEMM TFLOPS at M=N=K=4096 (1 MI355X); % of dense FP16 MFMA peak"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_table() -> dict:
    """The built library's kernels: name -> hash of its machine code and its
    resource use (written by the build beside the library)."""
    path = os.path.join(ROOT, "barrier_pipelined_tiled_amd", "libbpt_gemm.kernels.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        return json.load(f)


def template_code(table: dict, kernel_name: str):
    """Hash over the machine code of every instance of the kernel template a
    profiler's kernel name belongs to (None when the library has none)."""
    from barrier_pipelined_tiled_amd import asm_info
    base = asm_info.base_name(kernel_name)
    if base is None:
        return None
    return asm_info.template_hash({n: k["code"] for n, k in table.items()}, base)


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per step from the committed counter runs (profiles/traffic.json):
    FETCH_SIZE and WRITE_SIZE per dispatch, summed over the kernels of one
    step and scaled by the copy-kernel calibration; None when no run exists
    for this variant, or when the machine code of any kernel it covers
    differs from the built library's (each entry records a hash of the code
    the counters were taken on)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get("entries", {}).get(workload)
    if not e or e.get("variant") != kernel:
        return None
    table = kernel_table()
    for k in e["kernels"]:
        if not k.get("code") or template_code(table, k["name"]) != k["code"]:
            return None
    kib = sum(k["fetch_kib"] * t["fetch_scale"] + k["write_kib"] * t["write_scale"] for k in e["kernels"])
    return int(round(kib * 1024))


def cpu_model() -> str | None:
    """The host CPU's model name, as the kernel reports it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, A, B, budget_s: float = 15.0, min_s: float = 10.0):
    """Time the oracle on the first R rows of A times all of B (set 0), R
    grown until one call takes at least min_s seconds (or covers all rows)."""
    import oracle
    from barrier_pipelined_tiled_amd import inputs
    a_bits = inputs.bits(A if A.dim() == 2 else A[0])
    b_bits = inputs.bits(B if B.dim() == 2 else B[0])
    K, N = b_bits.shape
    rows_all = a_bits.shape[0]
    rows = min(8, rows_all)
    while True:
        t0 = time.perf_counter()
        oracle.gemm(a_bits[:rows], b_bits, w.dtype)
        t = time.perf_counter() - t0
        if t >= min_s or rows == rows_all:
            break
        # small calls overstate the per-row cost (thread start-up), so the
        # estimate is refined by the next, larger call
        rows = int(max(rows + 1, min(rows_all, rows * budget_s / max(t, 1e-3))))
        log(f"cpu_baseline: oracle on {rows} rows ...")
    flops = 2.0 * rows * N * K
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOPS",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"rows 0..{rows - 1} of A ({rows}x{K}) times B ({K}x{N}), "
                  f"{w.dtype}, fp64 accumulation, {t:.1f} s",
    }


def record_traffic(run_dir: str, path: str | None = None) -> None:
    """Write profiles/traffic.json from one measurement run: for every
    workload W with <run_dir>/bench_W.json (its config.kernel names the
    variant), <run_dir>/pmc_fetch_W and <run_dir>/pmc_write_W (rocprofv3
    --pmc FETCH_SIZE / WRITE_SIZE of that bench command), plus the copy
    calibration in <run_dir>/pmc_copy_fetch and pmc_copy_write (the calib
    tool's "copy 256": 256 MiB read and written per dispatch)."""
    import csv
    import glob
    import statistics

    def per_kernel(d):
        f = glob.glob(os.path.join(run_dir, d, "*counter_collection.csv"))
        if len(f) != 1:
            return None
        vals = {}
        with open(f[0]) as fh:
            for r in csv.DictReader(fh):
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: (statistics.mean(v), len(v)) for k, v in vals.items()}

    copy_kib = 256 * 1024
    cf, cw = per_kernel("pmc_copy_fetch"), per_kernel("pmc_copy_write")
    ck = [k for k in cf if k.startswith("copy_kernel")][0]
    fetch_scale = copy_kib / cf[ck][0]
    write_scale = copy_kib / cw[ck][0]
    entries = {}
    table = kernel_table()
    for bj in sorted(glob.glob(os.path.join(run_dir, "bench_*.json"))):
        wname = os.path.basename(bj)[len("bench_"):-len(".json")]
        fe, wr = per_kernel(f"pmc_fetch_{wname}"), per_kernel(f"pmc_write_{wname}")
        if not fe or not wr:
            continue
        with open(bj) as fh:
            variant = json.loads(fh.read().strip().splitlines()[-1])["config"]["kernel"]
        kernels = [{"name": k, "code": template_code(table, k), "dispatches": fe[k][1],
                    "fetch_kib": round(fe[k][0], 2), "write_kib": round(wr[k][0], 2)} for k in fe if k in wr]
        entries[wname] = {"variant": variant, "kernels": kernels}
    out = {
        "_comment": "HBM-side traffic per call from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE "
                    "(KiB per dispatch, mean over the dispatches of a bench run), one entry per "
                    "kernel of the call, scaled by what the same counters read for a plain copy "
                    f"of 256 MiB (FETCH_SIZE {cf[ck][0]:.2f} KiB, WRITE_SIZE {cw[ck][0]:.2f} KiB). "
                    "Written only by bench.py --record-traffic.  An entry is used only while every "
                    "instance of each of its kernels' templates has the machine code it had when the "
                    "counters were taken ('code': hash over the instances' gfx950 code).",
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "entries": entries,
    }
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(f"wrote {path}: {sorted(entries)}")


def parse_smi(text: str) -> dict:
    """Shader clock (mean over the XCDs' gfx clocks), memory clock and socket
    power of GPU 0 from `amd-smi metric -g 0 -c -p --json` output."""
    d = json.loads(text)
    g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
    clk = g.get("clock", {})

    def val(x):
        return x.get("value") if isinstance(x, dict) else None

    gfx = [val(v.get("clk")) for k, v in clk.items() if k.startswith("gfx_") and isinstance(v, dict)]
    gfx = [x for x in gfx if isinstance(x, (int, float))]
    mem = clk.get("mem_0", {})
    return {
        "gfx_mhz": round(sum(gfx) / len(gfx)) if gfx else None,
        "mem_mhz": val(mem.get("clk")) if isinstance(mem, dict) else None,
        "power_w": val(g.get("power", {}).get("socket_power")),
    }


def smi_start():
    """amd-smi started as a child process (the reading runs beside this one)."""
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(exe):
        return None
    try:
        return subprocess.Popen([exe, "metric", "-g", "0", "-c", "-p", "--json"], stdout=subprocess.PIPE,
                                stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None


def smi_finish(proc) -> dict | None:
    if proc is None:
        return None
    try:
        out, _ = proc.communicate(timeout=30)
        return parse_smi(out)
    except Exception as exc:                   # a reading is a report, never a failure
        proc.kill()
        try:
            proc.communicate(timeout=5)
        except Exception:
            pass
        return {"error": str(exc)[:120]}


def clocks_under_load(torch, step, settle_s: float = 2.0, max_s: float = 20.0) -> dict | None:
    """One amd-smi reading taken while the same steps keep the GPU busy: the
    steps run settle_s seconds first (the power reading is an average over a
    window), then on until amd-smi returns."""
    t0 = time.perf_counter()
    i = 0

    def burst():
        nonlocal i
        for _ in range(64):
            step(i)
            i += 1
        torch.cuda.synchronize()

    while time.perf_counter() - t0 < settle_s:
        burst()
    proc = smi_start()
    if proc is None:
        return None
    while proc.poll() is None and time.perf_counter() - t0 < max_s:
        burst()
    r = smi_finish(proc)
    if isinstance(r, dict):
        r["load_s"] = round(time.perf_counter() - t0, 2)
    return r


def time_steps(torch, step, args, stream, unit: int = 1):
    """The timing protocol: W untimed warm-up steps, the pause, the settle
    phase, then K timed steps between two synchronisations (wall clock and
    HIP events on the launch stream); then a per-call spread outside the
    timed block.  step(i) runs `unit` consecutive steps (a replayed graph of
    one pass over the rotating sets with --graph, else one call); K must then
    be a multiple of unit, and every figure is per step.

    The page's pause before timing is there so that the measurement starts
    at the GPU's steady frequency.  On MI355X a pause does the opposite: the
    shader clock drops to idle and needs some 50 ms of load to come back (on
    4096^3: 0.140 ms per call in the first 7 ms after a pause, 0.117 after
    25 ms, 0.1125 from 50 ms on, flat for the following 4 s).  So the pause
    is followed by untimed steps for settle_ms of GPU time before the timed
    block.  The first K steps after the pause are timed too, on their own,
    and reported as after_pause -- they are not the value."""
    if args.steps % unit:
        raise SystemExit(f"--steps must be a multiple of {unit} (one graph replay runs {unit} steps)")
    calls = args.steps // unit
    for i in range(0, args.warmup, unit):
        step(i)
    torch.cuda.synchronize()
    if args.sleep > 0:
        time.sleep(args.sleep)
    i = args.warmup
    settle = None
    if args.settle_ms > 0:
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(calls):
            step(i)
            i += unit
        a1.record(stream)
        torch.cuda.synchronize()
        after_ms = a0.elapsed_time(a1) / args.steps
        n = max(0, (int(args.settle_ms / after_ms) + 1 - args.steps + unit - 1) // unit)
        for _ in range(n):
            step(i)
            i += unit
        torch.cuda.synchronize()
        settle = {"after_pause_ms_per_step": after_ms, "settle_ms": args.settle_ms,
                  "settle_steps": args.steps + n * unit}
        log(f"after the pause: {after_ms:.4f} ms/step over the first {args.steps} steps; "
            f"settled with {args.steps + n * unit} untimed steps")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(calls):
        step(i)
        i += unit
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step wall, {kernel_ms:.4f} ms/launch (events)")
    # per-call spread, after and outside the timed block: each call between
    # its own pair of events on the launch stream
    n_calls = min(50, max(10, calls // 4))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_calls)]
    for a, b in evs:
        a.record(stream)
        step(i)
        i += unit
        b.record(stream)
    torch.cuda.synchronize()
    per_call = sorted(a.elapsed_time(b) / unit for a, b in evs)
    pct = lambda q: per_call[min(len(per_call) - 1, int(q * len(per_call)))]
    spread = {"calls": n_calls, "p10_ms": pct(0.1), "median_ms": pct(0.5), "p90_ms": pct(0.9)}
    if unit > 1:
        spread["steps_per_call"] = unit
    return ms_per_step, kernel_ms, spread, settle


def capture_pass(torch, step, steps: int, stream):
    """One HIP graph holding `steps` consecutive steps (whole passes over the
    rotating input sets, each step the same library call as without a
    graph), captured on `stream` after one eager run of them; replay() runs
    them again."""
    for j in range(steps):
        step(j)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for j in range(steps):
            step(j)
    torch.cuda.synchronize()
    return g


def roofline(flops, compulsory_bytes, kernel_ms):
    """The bound: HBM when the flops per compulsory byte fall below the
    machine balance (2516.6 TFLOP/s / 8 TB/s = 315 flop/B; the batched
    short-K GEMM (228, its fp16 C writes) and the skinny GEMM (63) are),
    else the matrix cores.  achieved = algorithmic work per launch over the
    average launch duration."""
    if flops / compulsory_bytes < PEAK_MFMA_F16_TFLOPS / PEAK_HBM_GBS * 1e3:
        achieved = compulsory_bytes / (kernel_ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": None}
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_F16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_MFMA_F16_TFLOPS, "traffic": None}


def gemm_setup(torch, pkg, inputs, args, dev):
    """GEMM workload: rotating (A, B, C) sets resident in HBM, the step, the
    config and the oracle baseline."""
    w = inputs.WORKLOADS[args.workload]
    R = w.rotating
    log(f"workload {w.name}: batch={w.batch} M={w.M} N={w.N} K={w.K} {w.dtype} "
        f"out={'fp32' if w.out_fp32 else w.dtype} rotating={R}")
    As, Bs, Cs = [], [], []
    A0 = B0 = None
    nt = args.b_layout == "nt"
    for j in range(R):
        A = w.make_a(j) if (w.rotate_a or j == 0) else None
        B = w.make_b(j)
        if j == 0:
            A0, B0 = A, B
        As.append(A.to(dev) if A is not None else As[0])
        Bd = B.to(dev)
        Bs.append(Bd.transpose(-1, -2).contiguous() if nt else Bd)
        out_t = torch.float32 if w.out_fp32 else (torch.float16 if w.dtype == "f16" else torch.bfloat16)
        Cs.append(torch.empty(w.c_shape(), dtype=out_t, device=dev))
    stream = torch.cuda.current_stream()
    # under graph capture the split paths keep their splits only through the
    # entry point that allocates nothing (its scratch is a fixed device array)
    gemm = pkg.gemm_ex_bt if nt else (pkg.gemm_ex_noalloc if args.graph else pkg.gemm_ex)

    def step(i):
        j = i % R
        gemm(As[j], Bs[j], Cs[j], dtype=w.dtype, out_fp32=w.out_fp32, variant=args.variant, stream=stream)

    variant_id = args.variant or pkg.select_variant(w.dtype, w.batch, w.M, w.N, w.K, w.K, w.K if nt else w.N,
                                                    w.out_fp32, bt=nt)
    names = {v: k for k, v in pkg.variants().items()}
    kernel = names.get(variant_id, str(variant_id))
    metric = (METRIC if w.name == "f16_4096" and not nt else
              f"{w.name}{' with B given transposed (N x K)' if nt else ''} TFLOPS (1 MI355X)")
    config = {"workload": w.name, "batch": w.batch, "M": w.M, "N": w.N, "K": w.K,
              "in": w.dtype, "out": "fp32" if w.out_fp32 else w.dtype, "accumulate": "fp32",
              "rotating_buffers": R, "kernel": kernel, "b_layout": "N x K (transposed)" if nt else "K x N"}
    return (w, step, stream, metric, config, kernel, lambda: cpu_baseline(w, A0, B0))


def attention_cpu_baseline(w, q, k, v, budget_s: float = 15.0, min_s: float = 10.0):
    """Time the oracle on the first R query rows (head by head, each against
    all keys of its head), R grown until one call takes at least min_s
    seconds (or covers every row)."""
    import numpy as np
    import oracle
    from barrier_pipelined_tiled_amd import inputs
    qb, kb, vb = inputs.bits(q), inputs.bits(k), inputs.bits(v)
    total = w.BH * w.Sq
    rows = 16
    while True:
        t_idx = np.arange(rows, dtype=np.int64)
        idx = (t_idx // w.Sq, t_idx % w.Sq)
        t0 = time.perf_counter()
        oracle.attention(qb, kb, vb, w.scale, w.dtype, rows=idx)
        t = time.perf_counter() - t0
        if t >= min_s or rows == total:
            break
        rows = int(max(rows + 1, min(total, rows * budget_s / max(t, 1e-3))))
        log(f"cpu_baseline: attention oracle on {rows} query rows ...")
    flops = 4.0 * rows * w.Skv * w.D
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOPS",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"the first {rows} query rows (heads 0..{(rows - 1) // w.Sq}), each against the "
                  f"{w.Skv} keys of its head, D = {w.D}, {w.dtype}, fp64, {t:.1f} s",
    }


def attention_setup(torch, pkg, inputs, args, dev):
    w = inputs.ATTENTION[args.workload]
    R = w.rotating
    log(f"workload {w.name}: BH={w.BH} Sq={w.Sq} Skv={w.Skv} D={w.D} {w.dtype} rotating={R}")
    sets = []
    q0 = k0 = v0 = None
    for j in range(R):
        q, k, v = w.make_q(j), w.make_k(j), w.make_v(j)
        if j == 0:
            q0, k0, v0 = q, k, v
        out_t = torch.float32 if w.out_fp32 else (torch.float16 if w.dtype == "f16" else torch.bfloat16)
        sets.append((q.to(dev), k.to(dev), v.to(dev), torch.empty(q.shape, dtype=out_t, device=dev)))
    stream = torch.cuda.current_stream()

    def step(i):
        q, k, v, o = sets[i % R]
        pkg.attention_fwd(q, k, v, o, scale=w.scale, dtype=w.dtype, out_fp32=w.out_fp32, stream=stream)

    kernel = f"attention_fwd_d{w.D}"
    metric = f"{w.name} TFLOPS (1 MI355X): fused attention forward, 4 * BH * Sq * Skv * D flops"
    config = {"workload": w.name, "batch_heads": w.BH, "seq_q": w.Sq, "seq_kv": w.Skv, "head_dim": w.D,
              "in": w.dtype, "out": "fp32" if w.out_fp32 else w.dtype, "accumulate": "fp32",
              "scale": w.scale, "rotating_buffers": R, "kernel": kernel}
    return (w, step, stream, metric, config, kernel, lambda: attention_cpu_baseline(w, q0, k0, v0))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 1000 timed calls, the page's preferred count for compute-bound kernels
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="f16_4096",
                    help="a GEMM workload (f16_4096, ...) or an attention one (attn_f16_...)")
    ap.add_argument("--variant", type=int, default=0, help="GEMM variant, 0 = automatic choice")
    ap.add_argument("--sleep", type=float, default=5.0, help="pause before timing (s)")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed steps after the pause, in ms of GPU time, so that the timed block "
                         "starts at the steady clock (0: none; the first --steps steps after the "
                         "pause are then the timed block)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads for the oracle's CPU baseline (0: all the host offers)")
    ap.add_argument("--no-clocks", action="store_true", help="skip the amd-smi clock and power readings")
    ap.add_argument("--b-layout", choices=["kn", "nt"], default="kn",
                    help="GEMM only.  kn: B is K x N (the workloads' layout); nt: the same B handed "
                         "over transposed (N x K) through gemm_ex_bt")
    ap.add_argument("--graph", type=int, nargs="?", const=1, default=0, metavar="PASSES",
                    help="capture PASSES passes over the rotating input sets (default 1) into one HIP "
                         "graph and time its replays: each replay runs PASSES x rotating steps (for "
                         "launch-bound shapes; --steps must be a multiple of that)")
    ap.add_argument("--record-traffic", metavar="RUN_DIR",
                    help="write profiles/traffic.json from the counter runs in RUN_DIR and exit")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.record_traffic)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the GEMM of this library runs on a single "
              "MI355X and has no multi-GPU path (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import barrier_pipelined_tiled_amd as pkg
    from barrier_pipelined_tiled_amd import inputs

    dev = torch.device("cuda:0")
    pkg.lib()
    if args.graph:
        # capture needs a stream other than the legacy default one; the whole
        # run uses it (default priority)
        torch.cuda.set_stream(torch.cuda.Stream())
    if args.workload in inputs.ATTENTION:
        setup = attention_setup
    elif args.workload in inputs.WORKLOADS:
        setup = gemm_setup
    else:
        print(f"unknown workload {args.workload}; GEMM: {sorted(inputs.WORKLOADS)}, "
              f"attention: {sorted(inputs.ATTENTION)}", file=sys.stderr)
        sys.exit(2)
    w, step, stream, metric, config, kernel, baseline = setup(torch, pkg, inputs, args, dev)
    torch.cuda.synchronize()
    log("inputs resident in HBM")

    unit = 1
    if args.graph:
        unit = args.graph * w.rotating
        graph = capture_pass(torch, step, unit, stream)
        step = lambda i: graph.replay()
        config["graph_steps_per_replay"] = unit
        log(f"captured {args.graph} pass(es) over the {w.rotating} rotating sets ({unit} steps) into a graph")
    clk_before = None if args.no_clocks else smi_finish(smi_start())
    ms_per_step, kernel_ms, spread, settle = time_steps(torch, step, args, stream, unit)
    clocks = None
    if not args.no_clocks:
        clocks = {"nominal_gfx_mhz": NOMINAL_GFX_MHZ, "before": clk_before,
                  "under_load": clocks_under_load(torch, step), "after": smi_finish(smi_start())}
    value = w.flops / (ms_per_step * 1e-3) / 1e12
    roof = roofline(w.flops, w.compulsory_bytes, kernel_ms)
    roof["traffic"] = measured_traffic(w.name, kernel)
    config["pct_of_dense_peak"] = 100.0 * value / PEAK_MFMA_F16_TFLOPS
    if args.cpu_threads > 0 and not args.no_cpu_baseline:
        import oracle
        oracle.set_num_threads(args.cpu_threads)
    cpu = None if args.no_cpu_baseline else baseline()

    out = {
        "metric": metric,
        "value": value,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if w.dtype == "f16" else "bf16",
        "data": "synthetic",
        "config": config,
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_call": spread,
        "settle": settle,
        "clocks": clocks,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
