#!/usr/bin/env python3
"""Benchmark of the W4A8 block-quantized matmul hot path on one MI355X.

Headline (the `value` of the JSON line): decode GEMV weight GB/s on the
4096 x 4096 Q4_0 decode workload (M = 1, float32 activations with 1% outliers
x20). One step is one pass of the decode hot path over one activation vector:
per-block int8 quantization of x, the exact per-block int8 dots against the
packed 4-bit weights, the per-block float rescale and the wavefront reduce,
all in one fused launch (q4_gemv_fused). Steps rotate through 100 copies of
the weights (944 MB, well above the 256 MB last-level cache), so every step
streams its weights from HBM; the steps are replayed from HIP graphs.

Protocol: W warm-up steps; every graph that the timed region replays is
replayed once before it. Exactly K steps are then timed with HIP events on
the launch stream: graphs of 1000 steps for every full thousand, the rest as
plain launches of the entry point. Untimed warm replays are queued just
before the first event, so the GPU stays busy while the host queues the timed
work and the events see the K steps back to back (`value`, `ms_per_step`); a
second, synchronize-bracketed pass gives the host's wall time for the same K
steps (`wall_ms_per_step`).

Before a variant is timed its output is checked against the oracle's values
at sampled coordinates (tests/golden/bench_gate.json, written by
tests/golden/make_bench_gate.py); a variant that disagrees is not timed.

The line also carries:
  floors        an empty kernel and a read-only stream of the same weight
                bytes, measured in the same process (the ceiling the decode
                kernel is compared against), and the observed GPU clocks;
  secondary     the prefill GEMM int8 TOPS (the second half of the metric) on
                the affine g128 4096-row workloads and the other workloads;
  cpu_baseline  the C oracle timed on the host's cores (1 thread and all
                threads of this process's CPU share) on bounded samples.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary]
       python bench.py --summarize-trace <rocprofv3 kernel_trace.csv>   (no GPU)
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import platform
import re
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode GEMV weight GB/s (%HBM peak); prefill GEMM int8 TOPS (%MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 (vector and matrix)
PEAK_SCLK_MHZ = 2400.0
GRAPH_STEPS = 100              # rotating weight copies (944 MB of decode weights)
BULK_STEPS = 1000              # steps per captured graph in the headline's timed region
PROFILES = os.path.join(ROOT, "profiles")
GATE_PATH = os.path.join(ROOT, "tests", "golden", "bench_gate.json")
GATE_TOL = 1e-5                # relative RMS over the sampled outputs


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--no-secondary", action="store_true", help="headline decode line only")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-floors", action="store_true")
    p.add_argument("--only", default=None,
                   help="run one workload alone (for profiling): gemv_fused (eager decode launches, --steps of "
                        "them), floors, gemm_3a, gemm_3b, gemm_2, gemm_0, q4k_gemv, q4k_gemm, gemv_plain, small_m, "
                        "q4k_backward, q4_backward, gemm_bits")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="run a plain device-to-device copy of this many MiB (counter calibration) and exit")
    p.add_argument("--summarize-trace", default=None,
                   help="print per-kernel statistics (calls, mean, median, min, max) of a rocprofv3 kernel-trace "
                        "CSV as a markdown table and exit (no GPU needed)")
    return p.parse_args()


# ------------------------------------------------------------------ trace summaries

def summarize_trace(path: str) -> str:
    """Per-kernel duration statistics of a rocprofv3 --kernel-trace CSV."""
    durs = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("KernelName") or row.get("Name")
            d = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
            durs.setdefault(name, []).append(d)
    total = sum(sum(v) for v in durs.values()) or 1
    lines = ["| Kernel | Calls | Mean ns | Median ns | Min ns | Max ns | % of GPU time |", "|---|---|---|---|---|---|---|"]
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        short = name if len(name) <= 110 else name[:107] + "..."
        lines.append(f"| `{short}` | {len(v)} | {statistics.mean(v):.0f} | {statistics.median(v):.0f} | {min(v)} | "
                     f"{max(v)} | {100.0 * sum(v) / total:.2f} |")
    return "\n".join(lines)


# ------------------------------------------------------------------ counters

def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        for f in (os.path.join(ROOT, "block_quantized_bit_amd", "csrc", n),
                  os.path.join(ROOT, "block_quantized_bit_amd", "csrc", "common.h")):
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(name: str, src_hash: str):
    """HBM bytes per launch from a committed counter summary, or None when the
    summary is missing or was taken on a different kernel source."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != src_hash:
        return None
    try:
        fetch = float(vals["fetch_kib_per_dispatch"]) * 1024 * float(vals["fetch_scale"])
        write = float(vals["write_kib_per_dispatch"]) * 1024 * float(vals["write_scale"])
    except (KeyError, ValueError):
        return None
    return fetch + write


# ------------------------------------------------------------------ host facts

def host_cpu():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        share = len(os.sched_getaffinity(0))
    except AttributeError:
        share = os.cpu_count() or 1
    return model, os.cpu_count() or 1, share


def sample_clocks():
    """Current GPU clocks in MHz from rocm-smi (read-only query), or {} if unavailable."""
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        data = json.loads(r.stdout)
    except Exception:  # noqa: BLE001 -- a missing or failing query only drops the clock fields
        return {}
    out = {}
    for card in data.values():
        if not isinstance(card, dict):
            continue
        for k, v in card.items():
            m = re.search(r"(\d+(?:\.\d+)?)\s*Mhz", str(v), flags=re.I)
            key = k.lower()
            for clk in ("sclk", "mclk", "fclk", "socclk"):
                if clk in key and m and clk not in out:
                    out[clk] = float(m.group(1))
        break
    return out


# ------------------------------------------------------------------ main

def main():
    args = parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_quantized_bit_amd as q4
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        a = torch.ones(n // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}))
        return

    gate_doc = json.load(open(GATE_PATH)) if os.path.exists(GATE_PATH) else {"cases": {}}

    def gate(key, y, extra_ok=True, extra=None):
        """Sampled outputs of y against the oracle's stored values; {'ok': bool, ...}."""
        c = gate_doc["cases"].get(key)
        if c is None:
            return {"ok": False, "reason": f"no stored oracle values for {key}"}
        ms = torch.tensor(c["ms"], dtype=torch.long, device=y.device)
        ns = torch.tensor(c["ns"], dtype=torch.long, device=y.device)
        got = y[ms, ns].double().cpu().numpy()
        ref = np.array(c["y_bits"], dtype=np.uint32).view(np.float32).astype(np.float64)
        rel = float(np.sqrt(((got - ref) ** 2).sum()) / max(np.sqrt((ref ** 2).sum()), 1e-300))
        ok = bool(np.isfinite(got).all() and rel <= GATE_TOL and extra_ok)
        out = {"ok": ok, "rel_rms": float(f"{rel:.3g}"), "samples": len(c["ms"])}
        if extra:
            out.update(extra)
        return out

    def graph_of(fn, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                fn(i)
        return g

    def event_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def time_replays(g, reps, spacer=None):
        """Seconds per replay of g over reps replays, by events; with a spacer graph queued just before the
        first event the GPU never waits for the host between the events."""
        e0, e1 = event_pair()
        torch.cuda.synchronize()
        if spacer is not None:
            spacer.replay()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    # ------------------------------------------------------------ decode (headline)
    wl = synth.workload("q4_0_decode_4096")
    weight_bytes = wl.N * wl.K // 2 + wl.N * (wl.K // 32) * 2
    x = torch.from_numpy(synth.gen.activations(wl)).to(dev)
    w = torch.from_numpy(synth.gen.weights(wl)).to(dev)
    wq, wd, _ = q4.quantize_weights(w, "q4_0", 32)          # model preparation on the GPU, untimed
    del w
    copies = [(wq.clone(), wd.clone()) for _ in range(GRAPH_STEPS)]
    y = torch.empty((1, wl.N), dtype=torch.float32, device=dev)

    def decode_step(i):
        c = copies[i % GRAPH_STEPS]
        q4.gemv_fused("q4_0", 32, x, c[0], c[1], None, y=y)

    result = {}
    if args.only == "gemv_fused":
        # eager launches over the cold copies, for counter collection (one dispatch per step)
        for i in range(args.steps):
            decode_step(i)
        torch.cuda.synchronize()
        print(json.dumps({"only": "gemv_fused", "launches": args.steps}), flush=True)
        return

    floors = {}
    if args.only is None:
        # agreement gate: the fused step's output and the activation codes it used
        act = (torch.empty((1, wl.K), dtype=torch.int8, device=dev),
               torch.empty((1, wl.K // 32), dtype=torch.float32, device=dev),
               torch.empty((1, wl.K // 32), dtype=torch.int32, device=dev))
        y.fill_(float("nan"))
        q4.gemv_fused("q4_0", 32, x, copies[0][0], copies[0][1], None, y=y, act_out=act)
        torch.cuda.synchronize()
        c = gate_doc["cases"].get("q4_0_decode_4096", {})
        codes_ok = (hashlib.sha256(act[0].cpu().numpy().tobytes()).hexdigest() == c.get("xq_sha256")
                    and act[1].cpu().numpy().view(np.uint32).reshape(-1).tolist() == c.get("xs_bits")
                    and act[2].cpu().numpy().reshape(-1).tolist() == c.get("xsum"))
        g_head = gate("q4_0_decode_4096", y, codes_ok, {"codes_bit_exact": bool(codes_ok)})
        if not g_head["ok"]:
            print(json.dumps({"metric": METRIC, "value": None, "unit": "GB/s", "error": "agreement gate failed: "
                              "the decode kernel disagrees with the oracle, not timed", "gate": g_head}), flush=True)
            sys.exit(1)

        for i in range(min(args.warmup, GRAPH_STEPS)):
            decode_step(i)
        torch.cuda.synchronize()
        # the timed steps: graphs of BULK_STEPS (every full thousand), then the remainder as plain launches of
        # the entry point; step i uses weight copy i % 100, so every step reads weights last read 99 steps
        # earlier (944 MB back), out of cache
        g_warm = graph_of(decode_step, GRAPH_STEPS)
        reps, rem = divmod(args.steps, BULK_STEPS)
        g_bulk = graph_of(decode_step, BULK_STEPS) if reps else None
        for _ in range(max(1, args.warmup // GRAPH_STEPS)):
            g_warm.replay()
        if g_bulk is not None:
            g_bulk.replay()
        torch.cuda.synchronize()
        # one graph replay costs a few microseconds of GPU time beyond its kernels, and plain launches are
        # host-bound unless queued behind work; so untimed warm replays are queued first (enough to cover the
        # host's queuing of the remainder), and the events bracket exactly the K steps, back to back
        spacers = 1 + rem // 50

        def timed_steps():
            for _ in range(reps):
                g_bulk.replay()
            for i in range(rem):
                decode_step(reps * BULK_STEPS + i)

        e0, e1 = event_pair()
        torch.cuda.synchronize()
        for _ in range(spacers):
            g_warm.replay()
        e0.record()
        timed_steps()
        e1.record()
        torch.cuda.synchronize()
        kern_s = e0.elapsed_time(e1) / 1e3 / args.steps
        # timed, wall clock: the same K steps bracketed by synchronizations (host launch latency included)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        timed_steps()
        torch.cuda.synchronize()
        wall_s = (time.perf_counter() - t0) / args.steps

        value = weight_bytes / kern_s / 1e9
        src_hash = kernel_source_hash(["gemv.hip"])
        traffic = read_traffic("gemv_fused_q4_0_decode_4096_counters.txt", src_hash)
        result = {
            "metric": METRIC,
            "value": round(value, 1),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(kern_s * 1e3, 6),
            "wall_ms_per_step": round(wall_s * 1e3, 6),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "int8",
            "data": "synthetic (seeded SplitMix64: N(0,0.02^2) weights quantized to Q4_0 on the GPU; "
                    "N(0,1) f32 activations, 1% of entries x20)",
            "config": {
                "workload": "q4_0_decode_4096: W4A8 decode GEMV, M=1, K=N=4096, Q4_0 (32-weight blocks, fp16 "
                            "scale), f32 activations quantized per 32-block to int8 inside the kernel",
                "M": 1, "K": wl.K, "N": wl.N, "format": "q4_0", "block": 32,
                "weight_bytes_per_step": weight_bytes,
                "cold_weight_copies": GRAPH_STEPS,
                "launch": "q4_gemv_fused, one launch per step (graphs of 1000 steps, the remainder launched "
                          "directly); value from HIP events over exactly the timed steps",
            },
            "gate": g_head,
            "roofline": {
                "bound": "hbm",
                "achieved": round(value, 1),
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": round(value / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "kernel": "q4::gemv_kernel (fused quantize + GEMV)",
                "kernel_avg_us": round(kern_s * 1e6, 3),
                "algorithmic_bytes_per_launch": weight_bytes,
            },
        }

    # ------------------------------------------------------------ floors
    if (args.only is None and not args.no_floors) or args.only == "floors":
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        shapes = [(256, 1024), (512, 1024), (1024, 1024), (1024, 512), (2048, 256), (4096, 256)]

        def stream_ceiling(nbytes, ncopies):
            bufs = [torch.full((nbytes,), 0x5A, dtype=torch.uint8, device=dev) for _ in range(ncopies)]
            best = None
            per_shape = {}
            for grid, block in shapes:
                def rd(i, grid=grid, block=block):
                    q4.measure_stream_read(bufs[i % ncopies], grid, block, sink)
                rd(0)
                g = graph_of(rd, ncopies)
                g.replay()
                t = time_replays(g, 10, spacer=g) / ncopies
                per_shape[f"{grid}x{block}"] = round(t * 1e6, 3)
                if best is None or t < best[0]:
                    best = (t, grid, block)
            del bufs
            return {"bytes": nbytes, "cold_copies": ncopies, "us": round(best[0] * 1e6, 3),
                    "GB/s": round(nbytes / best[0] / 1e9, 1), "frac_hbm": round(nbytes / best[0] / 1e9 / HBM_PEAK_GBS, 4),
                    "launch": f"{best[1]}x{best[2]}", "us_by_launch": per_shape}

        def empty_floor(grid, block):
            def ek(i):
                q4.measure_empty(grid, block)
            ek(0)
            g = graph_of(ek, GRAPH_STEPS)
            g.replay()
            return round(time_replays(g, 10, spacer=g) / GRAPH_STEPS * 1e6, 3)

        floors["empty_kernel_us"] = {"256x1024": empty_floor(256, 1024), "1792x256": empty_floor(1792, 256)}
        floors["stream_read_decode_weights"] = stream_ceiling(weight_bytes, GRAPH_STEPS)
        floors["stream_read_q4k_weights"] = stream_ceiling(14336 * 16 * 144, 32)
        clk = {}
        # clocks sampled while the GPU streams (a query from another thread during a busy loop)
        big = torch.full((1 << 30,), 1, dtype=torch.uint8, device=dev)
        th = threading.Thread(target=lambda: clk.update(sample_clocks()))
        th.start()
        t_end = time.perf_counter() + 30.0
        while th.is_alive() and time.perf_counter() < t_end:
            for _ in range(20):
                q4.measure_stream_read(big, 2048, 256, sink)
            torch.cuda.synchronize()
        th.join(timeout=30)
        del big
        floors["clocks_mhz_under_load"] = clk or None
        if result:
            ceil = floors["stream_read_decode_weights"]["GB/s"]
            result["roofline"]["frac_of_measured_stream"] = round(result["value"] / ceil, 4)
            result["roofline"]["measured_stream_GB/s"] = ceil
        if args.only == "floors":
            print(json.dumps({"floors": floors}), flush=True)
            return
    if floors:
        result["floors"] = floors

    # ------------------------------------------------------------ secondary
    secondary = {}
    want = (lambda k: args.only == k) if args.only else (lambda k: not args.no_secondary)

    def graphed_rotating(fn, ncop, reps=10):
        fn(0)
        g = graph_of(fn, ncop)
        g.replay()
        return time_replays(g, reps, spacer=g) / ncop

    if want("gemv_plain"):
        xq, xs, xsum = q4.quantize_act(x, 32)

        def plain(i):
            c = copies[i % GRAPH_STEPS]
            q4.gemv("q4_0", 32, c[0], c[1], None, xq, xs, xsum, y=y)
        y.fill_(float("nan"))
        plain(0)
        torch.cuda.synchronize()
        gt = gate("q4_0_decode_4096", y)
        entry = {"what": "q4_gemv (activation codes given), cold weights, HIP graph", "gate": gt}
        if gt["ok"]:
            t = graphed_rotating(plain, GRAPH_STEPS)
            entry.update({"us": round(t * 1e6, 3), "GB/s": round(weight_bytes / t / 1e9, 1),
                          "frac_hbm": round(weight_bytes / t / 1e9 / HBM_PEAK_GBS, 4)})
        secondary["gemv_plain_q4_0_decode_4096"] = entry

    if want("small_m"):
        # few-row decode: M rows of decode-like activations against the same cold weight copies
        rows = {}
        for M in (2, 4, 6, 8, 16, 32):
            xm = torch.from_numpy(synth.gen.activations(wl, M=M)).to(dev)
            xq_m, xs_m, xsum_m = q4.quantize_act(xm, 32)
            y_m = torch.full((M, wl.N), float("nan"), dtype=torch.float32, device=dev)

            def few(i, xq_m=xq_m, xs_m=xs_m, xsum_m=xsum_m, y_m=y_m):
                c = copies[i % GRAPH_STEPS]
                q4.gemm("q4_0", 32, c[0], c[1], None, xq_m, xs_m, xsum_m, y=y_m)
            few(0)
            torch.cuda.synchronize()
            gt = gate(f"q4_0_rows_{M}x4096x4096", y_m)
            r = {"gate": gt}
            if gt["ok"]:
                t = graphed_rotating(few, GRAPH_STEPS)
                r.update({"us": round(t * 1e6, 3), "GB/s": round(weight_bytes / t / 1e9, 1),
                          "frac_hbm": round(weight_bytes / t / 1e9 / HBM_PEAK_GBS, 4),
                          "TOPS": round(2.0 * M * wl.K * wl.N / t / 1e12, 2)})
            rows[str(M)] = r
        secondary["small_m_q4_0_rows_x4096x4096"] = {
            "what": "q4_gemm with M rows (few-row kernels: each weight block read once for all rows), cold weights, "
                    "HIP graph; activation codes given", "by_M": rows}

    del copies

    def time_graphed(fn, iters, warm=3, reps=3):
        # iters calls captured in one HIP graph and replayed reps times, so that
        # the host's launch rate does not enter the per-call time of short kernels
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(iters):
                fn()
        g.replay()
        return time_replays(g, reps, spacer=g) / iters

    gemm_cases = [("gemm_3a", "affine_g128_4096x4096x14336", 20), ("gemm_3b", "affine_g128_4096x14336x4096", 20),
                  ("gemm_2", "affine_g64_1024x4096x4096", 50), ("gemm_0", "q4_0_minilm_64x384x1536", 200)]
    for key, name, iters in gemm_cases:
        if not want(key):
            continue
        g = synth.workload(name)
        gx = synth.gen.activations(g)
        gw = synth.gen.weights(g)
        if g.xdtype == "bf16":
            xt = torch.from_numpy(gx.view(np.int16)).to(dev).view(torch.bfloat16)
            wt = torch.from_numpy(gw.view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            xt = torch.from_numpy(gx).to(dev)
            wt = torch.from_numpy(gw).to(dev)
        gwq, gws, gwb = q4.quantize_weights(wt, g.fmt, g.bs)
        del wt
        xq, xs, xsum = q4.quantize_act(xt, g.bs)
        yy = torch.full((g.M, g.N), float("nan"), dtype=torch.float32, device=dev)
        q4.gemm(g.fmt, g.bs, gwq, gws, gwb, xq, xs, xsum, y=yy)
        torch.cuda.synchronize()
        ops = 2.0 * g.M * g.N * g.K
        entry = {"gate": gate(name, yy)}
        if entry["gate"]["ok"]:
            t_gemm = time_graphed(lambda: q4.gemm(g.fmt, g.bs, gwq, gws, gwb, xq, xs, xsum, y=yy), iters)
            t_act = time_graphed(lambda: q4.quantize_act(xt, g.bs, out=(xq, xs, xsum)), iters)
            act_bytes = xt.numel() * xt.element_size() + xq.numel() + 8 * xs.numel()
            entry.update({
                "gemm_us": round(t_gemm * 1e6, 2), "gemm_TOPS": round(ops / t_gemm / 1e12, 1),
                "gemm_frac_int8_peak": round(ops / t_gemm / 1e12 / INT8_PEAK_TOPS, 4),
                "act_quant_us": round(t_act * 1e6, 2), "act_quant_GB/s": round(act_bytes / t_act / 1e9, 1),
                "step_TOPS": round(ops / (t_gemm + t_act) / 1e12, 1)})
        if g.M > 32:
            # pre-packed weights, fused quantize + GEMM (two launches, group-major activation scales)
            packed = q4.pack_weights(g.fmt, g.bs, gwq, gws, gwb)
            work = torch.empty(int(q4.lib().q4_gemm_packed_work_bytes(g.M, g.K, g.bs)), dtype=torch.uint8,
                               device=dev)
            yy.fill_(float("nan"))
            q4.gemm_packed(g.fmt, g.bs, xt, packed, g.N, y=yy, work=work)
            torch.cuda.synchronize()
            gp = gate(name, yy)
            entry["packed_gate"] = gp
            if gp["ok"]:
                t_pk = time_graphed(lambda: q4.gemm_packed(g.fmt, g.bs, xt, packed, g.N, y=yy, work=work), iters)
                entry.update({"packed_step_us": round(t_pk * 1e6, 2),
                              "packed_step_TOPS": round(ops / t_pk / 1e12, 1)})
                if "act_quant_us" in entry:
                    t_pg = t_pk - entry["act_quant_us"] * 1e-6
                    entry.update({"packed_gemm_us_est": round(t_pg * 1e6, 2),
                                  "packed_gemm_frac_int8_peak_est": round(ops / t_pg / 1e12 / INT8_PEAK_TOPS, 4)})
            del packed, work
        secondary[f"prefill_{name}"] = entry
        del gwq, gws, gwb, xq, xs, xsum, yy, xt

    if want("gemm_bits"):
        # affine 4-, 6- and 8-bit codes on the same int8-MFMA GEMM (two workload shapes, activation codes given)
        out = {}
        for name in ("affine_g64_1024x4096x4096", "affine_g128_4096x4096x14336"):
            g = synth.workload(name)
            xt = torch.from_numpy(synth.gen.activations(g).view(np.int16)).to(dev).view(torch.bfloat16)
            wt = torch.from_numpy(synth.gen.weights(g).view(np.int16)).to(dev).view(torch.bfloat16)
            xq, xs, xsum = q4.quantize_act(xt, g.bs)
            yy = torch.empty((g.M, g.N), dtype=torch.float32, device=dev)
            ops = 2.0 * g.M * g.N * g.K
            for bits in (4, 6, 8):
                gwq, gws, gwb = q4.quantize_weights(wt, "affine", g.bs, bits=bits)
                yy.fill_(float("nan"))
                q4.gemm("affine", g.bs, gwq, gws, gwb, xq, xs, xsum, y=yy, bits=bits)
                torch.cuda.synchronize()
                gt = gate(name if bits == 4 else f"{name}_{bits}bit", yy)
                r = {"gate": gt, "weight_bytes": gwq.numel() + 2 * gws.numel() * 2}
                if gt["ok"]:
                    t = time_graphed(lambda: q4.gemm("affine", g.bs, gwq, gws, gwb, xq, xs, xsum, y=yy, bits=bits),
                                     20 if g.M >= 4096 else 50)
                    r.update({"gemm_us": round(t * 1e6, 2), "TOPS": round(ops / t / 1e12, 1),
                              "frac_int8_peak": round(ops / t / 1e12 / INT8_PEAK_TOPS, 4)})
                out[f"{name}_{bits}bit"] = r
                del gwq, gws, gwb
            del xt, wt, xq, xs, xsum, yy
        secondary["affine_code_widths"] = out

    if want("q4k_gemv") or want("q4k_gemm"):
        g1 = synth.workload("q4_k_gemv_1x4096x14336")
        w4 = torch.from_numpy(synth.gen.weights(g1)).to(dev)
        blocks = q4.q4k_quantize_weights(w4)
        del w4
        qbytes = blocks.numel()
        if want("q4k_gemv"):
            ncop = 32
            bcopies = [blocks.clone() for _ in range(ncop)]
            x1 = torch.from_numpy(synth.gen.activations(g1)).to(dev)
            y1 = torch.full((1, g1.N), float("nan"), dtype=torch.float32, device=dev)

            def kv(i):
                q4.q4k_gemv(bcopies[i % ncop], x1, g1.N, y=y1)
            kv(0)
            torch.cuda.synchronize()
            entry = {"gate": gate(g1.name, y1), "cold_weight_copies": ncop}
            if entry["gate"]["ok"]:
                t = graphed_rotating(kv, ncop, reps=20)
                entry.update({"us": round(t * 1e6, 3), "GB/s": round(qbytes / t / 1e9, 1),
                              "frac_hbm": round(qbytes / t / 1e9 / HBM_PEAK_GBS, 4)})
                if floors:
                    entry["frac_of_measured_stream"] = round(qbytes / t / 1e9 /
                                                             floors["stream_read_q4k_weights"]["GB/s"], 4)
            secondary["q4k_gemv_1x4096x14336"] = entry
            del bcopies
        if want("q4k_gemm"):
            g16 = synth.workload("q4_k_gemm_16x4096x14336")
            x16 = torch.from_numpy(synth.gen.activations(g16)).to(dev)
            y16 = torch.full((16, g16.N), float("nan"), dtype=torch.float32, device=dev)
            q4.q4k_gemm(blocks, x16, g16.N, y=y16)
            torch.cuda.synchronize()
            entry = {"gate": gate(g16.name, y16)}
            if entry["gate"]["ok"]:
                t = time_graphed(lambda: q4.q4k_gemm(blocks, x16, g16.N, y=y16), 200)
                flops = 2.0 * 16 * g16.N * g16.K
                # the products run on the f16 matrix cores (exact codes, split activations); the weight
                # stream is the bound, the float32 figure is for reference
                entry.update({"us": round(t * 1e6, 2), "TFLOPS": round(flops / t / 1e12, 2),
                              "GB/s": round(qbytes / t / 1e9, 1), "frac_hbm": round(qbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                              "frac_fp32_peak_reference": round(flops / t / 1e12 / FP32_PEAK_TFLOPS, 4),
                              "matrix_unit": "f16 (float32-accurate split)"})
            # the same product with the activations split once per call into a workspace (two launches)
            work = torch.empty(int(q4.lib().q4k_gemm_work_bytes(16, g16.K)), dtype=torch.uint8, device=dev)
            y16.fill_(float("nan"))
            q4.q4k_gemm_work(blocks, x16, g16.N, y=y16, work=work)
            torch.cuda.synchronize()
            gw = gate(g16.name, y16)
            entry["work_gate"] = gw
            if gw["ok"]:
                t = time_graphed(lambda: q4.q4k_gemm_work(blocks, x16, g16.N, y=y16, work=work), 200)
                entry.update({"work_us": round(t * 1e6, 2), "work_GB/s": round(qbytes / t / 1e9, 1),
                              "work_frac_hbm": round(qbytes / t / 1e9 / HBM_PEAK_GBS, 4)})
            secondary["q4k_gemm_16x4096x14336"] = entry

    if want("q4k_backward") or want("q4_backward"):
        # input gradient with frozen weights, dx [M][4096] = dy [M][14336] . dequant(W), 8 rotating weight copies
        g1 = synth.workload("q4_k_gemv_1x4096x14336")
        w4 = torch.from_numpy(synth.gen.weights(g1)).to(dev)
        out = {}
        for kind in ("q4_k", "q4_0"):
            if not want("q4k_backward" if kind == "q4_k" else "q4_backward"):
                continue
            if kind == "q4_k":
                blocks = q4.q4k_quantize_weights(w4)
                wts = [blocks.clone() for _ in range(8)]
                wbytes = blocks.numel()
                del blocks
            else:
                wq4, wd4, _ = q4.quantize_weights(w4, "q4_0", 32)
                wts = [(wq4.clone(), wd4.clone()) for _ in range(8)]
                wbytes = wq4.numel() + 2 * wd4.numel()
                del wq4, wd4
            for M in (1, 16):
                dyt = torch.from_numpy(synth.gen.activations(g1, M=M, K=g1.N)).to(dev)
                dxt = torch.full((M, g1.K), float("nan"), dtype=torch.float32, device=dev)
                work = torch.empty(int(q4.lib().q4_backward_work_bytes(M, g1.K, g1.N)) // 4, dtype=torch.float32,
                                   device=dev)

                def bw(i, dyt=dyt, dxt=dxt, work=work, kind=kind, wts=wts):
                    if kind == "q4_k":
                        q4.q4k_gemm_backward(wts[i % 8], dyt, g1.K, dx=dxt, work=work)
                    else:
                        q4.gemm_backward("q4_0", 32, wts[i % 8][0], wts[i % 8][1], None, dyt, dx=dxt, work=work)
                bw(0)
                torch.cuda.synchronize()
                r = {"gate": gate(f"backward_{kind}_{M}x4096x14336", dxt)}
                if r["gate"]["ok"]:
                    t = graphed_rotating(bw, 64, reps=3)
                    r.update({"us": round(t * 1e6, 2), "weight_GB/s": round(wbytes / t / 1e9, 1),
                              "TFLOPS": round(2.0 * M * g1.K * g1.N / t / 1e12, 2)})
                out[f"{kind}_{M}x4096x14336"] = r
            del wts
        secondary["input_gradient_frozen_weights"] = out
        del w4

    if secondary:
        result["secondary"] = secondary
    if floors.get("clocks_mhz_under_load") and floors["clocks_mhz_under_load"].get("sclk") and result:
        # MFMA rates scale with the shader clock; the percentages above use the 2.4 GHz peak
        result["clock_adjusted"] = {"sclk_mhz": floors["clocks_mhz_under_load"]["sclk"],
                                    "int8_peak_tops_at_sclk": round(INT8_PEAK_TOPS * floors["clocks_mhz_under_load"]
                                                                    ["sclk"] / PEAK_SCLK_MHZ, 1)}

    # ------------------------------------------------------------ CPU baseline (oracle)
    if args.only is None and not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, weight_bytes)

    print(json.dumps(result), flush=True)


def cpu_baseline(wl, weight_bytes):
    """The C oracle as it stands, timed on this process's host CPU share at 1 thread and at all of its threads
    (at most 16), on bounded samples of three workloads. The output column partition leaves every result
    bit-identical across thread counts."""
    import numpy as np

    import oracle
    import synth

    model, ncpu, share = host_cpu()
    T_all = max(1, min(share, 16))

    def timed(fn, budget_s=2.0, min_runs=1, max_runs=200):
        runs, t0 = 0, time.perf_counter()
        best = None
        while True:
            s = time.perf_counter()
            fn()
            d = time.perf_counter() - s
            best = d if best is None else min(best, d)
            runs += 1
            if (time.perf_counter() - t0 >= budget_s and runs >= min_runs) or runs >= max_runs:
                break
        return best, runs

    runs = []
    # decode workload: quantize + 1 x 4096 x 4096 Q4_0 GEMV (the headline's step)
    x1 = synth.gen.activations(wl)
    wq, wd = oracle.quantize_q4_0(synth.gen.weights(wl))

    def decode():
        a = oracle.quantize_act(x1, 32)
        oracle.q4_gemm(wq, wd, None, *a, wl.K, wl.N, 32, oracle.FMT_Q4_0)
    for T in sorted({1, T_all}):
        oracle.set_threads(T)
        best, n = timed(decode)
        runs.append({"workload": "q4_0_decode_4096 (quantize + GEMV, full)", "threads": T, "best_ms": round(best * 1e3, 3),
                     "runs": n, "GB/s": round(weight_bytes / best / 1e9, 3)})
    decode_best = {r["threads"]: r for r in runs}

    # MiniLM-shaped prefill: quantize + 64 x 384 x 1536 Q4_0 GEMM
    g0 = synth.workload("q4_0_minilm_64x384x1536")
    x0 = synth.gen.activations(g0)
    wq0, wd0 = oracle.quantize_q4_0(synth.gen.weights(g0))

    def minilm():
        a = oracle.quantize_act(x0, 32)
        oracle.q4_gemm(wq0, wd0, None, *a, g0.K, g0.N, 32, oracle.FMT_Q4_0)
    for T in sorted({1, T_all}):
        oracle.set_threads(T)
        best, n = timed(minilm)
        runs.append({"workload": "q4_0_minilm_64x384x1536 (quantize + GEMM, full)", "threads": T,
                     "best_ms": round(best * 1e3, 3), "runs": n,
                     "GOPS": round(2.0 * g0.M * g0.K * g0.N / best / 1e9, 2)})

    # Q4_K GEMV: the first 2048 of the 14336 weight rows (a bounded sample; GB/s of the rows read)
    g4 = synth.workload("q4_k_gemv_1x4096x14336")
    rows = 2048
    blocks = oracle.quantize_q4k(synth.gen.weights(g4, N=rows))
    x4 = synth.gen.activations(g4)
    for T in sorted({1, T_all}):
        oracle.set_threads(T)
        best, n = timed(lambda: oracle.q4k_gemv(blocks, x4, g4.K, rows), budget_s=2.0)
        runs.append({"workload": f"q4_k_gemv_1x4096x14336 (first {rows} of 14336 rows)", "threads": T,
                     "best_ms": round(best * 1e3, 3), "runs": n, "GB/s": round(blocks.nbytes / best / 1e9, 3)})
    oracle.set_threads(1)
    head = decode_best[T_all]
    return {"value": head["GB/s"], "unit": "GB/s", "cores": T_all, "kind": "oracle",
            "sample": f"the decode workload's full step (activation quantization + 1x4096x4096 Q4_0 W4A8 GEMV), "
                      f"best of {head['runs']} runs at {T_all} threads (output columns split over the threads); "
                      f"C oracle built with gcc -O2, no fast-math",
            "host_cpu": model, "host_logical_cpus": ncpu, "process_cpu_share": share,
            "runs": runs}


if __name__ == "__main__":
    main()
