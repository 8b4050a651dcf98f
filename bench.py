#!/usr/bin/env python3
"""Benchmark of the W4A8 block-quantized matmul hot path on one MI355X.

Headline (the `value` of the JSON line): decode GEMV weight GB/s on the
4096 x 4096 Q4_0 decode workload (M = 1, float32 activations with 1% outliers
x20). One step is one pass of the decode hot path over one activation vector:
per-block int8 quantization of x, the exact per-block int8 dots against the
packed 4-bit weights, the per-block float rescale and the wavefront reduce,
all in one fused launch (q4_gemv_fused). Steps rotate through 100 copies of
the weights (944 MB, well above the 256 MB last-level cache), so every step
streams its weights from HBM; the steps are replayed from a HIP graph.

The same line carries, under "secondary", the prefill GEMM int8 TOPS (the
second half of the metric) on the affine g128 4096-row workloads and the
other workloads of the pages, and under "cpu_baseline" the C oracle timed on
the host on a bounded sample of the decode workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode GEMV weight GB/s (%HBM peak); prefill GEMM int8 TOPS (%MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 (vector and matrix)
GRAPH_STEPS = 100              # steps per captured graph = rotating weight copies
PROFILES = os.path.join(ROOT, "profiles")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--no-secondary", action="store_true", help="headline decode line only")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", default=None,
                   help="run one workload alone (for profiling): gemv_fused (eager decode launches, --steps of "
                        "them), gemm_3a, gemm_3b, gemm_2, gemm_0, q4k_gemv, q4k_gemm, act_quant, gemv_plain, "
                        "small_m, q4k_backward, q4_backward, gemm_bits")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="run a plain device-to-device copy of this many MiB (counter calibration) and exit")
    return p.parse_args()


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        for f in (os.path.join(ROOT, "block_quantized_bit_amd", "csrc", n),
                  os.path.join(ROOT, "block_quantized_bit_amd", "csrc", "common.h")):
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(name: str, src_hash: str, launches_per_counter: int = 1):
    """HBM bytes per launch from a committed counter summary, or None when the
    summary is missing or was taken on a different kernel source."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
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


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}, "
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

    def graph_of(fn, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                fn(i)
        return g

    def event_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

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
    if args.only is None:
        for i in range(min(args.warmup, GRAPH_STEPS)):
            decode_step(i)
        torch.cuda.synchronize()
        g_main = graph_of(decode_step, GRAPH_STEPS)
        rem = args.steps % GRAPH_STEPS
        g_rem = graph_of(decode_step, rem) if rem else None
        reps = args.steps // GRAPH_STEPS
        warm_reps = max(1, args.warmup // GRAPH_STEPS)
        for _ in range(warm_reps):
            g_main.replay()
        torch.cuda.synchronize()

        e0, e1 = event_pair()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(reps):
            g_main.replay()
        if g_rem is not None:
            g_rem.replay()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        wall_s = t1 - t0
        # one launch per step: the events over the timed region give the
        # fused kernel's average launch duration (graph-dispatched, back to back)
        kern_s = e0.elapsed_time(e1) / 1e3 / args.steps
        ms_per_step = wall_s * 1e3 / args.steps
        value = weight_bytes / (wall_s / args.steps) / 1e9
        achieved = weight_bytes / kern_s / 1e9
        src_hash = kernel_source_hash(["gemv.hip"])
        traffic = read_traffic("gemv_fused_q4_0_decode_4096_counters.txt", src_hash)
        result = {
            "metric": METRIC,
            "value": round(value, 1),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 6),
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
                "launch": "q4_gemv_fused, one launch per step, replayed from a HIP graph",
            },
            "roofline": {
                "bound": "hbm",
                "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "kernel": "q4::gemv_kernel (fused quantize + GEMV)",
                "kernel_avg_us": round(kern_s * 1e6, 3),
                "algorithmic_bytes_per_launch": weight_bytes,
            },
        }

    # ------------------------------------------------------------ secondary
    secondary = {}
    want = (lambda k: args.only == k) if args.only else (lambda k: not args.no_secondary)

    if want("gemv_plain"):
        xq, xs, xsum = q4.quantize_act(x, 32)

        def plain(i):
            c = copies[i % GRAPH_STEPS]
            q4.gemv("q4_0", 32, c[0], c[1], None, xq, xs, xsum, y=y)
        plain(0)
        g = graph_of(plain, GRAPH_STEPS)
        g.replay()
        e0, e1 = event_pair()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 1e3 / (10 * GRAPH_STEPS)
        secondary["gemv_plain_q4_0_decode_4096"] = {
            "what": "q4_gemv (activation codes given), cold weights, HIP graph", "us": round(t * 1e6, 3),
            "GB/s": round(weight_bytes / t / 1e9, 1), "frac_hbm": round(weight_bytes / t / 1e9 / HBM_PEAK_GBS, 4)}

    if want("small_m"):
        # few-row decode: M rows of decode-like activations against the same cold weight copies
        rows = {}
        for M in (2, 4, 6, 8, 16, 32):
            xm = torch.from_numpy(synth.gen.activations(wl, M=M)).to(dev)
            xq_m, xs_m, xsum_m = q4.quantize_act(xm, 32)
            y_m = torch.empty((M, wl.N), dtype=torch.float32, device=dev)

            def few(i, xq_m=xq_m, xs_m=xs_m, xsum_m=xsum_m, y_m=y_m):
                c = copies[i % GRAPH_STEPS]
                q4.gemm("q4_0", 32, c[0], c[1], None, xq_m, xs_m, xsum_m, y=y_m)
            few(0)
            g = graph_of(few, GRAPH_STEPS)
            g.replay()
            e0, e1 = event_pair()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(10):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / 1e3 / (10 * GRAPH_STEPS)
            rows[str(M)] = {"us": round(t * 1e6, 3), "GB/s": round(weight_bytes / t / 1e9, 1),
                            "frac_hbm": round(weight_bytes / t / 1e9 / HBM_PEAK_GBS, 4),
                            "TOPS": round(2.0 * M * wl.K * wl.N / t / 1e12, 2)}
        secondary["small_m_q4_0_rows_x4096x4096"] = {
            "what": "q4_gemm with M rows (few-row kernel: each weight block read once for all rows), cold weights, "
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
        torch.cuda.synchronize()
        e0, e1 = event_pair()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / (iters * reps)

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
        yy = torch.empty((g.M, g.N), dtype=torch.float32, device=dev)
        t_gemm = time_graphed(lambda: q4.gemm(g.fmt, g.bs, gwq, gws, gwb, xq, xs, xsum, y=yy), iters)
        t_act = time_graphed(lambda: q4.quantize_act(xt, g.bs, out=(xq, xs, xsum)), iters)
        ops = 2.0 * g.M * g.N * g.K
        act_bytes = xt.numel() * xt.element_size() + xq.numel() + 8 * xs.numel()
        entry = {
            "gemm_us": round(t_gemm * 1e6, 2), "gemm_TOPS": round(ops / t_gemm / 1e12, 1),
            "gemm_frac_int8_peak": round(ops / t_gemm / 1e12 / INT8_PEAK_TOPS, 4),
            "act_quant_us": round(t_act * 1e6, 2), "act_quant_GB/s": round(act_bytes / t_act / 1e9, 1),
            "step_TOPS": round(ops / (t_gemm + t_act) / 1e12, 1)}
        if g.M > 32:
            # pre-packed weights, fused quantize + GEMM (two launches, group-major activation scales)
            packed = q4.pack_weights(g.fmt, g.bs, gwq, gws, gwb)
            work = torch.empty(int(q4.lib().q4_gemm_packed_work_bytes(g.M, g.K, g.bs)), dtype=torch.uint8,
                               device=dev)
            t_pk = time_graphed(lambda: q4.gemm_packed(g.fmt, g.bs, xt, packed, g.N, y=yy, work=work), iters)
            entry.update({"packed_step_us": round(t_pk * 1e6, 2), "packed_step_TOPS": round(ops / t_pk / 1e12, 1),
                          "packed_gemm_us_est": round((t_pk - t_act) * 1e6, 2),
                          "packed_gemm_frac_int8_peak_est": round(ops / (t_pk - t_act) / 1e12 / INT8_PEAK_TOPS, 4)})
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
                t = time_graphed(lambda: q4.gemm("affine", g.bs, gwq, gws, gwb, xq, xs, xsum, y=yy, bits=bits),
                               20 if g.M >= 4096 else 50)
                out[f"{name}_{bits}bit"] = {"gemm_us": round(t * 1e6, 2), "TOPS": round(ops / t / 1e12, 1),
                                            "frac_int8_peak": round(ops / t / 1e12 / INT8_PEAK_TOPS, 4),
                                            "weight_bytes": gwq.numel() + 2 * gws.numel() * 2}
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
            y1 = torch.empty((1, g1.N), dtype=torch.float32, device=dev)

            def kv(i):
                q4.q4k_gemv(bcopies[i % ncop], x1, g1.N, y=y1)
            kv(0)
            gg = graph_of(kv, ncop)
            gg.replay()
            e0, e1 = event_pair()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(20):
                gg.replay()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / 1e3 / (20 * ncop)
            secondary["q4k_gemv_1x4096x14336"] = {
                "us": round(t * 1e6, 3), "GB/s": round(qbytes / t / 1e9, 1),
                "frac_hbm": round(qbytes / t / 1e9 / HBM_PEAK_GBS, 4), "cold_weight_copies": ncop}
            del bcopies
        if want("q4k_gemm"):
            g16 = synth.workload("q4_k_gemm_16x4096x14336")
            x16 = torch.from_numpy(synth.gen.activations(g16)).to(dev)
            y16 = torch.empty((16, g16.N), dtype=torch.float32, device=dev)
            t = time_graphed(lambda: q4.q4k_gemm(blocks, x16, g16.N, y=y16), 200)
            flops = 2.0 * 16 * g16.N * g16.K
            # float32-equivalent work; the products run on the f16 matrix cores (exact codes, split
            # activations), so the float32 peak is a reference figure, and the weight stream is the bound
            secondary["q4k_gemm_16x4096x14336"] = {
                "us": round(t * 1e6, 2), "TFLOPS": round(flops / t / 1e12, 2),
                "frac_fp32_peak": round(flops / t / 1e12 / FP32_PEAK_TFLOPS, 4), "GB/s": round(qbytes / t / 1e9, 1),
                "frac_hbm": round(qbytes / t / 1e9 / HBM_PEAK_GBS, 4), "matrix_unit": "f16 (float32-accurate split)"}

    if want("q4k_backward") or want("q4_backward"):
        # input gradient with frozen weights, dx [M][4096] = dy [M][14336] . dequant(W), 8 rotating weight copies
        g1 = synth.workload("q4_k_gemv_1x4096x14336")
        w4 = torch.from_numpy(synth.gen.weights(g1)).to(dev)
        out = {}
        if want("q4k_backward"):
            blocks = q4.q4k_quantize_weights(w4)
            wcopies = [blocks.clone() for _ in range(8)]
            wbytes = blocks.numel()
            for M in (1, 16):
                dyt = torch.randn((M, g1.N), generator=torch.Generator(device="cpu").manual_seed(M)).to(dev)
                dxt = torch.empty((M, g1.K), dtype=torch.float32, device=dev)
                work = torch.empty(int(q4.lib().q4_backward_work_bytes(M, g1.K, g1.N)) // 4, dtype=torch.float32,
                                   device=dev)
                it = [0]

                def bw():
                    q4.q4k_gemm_backward(wcopies[it[0] % 8], dyt, g1.K, dx=dxt, work=work)
                    it[0] += 1
                t = time_graphed(bw, 64)
                out[f"q4k_{M}x4096x14336"] = {"us": round(t * 1e6, 2), "weight_GB/s": round(wbytes / t / 1e9, 1),
                                              "TFLOPS": round(2.0 * M * g1.K * g1.N / t / 1e12, 2)}
            del wcopies, blocks
        if want("q4_backward"):
            wq, wd, _ = q4.quantize_weights(w4, "q4_0", 32)
            wbytes = wq.numel() + 2 * wd.numel()
            for M in (1, 16):
                dyt = torch.randn((M, g1.N), generator=torch.Generator(device="cpu").manual_seed(M)).to(dev)
                dxt = torch.empty((M, g1.K), dtype=torch.float32, device=dev)
                work = torch.empty(int(q4.lib().q4_backward_work_bytes(M, g1.K, g1.N)) // 4, dtype=torch.float32,
                                   device=dev)
                t = time_graphed(lambda: q4.gemm_backward("q4_0", 32, wq, wd, None, dyt, dx=dxt, work=work), 64)
                out[f"q4_0_{M}x4096x14336"] = {"us": round(t * 1e6, 2), "weight_GB/s": round(wbytes / t / 1e9, 1),
                                               "TFLOPS": round(2.0 * M * g1.K * g1.N / t / 1e12, 2)}
        secondary["input_gradient_frozen_weights"] = out
        del w4

    if secondary:
        result["secondary"] = secondary

    # ------------------------------------------------------------ CPU baseline (oracle)
    if args.only is None and not args.no_cpu_baseline:
        import oracle
        xw = synth.gen.activations(wl)
        ww = synth.gen.weights(wl)
        owq, owd = oracle.quantize_q4_0(ww)
        runs, t0 = 0, time.perf_counter()
        while True:
            act = oracle.quantize_act(xw, 32)
            oracle.q4_gemm(owq, owd, None, *act, wl.K, wl.N, 32, oracle.FMT_Q4_0)
            runs += 1
            el = time.perf_counter() - t0
            if el >= 10.0 or runs >= 2000:
                break
        per = el / runs
        result["cpu_baseline"] = {
            "value": round(weight_bytes / per / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{runs} full decode steps (activation quantization + 1x4096x4096 Q4_0 W4A8 GEMV) of the "
                      f"same workload, single-threaded C oracle (gcc -O2), {el:.1f} s",
            "ms_per_step": round(per * 1e3, 3)}

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
