"""Write tests/golden/bench_gate.json: the oracle's outputs at sampled coordinates
of every workload the benchmark times, for its agreement gate.

The benchmark checks each variant's output against these values on the GPU
before timing it (outside the timed region) and refuses to time a variant that
disagrees (meTile PR #29, "What I got wrong, and what it cost": only an
agreement gate keeps a fast wrong kernel from being measured and kept). The
benchmark itself never loads the oracle; this script is the only producer of
the file and calls nothing but `oracle` (quantizers, sampled products) and
`synth` (the seeded inputs, the same draws the benchmark makes).

Usage (repository root, CPU only, about a minute): python tests/golden/make_bench_gate.py
"""
from __future__ import annotations

import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "bench_gate.json")
SAMPLES = 64
FMT = {"q4_0": oracle.FMT_Q4_0, "affine": oracle.FMT_AFFINE}


def coords(M: int, N: int, seed: int, count: int = SAMPLES):
    """The four corners plus seeded random output coordinates."""
    rng = np.random.default_rng(seed)
    ms = np.concatenate([[0, 0, M - 1, M - 1], rng.integers(0, M, count)]).astype(np.int32)
    ns = np.concatenate([[0, N - 1, 0, N - 1], rng.integers(0, N, count)]).astype(np.int32)
    return ms, ns


def entry(ms, ns, y, **extra):
    d = {"ms": [int(v) for v in ms], "ns": [int(v) for v in ns],
         "y_bits": [int(v) for v in np.asarray(y, dtype=np.float32).view(np.uint32)]}
    d.update(extra)
    return d


def w4_case(wts, fmt, bs, x, seed, bits=4):
    K = x.shape[1]
    N = wts[1].shape[0]
    act = oracle.quantize_act(x, bs)
    ms, ns = coords(x.shape[0], N, seed)
    wb = wts[2] if fmt == "affine" else None
    y = oracle.q4_gemm_sample(wts[0], wts[1], wb, *act, K, N, bs, FMT[fmt], ms, ns, bits=bits)
    return entry(ms, ns, y)


def main():
    cases = {}

    # decode workload (Q4_0 1 x 4096 x 4096): fused and plain GEMV, few-row rows
    wl = synth.workload("q4_0_decode_4096")
    x = synth.gen.activations(wl)
    wts = oracle.quantize_q4_0(synth.gen.weights(wl))
    xq, xs, xsum = oracle.quantize_act(x, 32)
    ms, ns = coords(1, wl.N, 1, 256)
    y = oracle.q4_gemm_sample(wts[0], wts[1], None, xq, xs, xsum, wl.K, wl.N, 32, oracle.FMT_Q4_0, ms, ns)
    cases["q4_0_decode_4096"] = entry(ms, ns, y, xs_bits=[int(v) for v in xs.view(np.uint32).reshape(-1)],
                                      xsum=[int(v) for v in xsum.reshape(-1)],
                                      xq_sha256=hashlib.sha256(xq.tobytes()).hexdigest())
    for M in (2, 4, 6, 8, 16, 32):
        cases[f"q4_0_rows_{M}x4096x4096"] = w4_case(wts, "q4_0", 32, synth.gen.activations(wl, M=M), 100 + M)

    # prefill workloads
    for name in ("q4_0_minilm_64x384x1536", "affine_g64_1024x4096x4096", "affine_g128_4096x4096x14336",
                 "affine_g128_4096x14336x4096"):
        g = synth.workload(name)
        xg = synth.gen.activations(g)
        wg = synth.gen.weights(g)
        bit_list = (4, 6, 8) if name in ("affine_g64_1024x4096x4096", "affine_g128_4096x4096x14336") else (4,)
        for bits in bit_list:
            if g.fmt == "q4_0":
                wt = oracle.quantize_q4_0(wg)
            else:
                wt = oracle.quantize_affine(wg, g.bs, bits=bits)
            key = name if bits == 4 else f"{name}_{bits}bit"
            cases[key] = w4_case(wt, g.fmt, g.bs, xg, 7, bits=bits)
            print(key, flush=True)

    # Q4_K: GEMV (M = 1) and GEMM (M = 16) share the weights; input gradient
    g1 = synth.workload("q4_k_gemv_1x4096x14336")
    g16 = synth.workload("q4_k_gemm_16x4096x14336")
    w4 = synth.gen.weights(g1)
    blocks = oracle.quantize_q4k(w4)
    for g in (g1, g16):
        xk = synth.gen.activations(g)
        ms, ns = coords(g.M, g.N, 11)
        cases[g.name] = entry(ms, ns, oracle.q4k_gemm_sample(blocks, xk, g.K, g.N, ms, ns))
    q0 = oracle.quantize_q4_0(w4)
    for M in (1, 16):
        dy = synth.gen.activations(g1, M=M, K=g1.N)
        ms, ks = coords(M, g1.K, 20 + M)
        cases[f"backward_q4_k_{M}x4096x14336"] = entry(
            ms, ks, oracle.q4k_backward_sample(blocks, dy, g1.K, g1.N, ms, ks))
        cases[f"backward_q4_0_{M}x4096x14336"] = entry(
            ms, ks, oracle.q4_backward_sample(q0[0], q0[1], None, dy, g1.K, g1.N, 32, oracle.FMT_Q4_0, ms, ks))
    print("q4_k, backward", flush=True)

    doc = {"about": "Oracle outputs at sampled coordinates of the benchmark's workloads (seeded synth inputs), "
                    "written by tests/golden/make_bench_gate.py; y as float32 bit patterns. The benchmark's "
                    "agreement gate compares each variant against these before timing it.",
           "samples_per_case": SAMPLES, "cases": cases}
    with open(OUT, "w") as f:
        json.dump(doc, f, separators=(",", ":"))
        f.write("\n")
    print(f"wrote {OUT} ({len(cases)} cases)")


if __name__ == "__main__":
    main()
