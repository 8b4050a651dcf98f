"""Host-side parts of bench.py (no GPU): the trace summary, the refusal of
more than one GPU, and the stored agreement-gate values."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_summarize_trace_median(tmp_path):
    p = tmp_path / "k_kernel_trace.csv"
    rows = ["Kind,Kernel_Name,Start_Timestamp,End_Timestamp"]
    for i, d in enumerate([100, 300, 200, 1000]):
        rows.append(f"KERNEL_DISPATCH,kern_a,{10000 * i},{10000 * i + d}")
    rows.append("KERNEL_DISPATCH,kern_b,0,50")
    p.write_text("\n".join(rows) + "\n")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-trace", str(p)],
                       capture_output=True, text=True, check=True)
    line = [ln for ln in r.stdout.splitlines() if "kern_a" in ln][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[1:6] == ["4", "400", "250", "100", "1000"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_gate_values_cover_every_timed_variant():
    doc = json.load(open(os.path.join(ROOT, "tests", "golden", "bench_gate.json")))
    cases = doc["cases"]
    want = ["q4_0_decode_4096", "q4_0_minilm_64x384x1536", "affine_g64_1024x4096x4096",
            "affine_g128_4096x4096x14336", "affine_g128_4096x14336x4096", "q4_k_gemv_1x4096x14336",
            "q4_k_gemm_16x4096x14336"]
    want += [f"q4_0_rows_{M}x4096x4096" for M in (2, 4, 6, 8, 16, 32)]
    want += [f"affine_g64_1024x4096x4096_{b}bit" for b in (6, 8)]
    want += [f"backward_{k}_{M}x4096x14336" for k in ("q4_k", "q4_0") for M in (1, 16)]
    for k in want:
        c = cases[k]
        assert len(c["ms"]) == len(c["ns"]) == len(c["y_bits"]) >= 64
        y = np.array(c["y_bits"], dtype=np.uint32).view(np.float32)
        assert np.isfinite(y).all() and np.abs(y).sum() > 0
    assert len(cases["q4_0_decode_4096"]["xs_bits"]) == 4096 // 32


def test_gate_values_reproduce_from_the_oracle(orc):
    # one case recomputed: the stored values are the oracle's on the seeded inputs
    import synth
    doc = json.load(open(os.path.join(ROOT, "tests", "golden", "bench_gate.json")))
    c = doc["cases"]["q4_0_rows_4x4096x4096"]
    wl = synth.workload("q4_0_decode_4096")
    wq, wd = orc.quantize_q4_0(synth.gen.weights(wl))
    act = orc.quantize_act(synth.gen.activations(wl, M=4), 32)
    y = orc.q4_gemm_sample(wq, wd, None, *act, 4096, 4096, 32, orc.FMT_Q4_0, np.array(c["ms"], np.int32),
                           np.array(c["ns"], np.int32))
    assert y.view(np.uint32).tolist() == c["y_bits"]
