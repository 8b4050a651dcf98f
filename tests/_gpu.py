"""Helpers of the GPU parity tests: device copies and the comparison metric."""
import functools

import numpy as np
import torch

import oracle
import synth

TOL = 1e-5   # relative RMS bound of float outputs against the oracle


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are reinterpreted as `dtype` (bf16 / fp16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).to(dev())
        return t.view(dtype if dtype is not None else torch.bfloat16)
    return torch.from_numpy(a).to(dev())


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def rel_rms(y, ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.sqrt(((y - ref) ** 2).sum()) / np.sqrt((ref ** 2).sum()))


@functools.lru_cache(maxsize=4)
def workload_data(name: str):
    """Seeded inputs of a named workload, quantized by the oracle:
    (workload, x, w, (xq, xs, xsum), weight arrays)."""
    wl = synth.workload(name)
    x = synth.gen.activations(wl)
    w = synth.gen.weights(wl)
    act = oracle.quantize_act(x, wl.bs) if wl.fmt != "q4_k" else None
    if wl.fmt == "q4_0":
        wts = oracle.quantize_q4_0(w)
    elif wl.fmt == "affine":
        wts = oracle.quantize_affine(w, wl.bs)
    else:
        wts = oracle.quantize_q4k(w)
    return wl, x, w, act, wts


def sample_pairs(M: int, N: int, count: int, seed: int):
    """Output coordinates for sampled parity: the four corners, the last row and
    column, and seeded random pairs."""
    rng = np.random.default_rng(seed)
    ms = [0, 0, M - 1, M - 1] + list(rng.integers(0, M, count)) + [M - 1] * 16
    ns = [0, N - 1, 0, N - 1] + list(rng.integers(0, N, count)) + list(rng.integers(0, N, 16))
    return np.array(ms, dtype=np.int32), np.array(ns, dtype=np.int32)
