"""ctypes binding of the C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path. It shares no
code with the HIP library; both sides receive the same seeded inputs from
`synth`.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FMT_Q4_0 = 0
FMT_AFFINE = 1
Q4K_BLOCK_BYTES = 144
Q4K_QK = 256

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-pthread"]
# The sanitizer build of the same source (host code only; run by the CPU tests
# with the sanitizer runtimes preloaded into the Python process).
SAN_CFLAGS = ["-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-pthread",
              "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
# ORACLE_LIB names a prebuilt oracle library to load instead (the sanitizer build).
_ENV_LIB = os.environ.get("ORACLE_LIB")


def build(force: bool = True) -> str:
    """Compile oracle.c with plain gcc (no -ffast-math, no -march=native)."""
    if _ENV_LIB:
        return _ENV_LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(path: str) -> str:
    """Compile oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer into `path`."""
    subprocess.check_call(["gcc", *SAN_CFLAGS, _SRC, "-o", path, "-lm"])
    return path


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_ENV_LIB or _LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.or_set_threads.argtypes = [I]
        L.or_set_threads.restype = I
        L.or_f16_to_f32.restype = ctypes.c_float
        L.or_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.or_f32_to_f16.restype = ctypes.c_uint16
        L.or_f32_to_f16.argtypes = [ctypes.c_float]
        L.or_bf16_to_f32.restype = ctypes.c_float
        L.or_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.or_f32_to_bf16.restype = ctypes.c_uint16
        L.or_f32_to_bf16.argtypes = [ctypes.c_float]
        for name in ("or_f16_to_f32_array", "or_f32_to_f16_array", "or_f32_to_bf16_array"):
            getattr(L, name).argtypes = [P, P, ctypes.c_long]
            getattr(L, name).restype = None
        L.or_quantize_act.argtypes = [I, I, I, I, P, P, P, P]
        L.or_quantize_q4_0.argtypes = [I, I, P, P, P]
        L.or_quantize_affine.argtypes = [I, I, I, P, P, P, P]
        L.or_q4_partials.argtypes = [I, I, I, I, I, P, P, I, I, P]
        L.or_q4_gemm.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P]
        L.or_q4_gemm_sample.argtypes = [I, I, I, I, I, P, P, P, P, P, P, I, P, P, P]
        L.or_get_code.argtypes = [P, I, I, I]
        L.or_q4k_pack_scales.argtypes = [P, P, P]
        L.or_q4k_pack_scales.restype = None
        L.or_q4k_unpack_scales.argtypes = [P, P, P]
        L.or_q4k_unpack_scales.restype = None
        L.or_q4k_dequant.argtypes = [I, I, P, P]
        L.or_quantize_q4k.argtypes = [I, I, P, P]
        L.or_q4k_gemv.argtypes = [I, I, P, P, P]
        L.or_q4k_gemm.argtypes = [I, I, I, P, P, P]
        L.or_q4k_gemm_sample.argtypes = [I, I, I, P, P, I, P, P, P]
        L.or_q4k_backward.argtypes = [I, I, I, P, P, P]
        L.or_code_bytes.argtypes = [I, I, I]
        L.or_code_bytes.restype = ctypes.c_long
        L.or_get_code_bits.argtypes = [P, I, I, I, I, I]
        L.or_quantize_affine_bits.argtypes = [I, I, I, I, P, P, P, P]
        L.or_q4_partials_bits.argtypes = [I, I, I, I, I, I, P, P, I, I, P]
        L.or_q4_gemm_bits.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P]
        L.or_q4_gemm_sample_bits.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, I, P, P, P]
        L.or_q4_backward.argtypes = [I, I, I, I, I, P, P, P, P, P]
        L.or_q4k_backward_sample.argtypes = [I, I, I, P, P, I, P, P, P]
        L.or_q4_backward_sample.argtypes = [I, I, I, I, I, P, P, P, P, I, P, P, P]
        _lib = L
    return _lib


def set_threads(t: int) -> int:
    """Threads the products (q4_gemm, q4k_gemv, q4k_gemm) split their output
    columns over; results are bit-identical for every count. Returns the count set."""
    return lib().or_set_threads(int(t))


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _ok(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle: {what} rejected its arguments")


# ---- number formats --------------------------------------------------------

def f16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().or_f16_to_f32_array(_p(h), _p(out), h.size)
    return out


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().or_f32_to_f16_array(_p(x), _p(out), x.size)
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().or_f32_to_bf16_array(_p(x), _p(out), x.size)
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return np.array([lib().or_bf16_to_f32(int(v)) for v in b.reshape(-1)],
                    dtype=np.float32).reshape(b.shape)


# ---- quantizers ------------------------------------------------------------

def quantize_act(x: np.ndarray, bs: int):
    """x [M][K] float32 or bfloat16 bits (uint16) -> (xq int8, xs float32, xsum int32)."""
    x = np.ascontiguousarray(x)
    xdt = 1 if x.dtype == np.uint16 else 0
    if xdt == 0:
        x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    xq = np.empty((M, K), dtype=np.int8)
    xs = np.empty((M, K // bs), dtype=np.float32)
    xsum = np.empty((M, K // bs), dtype=np.int32)
    _ok(lib().or_quantize_act(M, K, bs, xdt, _p(x), _p(xq), _p(xs), _p(xsum)), "quantize_act")
    return xq, xs, xsum


def quantize_q4_0(w: np.ndarray):
    """w [N][K] float32 -> (wq uint8 [N][K/2], wd fp16 bits [N][K/32])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    wq = np.empty((N, K // 2), dtype=np.uint8)
    wd = np.empty((N, K // 32), dtype=np.uint16)
    _ok(lib().or_quantize_q4_0(N, K, _p(w), _p(wq), _p(wd)), "quantize_q4_0")
    return wq, wd


def code_array_shape(N: int, K: int, bits: int):
    """Shape of the code array at a bit width: [N][K/2] (4), [N][K] (8), or one flat buffer of
    N*K*3/4 bytes (6: the low-nibble layout of 4 bits, then the high 2-bit plane)."""
    return {4: (N, K // 2), 8: (N, K), 6: (N * K * 3 // 4,)}[bits]


def quantize_affine(w_bf16: np.ndarray, g: int, bits: int = 4):
    """w [N][K] bfloat16 bits -> (wq uint8 codes, ws, wb bfloat16 bits [N][K/g]); codes 0 .. 2^bits - 1."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    N, K = w.shape
    wq = np.empty(code_array_shape(N, K, bits), dtype=np.uint8)
    ws = np.empty((N, K // g), dtype=np.uint16)
    wb = np.empty((N, K // g), dtype=np.uint16)
    _ok(lib().or_quantize_affine_bits(N, K, g, bits, _p(w), _p(wq), _p(ws), _p(wb)), "quantize_affine")
    return wq, ws, wb


def quantize_q4k(w: np.ndarray) -> np.ndarray:
    """w [N][K] float32 -> blocks uint8 [N][K/256 * 144]."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    blocks = np.empty((N, K // Q4K_QK * Q4K_BLOCK_BYTES), dtype=np.uint8)
    _ok(lib().or_quantize_q4k(N, K, _p(w), _p(blocks)), "quantize_q4k")
    return blocks


def get_code(wq: np.ndarray, K: int, n: int, k: int, bits: int = 4, N: int | None = None) -> int:
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    if bits == 4:
        return lib().or_get_code(_p(wq), K, n, k)
    if N is None:
        N = wq.size * 8 // (K * bits)
    return lib().or_get_code_bits(_p(wq), N, K, bits, n, k)


def q4k_pack_scales(sc, mn) -> np.ndarray:
    sc = np.ascontiguousarray(sc, dtype=np.uint8)
    mn = np.ascontiguousarray(mn, dtype=np.uint8)
    out = np.zeros(12, dtype=np.uint8)
    lib().or_q4k_pack_scales(_p(sc), _p(mn), _p(out))
    return out


def q4k_unpack_scales(b12):
    b12 = np.ascontiguousarray(b12, dtype=np.uint8)
    sc = np.zeros(8, dtype=np.uint8)
    mn = np.zeros(8, dtype=np.uint8)
    lib().or_q4k_unpack_scales(_p(b12), _p(sc), _p(mn))
    return sc, mn


def q4k_dequant(blocks: np.ndarray, N: int, K: int) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    w = np.empty((N, K), dtype=np.float64)
    _ok(lib().or_q4k_dequant(N, K, _p(blocks), _p(w)), "q4k_dequant")
    return w


# ---- results ---------------------------------------------------------------

def q4_partials(wq, xq, K: int, N: int, bs: int, fmt: int, m0: int = 0, m1: int | None = None, bits: int = 4):
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    M = xq.shape[0]
    m1 = M if m1 is None else m1
    out = np.empty((m1 - m0, N, K // bs), dtype=np.int32)
    _ok(lib().or_q4_partials_bits(M, K, N, bs, fmt, bits, _p(wq), _p(xq), m0, m1, _p(out)), "q4_partials")
    return out


def _scales(wscale, wbias):
    ws = np.ascontiguousarray(wscale, dtype=np.uint16)
    wb = None if wbias is None else np.ascontiguousarray(wbias, dtype=np.uint16)
    return ws, wb


def q4_gemm(wq, wscale, wbias, xq, xs, xsum, K: int, N: int, bs: int, fmt: int, bits: int = 4) -> np.ndarray:
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    ws, wb = _scales(wscale, wbias)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    xsum = np.ascontiguousarray(xsum, dtype=np.int32)
    M = xq.shape[0]
    y = np.empty((M, N), dtype=np.float32)
    _ok(lib().or_q4_gemm_bits(M, K, N, bs, fmt, bits, _p(wq), _p(ws), None if wb is None else _p(wb),
                              _p(xq), _p(xs), _p(xsum), _p(y)), "q4_gemm")
    return y


def q4_gemm_sample(wq, wscale, wbias, xq, xs, xsum, K: int, N: int, bs: int, fmt: int,
                   ms, ns, bits: int = 4) -> np.ndarray:
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    ws, wb = _scales(wscale, wbias)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    xsum = np.ascontiguousarray(xsum, dtype=np.int32)
    ms = np.ascontiguousarray(ms, dtype=np.int32)
    ns = np.ascontiguousarray(ns, dtype=np.int32)
    M = xq.shape[0]
    y = np.empty(ms.shape[0], dtype=np.float32)
    _ok(lib().or_q4_gemm_sample_bits(M, K, N, bs, fmt, bits, _p(wq), _p(ws), None if wb is None else _p(wb),
                                     _p(xq), _p(xs), _p(xsum), ms.shape[0], _p(ms), _p(ns), _p(y)),
        "q4_gemm_sample")
    return y


def q4k_gemm(blocks, x, K: int, N: int) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    M = x.shape[0]
    y = np.empty((M, N), dtype=np.float32)
    _ok(lib().or_q4k_gemm(M, K, N, _p(blocks), _p(x), _p(y)), "q4k_gemm")
    return y


def q4k_gemv(blocks, x, K: int, N: int) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    y = np.empty(N, dtype=np.float32)
    _ok(lib().or_q4k_gemv(K, N, _p(blocks), _p(x), _p(y)), "q4k_gemv")
    return y


def q4k_gemm_sample(blocks, x, K: int, N: int, ms, ns) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    ms = np.ascontiguousarray(ms, dtype=np.int32)
    ns = np.ascontiguousarray(ns, dtype=np.int32)
    y = np.empty(ms.shape[0], dtype=np.float32)
    _ok(lib().or_q4k_gemm_sample(x.shape[0], K, N, _p(blocks), _p(x), ms.shape[0], _p(ms),
                                 _p(ns), _p(y)), "q4k_gemm_sample")
    return y


# ---- input gradient with frozen weights ---------------------------------------

def q4k_backward(blocks, dy, K: int, N: int) -> np.ndarray:
    """dx [M][K] = dy [M][N] . dequant(W) (C-Kernel-Engine backward pass: W^T . dY per row)."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    M = dy.shape[0]
    dx = np.empty((M, K), dtype=np.float32)
    _ok(lib().or_q4k_backward(M, K, N, _p(blocks), _p(dy), _p(dx)), "q4k_backward")
    return dx


def q4_backward(wq, wscale, wbias, dy, K: int, N: int, bs: int, fmt: int) -> np.ndarray:
    """dx [M][K] = dy [M][N] . dequant(W) for Q4_0 / affine weights."""
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    ws, wb = _scales(wscale, wbias)
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    M = dy.shape[0]
    dx = np.empty((M, K), dtype=np.float32)
    _ok(lib().or_q4_backward(M, K, N, bs, fmt, _p(wq), _p(ws), None if wb is None else _p(wb), _p(dy), _p(dx)),
        "q4_backward")
    return dx


def q4k_backward_sample(blocks, dy, K: int, N: int, ms, ks) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    ms = np.ascontiguousarray(ms, dtype=np.int32)
    ks = np.ascontiguousarray(ks, dtype=np.int32)
    dx = np.empty(ms.shape[0], dtype=np.float32)
    _ok(lib().or_q4k_backward_sample(dy.shape[0], K, N, _p(blocks), _p(dy), ms.shape[0], _p(ms), _p(ks), _p(dx)),
        "q4k_backward_sample")
    return dx


def q4_backward_sample(wq, wscale, wbias, dy, K: int, N: int, bs: int, fmt: int, ms, ks) -> np.ndarray:
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    ws, wb = _scales(wscale, wbias)
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    ms = np.ascontiguousarray(ms, dtype=np.int32)
    ks = np.ascontiguousarray(ks, dtype=np.int32)
    dx = np.empty(ms.shape[0], dtype=np.float32)
    _ok(lib().or_q4_backward_sample(dy.shape[0], K, N, bs, fmt, _p(wq), _p(ws), None if wb is None else _p(wb),
                                    _p(dy), ms.shape[0], _p(ms), _p(ks), _p(dx)), "q4_backward_sample")
    return dx
