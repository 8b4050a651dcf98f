"""ctypes binding of libq4.so (argument marshalling only).

Every function here takes torch device tensors, checks their dtypes and
shapes, passes raw device pointers and the current HIP stream to the C ABI
declared in include/q4.h, and raises if the library returns an error. No
arithmetic of the method happens here; there is no CPU fallback: without the
built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4.so")

Q4_DT_F32, Q4_DT_BF16 = 0, 1
Q4_FMT_Q4_0, Q4_FMT_AFFINE = 0, 1
Q4_PATH_GEMV, Q4_PATH_GEMM, Q4_PATH_SMALL = 0, 1, 2
Q4K_BLOCK_BYTES = 144

EXPORTS = ("q4_quantize_act", "q4_gemv", "q4_gemv_fused", "q4_gemm", "q4_debug_partials", "q4k_gemv", "q4k_gemm",
           "q4_quantize_weights", "q4k_quantize_weights", "q4_status_string", "q4_packed_bytes", "q4_pack_weights",
           "q4_gemm_packed_work_bytes", "q4_gemm_packed", "q4_backward_work_bytes", "q4k_gemm_backward",
           "q4_gemm_backward", "q4_measure_empty", "q4_measure_stream_read", "q4_debug_partials_fused",
           "q4k_gemm_backward_noalloc", "q4k_gemm_work_bytes", "q4k_gemm_work")
_SIZE_T_FUNCS = ("q4_packed_bytes", "q4_gemm_packed_work_bytes", "q4_backward_work_bytes", "q4k_gemm_work_bytes")


class Q4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libq4.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with block_quantized_bit_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int
        L.q4_status_string.restype = ctypes.c_char_p
        L.q4_status_string.argtypes = [I]
        L.q4_quantize_act.argtypes = [I, I, I, I, P, P, P, P, P]
        L.q4_gemv.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P]
        L.q4_gemm.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P]
        L.q4_gemv_fused.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P]
        L.q4_debug_partials.argtypes = [I, I, I, I, I, I, I, P, P, P, I, I, P, P]
        L.q4k_gemv.argtypes = [I, I, I, P, P, P, P]
        L.q4k_gemm.argtypes = [I, I, I, P, P, P, P]
        L.q4_quantize_weights.argtypes = [I, I, I, I, I, I, P, P, P, P, P]
        L.q4k_quantize_weights.argtypes = [I, I, P, P, P]
        L.q4_packed_bytes.argtypes = [I, I, I, I]
        L.q4_pack_weights.argtypes = [I, I, I, I, I, P, P, P, P, P]
        L.q4_gemm_packed_work_bytes.argtypes = [I, I, I]
        L.q4_gemm_packed.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P]
        L.q4_backward_work_bytes.argtypes = [I, I, I]
        L.q4k_gemm_backward.argtypes = [I, I, I, P, P, P, P, P]
        L.q4_gemm_backward.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P]
        L.q4_debug_partials_fused.argtypes = [I, I, I, I, I, I, P, P, P, P]
        L.q4k_gemm_backward_noalloc.argtypes = [I, I, I, P, P, P, P]
        L.q4k_gemm_work_bytes.argtypes = [I, I]
        L.q4k_gemm_work.argtypes = [I, I, I, P, P, P, P, P]
        L.q4_measure_empty.argtypes = [I, I, P]
        L.q4_measure_stream_read.argtypes = [P, ctypes.c_size_t, I, I, ctypes.c_uint32, P, P]
        for name in EXPORTS:
            if name in _SIZE_T_FUNCS:
                getattr(L, name).restype = ctypes.c_size_t
            elif name != "q4_status_string":
                getattr(L, name).restype = I
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().q4_status_string(int(status)).decode()


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int, what: str):
    if rc != 0:
        raise Q4Error(rc, what)


def _xdtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return Q4_DT_F32
    if t.dtype == torch.bfloat16:
        return Q4_DT_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _fmt(fmt: str) -> int:
    if fmt == "q4_0":
        return Q4_FMT_Q4_0
    if fmt == "affine":
        return Q4_FMT_AFFINE
    raise ValueError(f"unknown format {fmt!r}")


# ---- entry points --------------------------------------------------------------

def quantize_act(x: torch.Tensor, bs: int, out=None, stream=None):
    """x [M][K] float32 or bfloat16 -> (xq int8 [M][K], xs float32 [M][K/bs], xsum int32 [M][K/bs])."""
    M, K = x.shape
    if out is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
        xs = torch.empty((M, K // bs), dtype=torch.float32, device=x.device)
        xsum = torch.empty((M, K // bs), dtype=torch.int32, device=x.device)
    else:
        xq, xs, xsum = out
    _check(lib().q4_quantize_act(M, K, bs, _xdtype(x), _ptr(x), _ptr(xq), _ptr(xs), _ptr(xsum), _stream(stream)),
           "q4_quantize_act")
    return xq, xs, xsum


def code_shape(N: int, K: int, bits: int):
    """Shape of a code array: [N][K/2] (4 bits), [N][K] (8 bits), or a flat N*K*3/4 bytes (6 bits: the 4-bit
    nibble layout of the low bits, then the plane of the high 2 bits; layout in include/q4.h)."""
    return {4: (N, K // 2), 8: (N, K), 6: (N * K * 3 // 4,)}[bits]


def _matmul(entry: str, M: int, fmt: str, bs: int, wq, wscale, wbias, xq, xs, xsum, y, bits, stream):
    K = xq.shape[1]
    N = wscale.shape[0]
    if wq.numel() * 8 != N * K * bits:
        raise ValueError("wq does not hold N*K codes of the given width")
    _check(getattr(lib(), entry)(M, K, N, bs, _fmt(fmt), bits, _ptr(wq), _ptr(wscale), _ptr(wbias), _ptr(xq),
                                 _ptr(xs), _ptr(xsum), _ptr(y), _stream(stream)), entry)
    return y


def gemv(fmt: str, bs: int, wq, wscale, wbias, xq, xs, xsum, y=None, bits: int = 4, stream=None):
    """Decode GEMV (xq is [1][K]) -> y float32 [1][N]."""
    if y is None:
        y = torch.empty((xq.shape[0], wscale.shape[0]), dtype=torch.float32, device=wq.device)
    return _matmul("q4_gemv", xq.shape[0], fmt, bs, wq, wscale, wbias, xq, xs, xsum, y, bits, stream)


def gemv_fused(fmt: str, bs: int, x, wq, wscale, wbias, y=None, act_out=None, bits: int = 4, stream=None):
    """Fused decode step: quantize x [1][K] and run the GEMV in one launch -> y float32 [1][N].
    act_out = (xq, xs, xsum) receives the activation codes the kernel used."""
    N, Kh = wq.shape
    K = 2 * Kh
    if x.shape[1] != K:
        raise ValueError("x and wq disagree on K")
    if y is None:
        y = torch.empty((x.shape[0], N), dtype=torch.float32, device=wq.device)
    xq, xs, xsum = act_out if act_out is not None else (None, None, None)
    _check(lib().q4_gemv_fused(x.shape[0], K, N, bs, _fmt(fmt), bits, _xdtype(x), _ptr(x), _ptr(wq), _ptr(wscale),
                               _ptr(wbias), _ptr(y), _ptr(xq), _ptr(xs), _ptr(xsum), _stream(stream)),
           "q4_gemv_fused")
    return y


def gemm(fmt: str, bs: int, wq, wscale, wbias, xq, xs, xsum, y=None, bits: int = 4, stream=None):
    """Prefill GEMM (xq is [M][K]) -> y float32 [M][N]."""
    if y is None:
        y = torch.empty((xq.shape[0], wscale.shape[0]), dtype=torch.float32, device=wq.device)
    return _matmul("q4_gemm", xq.shape[0], fmt, bs, wq, wscale, wbias, xq, xs, xsum, y, bits, stream)


def debug_partials(path: str, fmt: str, bs: int, wq, xq, xsum, m0: int = 0, m1: int | None = None, out=None,
                   bits: int = 4, stream=None):
    """Exact per-block int32 partials [(m1-m0)][N][K/bs] from the GEMV ('gemv'), tiled GEMM ('gemm') or
    few-row GEMM ('small') kernel."""
    M, K = xq.shape
    N = wq.numel() * 8 // (K * bits)
    m1 = M if m1 is None else m1
    if out is None:
        out = torch.empty((max(m1 - m0, 1), N, K // bs), dtype=torch.int32, device=wq.device)
    p = {"gemv": Q4_PATH_GEMV, "gemm": Q4_PATH_GEMM, "small": Q4_PATH_SMALL}[path]
    _check(lib().q4_debug_partials(p, M, K, N, bs, _fmt(fmt), bits, _ptr(wq), _ptr(xq), _ptr(xsum), m0, m1,
                                   _ptr(out), _stream(stream)), "q4_debug_partials")
    return out


def debug_partials_fused(fmt: str, bs: int, x, wq, out=None, bits: int = 4, stream=None):
    """Exact per-block int32 partials [N][K/bs] of the fused decode kernel (it quantizes x [1][K] itself)."""
    K = x.shape[1]
    N = wq.numel() * 8 // (K * bits)
    if out is None:
        out = torch.empty((N, K // bs), dtype=torch.int32, device=wq.device)
    _check(lib().q4_debug_partials_fused(K, N, bs, _fmt(fmt), bits, _xdtype(x), _ptr(x), _ptr(wq), _ptr(out),
                                         _stream(stream)), "q4_debug_partials_fused")
    return out


def packed_bytes(K: int, N: int, bs: int, fmt: str) -> int:
    """Size of the packed weight buffer (0 if the arguments are invalid)."""
    return int(lib().q4_packed_bytes(K, N, bs, _fmt(fmt)))


def pack_weights(fmt: str, bs: int, wq, wscale, wbias, bits: int = 4, stream=None):
    """(wq [N][K/2], wscale, wbias) -> packed uint8 buffer for gemm_packed (layout in include/q4.h)."""
    N, Kh = wq.shape
    K = 2 * Kh
    nbytes = packed_bytes(K, N, bs, fmt)
    if nbytes == 0:
        raise ValueError("invalid shape or format for packing")
    packed = torch.empty(nbytes, dtype=torch.uint8, device=wq.device)
    _check(lib().q4_pack_weights(N, K, bs, _fmt(fmt), bits, _ptr(wq), _ptr(wscale), _ptr(wbias), _ptr(packed),
                                 _stream(stream)), "q4_pack_weights")
    return packed


def gemm_packed(fmt: str, bs: int, x, packed, N: int, y=None, work=None, bits: int = 4, stream=None):
    """Fused quantize + GEMM on packed weights: x [M][K] float32 / bfloat16 -> y float32 [M][N].
    Returns (y, (xq, xs_gm, xsum_gm)): the activation codes the call used, as views of its workspace
    (xs and xsum group-major, [K/bs][M])."""
    M, K = x.shape
    wbytes = int(lib().q4_gemm_packed_work_bytes(M, K, bs))
    if wbytes == 0:
        raise ValueError("invalid shape for the packed GEMM")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if work is None:
        work = torch.empty(wbytes, dtype=torch.uint8, device=x.device)
    elif work.numel() < wbytes:
        raise ValueError(f"workspace needs {wbytes} bytes")
    _check(lib().q4_gemm_packed(M, K, N, bs, _fmt(fmt), bits, _xdtype(x), _ptr(x), _ptr(packed), _ptr(y),
                                _ptr(work), _stream(stream)), "q4_gemm_packed")
    a = (M * K + 255) // 256 * 256
    g = K // bs
    sb = (M * g * 4 + 255) // 256 * 256
    xq = work[:M * K].view(M, K).view(torch.int8)
    xs = work[a:a + M * g * 4].view(torch.float32).view(g, M)
    xsum = work[a + sb:a + sb + M * g * 4].view(torch.int32).view(g, M)
    return y, (xq, xs, xsum)


def _backward_work(M: int, K: int, N: int, work, device):
    nbytes = int(lib().q4_backward_work_bytes(M, K, N))
    if nbytes == 0:
        raise ValueError("invalid shape for the input gradient (K must be a multiple of 256)")
    if work is None:
        return torch.empty(nbytes // 4, dtype=torch.float32, device=device)
    if work.numel() * work.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return work


def q4k_gemm_backward(blocks, dy, K: int, dx=None, work=None, stream=None):
    """Input gradient with frozen Q4_K weights: dy [M][N] -> dx [M][K] = dy . dequant(W)."""
    M, N = dy.shape
    if dx is None:
        dx = torch.empty((M, K), dtype=torch.float32, device=dy.device)
    work = _backward_work(M, K, N, work, dy.device)
    _check(lib().q4k_gemm_backward(M, K, N, _ptr(blocks), _ptr(dy), _ptr(dx), _ptr(work), _stream(stream)),
           "q4k_gemm_backward")
    return dx


def q4k_gemm_backward_noalloc(blocks, dy, K: int, dx, stream=None):
    """q4k_gemm_backward with the library's static per-device scratch buffer instead of a workspace (the
    call allocates nothing; dx [M][K] float32 must be given). Calls that overlap on one GPU race."""
    M, N = dy.shape
    _check(lib().q4k_gemm_backward_noalloc(M, K, N, _ptr(blocks), _ptr(dy), _ptr(dx), _stream(stream)),
           "q4k_gemm_backward_noalloc")
    return dx


def gemm_backward(fmt: str, bs: int, wq, wscale, wbias, dy, dx=None, work=None, bits: int = 4, stream=None):
    """Input gradient with frozen Q4_0 / affine weights: dy [M][N] -> dx [M][K] = dy . dequant(W)."""
    M, N = dy.shape
    K = 2 * wq.shape[1]
    if dx is None:
        dx = torch.empty((M, K), dtype=torch.float32, device=dy.device)
    work = _backward_work(M, K, N, work, dy.device)
    _check(lib().q4_gemm_backward(M, K, N, bs, _fmt(fmt), bits, _ptr(wq), _ptr(wscale), _ptr(wbias), _ptr(dy),
                                  _ptr(dx), _ptr(work), _stream(stream)), "q4_gemm_backward")
    return dx


def q4k_gemv(blocks, x, N: int, y=None, stream=None):
    M, K = x.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check(lib().q4k_gemv(M, K, N, _ptr(blocks), _ptr(x), _ptr(y), _stream(stream)), "q4k_gemv")
    return y


def q4k_gemm(blocks, x, N: int, y=None, stream=None):
    M, K = x.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check(lib().q4k_gemm(M, K, N, _ptr(blocks), _ptr(x), _ptr(y), _stream(stream)), "q4k_gemm")
    return y


def q4k_gemm_work(blocks, x, N: int, y=None, work=None, stream=None):
    """q4k_gemm with the activations split once per call into a workspace (two launches)."""
    M, K = x.shape
    nbytes = int(lib().q4k_gemm_work_bytes(M, K))
    if nbytes == 0:
        raise ValueError("invalid shape for the Q4_K GEMM (K must be a multiple of 256)")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if work is None:
        work = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    elif work.numel() * work.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    _check(lib().q4k_gemm_work(M, K, N, _ptr(blocks), _ptr(x), _ptr(y), _ptr(work), _stream(stream)),
           "q4k_gemm_work")
    return y


def quantize_weights(w: torch.Tensor, fmt: str, bs: int, bits: int = 4, stream=None):
    """w [N][K] float32 or bfloat16 -> (wq uint8 codes (code_shape), wscale, wbias) with fp16 (Q4_0) or bf16
    (affine) scales; affine codes may be 4, 6 or 8 bits wide."""
    N, K = w.shape
    f = _fmt(fmt)
    wq = torch.empty(code_shape(N, K, bits) if bits in (4, 6, 8) else (N, K // 2), dtype=torch.uint8,
                     device=w.device)
    sdt = torch.float16 if f == Q4_FMT_Q4_0 else torch.bfloat16
    ws = torch.empty((N, K // bs), dtype=sdt, device=w.device)
    wb = None if f == Q4_FMT_Q4_0 else torch.empty((N, K // bs), dtype=sdt, device=w.device)
    _check(lib().q4_quantize_weights(N, K, bs, f, bits, _xdtype(w), _ptr(w), _ptr(wq), _ptr(ws), _ptr(wb),
                                     _stream(stream)), "q4_quantize_weights")
    return wq, ws, wb


def q4k_quantize_weights(w: torch.Tensor, stream=None):
    """w [N][K] float32 -> Q4_K blocks uint8 [N][K/256*144]."""
    N, K = w.shape
    blocks = torch.empty((N, K // 256 * Q4K_BLOCK_BYTES), dtype=torch.uint8, device=w.device)
    _check(lib().q4k_quantize_weights(N, K, _ptr(w), _ptr(blocks), _stream(stream)), "q4k_quantize_weights")
    return blocks


# ---- measurement kernels (include/q4_measure.h) ------------------------------------

def measure_empty(grid: int, block: int, stream=None):
    """One empty kernel of the given launch shape (the dispatch floor)."""
    _check(lib().q4_measure_empty(grid, block, _stream(stream)), "q4_measure_empty")


def measure_stream_read(buf: torch.Tensor, grid: int, block: int, sink: torch.Tensor, key: int = 0x9E3779B9,
                        stream=None):
    """Read every byte of buf once (128-bit non-temporal loads); sink (one int32) is written only if the XOR of
    the data equals key."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().q4_measure_stream_read(_ptr(buf), nbytes, grid, block, key, _ptr(sink), _stream(stream)),
           "q4_measure_stream_read")
