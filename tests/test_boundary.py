"""The C ABI without a GPU: the library loads, exports every function that
include/q4.h declares, and rejects invalid calls on the host with the
documented status before any device work (no compute call is made here).

The bit-width guard follows meTile PR #29 ("keep the four-bit guard that was
protecting us"): a four-bit-only decoder handed another width reads the data
wrongly without failing, so the guard is load-bearing and pinned by a test.
"""
import ctypes
import os
import re

import pytest

import block_quantized_bit_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, DIM, BLOCK, FORMAT, ALIGN, HIP, RANGE, SCRATCH = range(9)
# stand-ins for device pointers: never dereferenced, every call below fails validation first
A = 0x100000
MIS = 0x100001


def declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            names |= set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(q4k?_\w+)\(", text, flags=re.M))
    return sorted(names)


def test_library_exports_every_declared_function():
    L = q4.lib()
    names = declared_functions()
    assert len(names) == 23
    assert sorted(q4.EXPORTS) == names
    for name in names:
        assert getattr(L, name) is not None


def test_status_strings():
    assert q4.status_string(OK) == "ok"
    assert "4-bit" in q4.status_string(FORMAT)
    assert q4.status_string(99) == "unknown status"


def gemm_args(**kw):
    a = dict(M=4, K=128, N=8, bs=32, fmt=0, bits=4, wq=A, ws=A, wb=None, xq=A, xs=A, xsum=A, y=A)
    a.update(kw)
    return (a["M"], a["K"], a["N"], a["bs"], a["fmt"], a["bits"], a["wq"], a["ws"], a["wb"], a["xq"], a["xs"],
            a["xsum"], a["y"], None)


@pytest.mark.parametrize("entry", ["q4_gemm", "q4_gemv"])
@pytest.mark.parametrize("kw,status", [
    (dict(bits=8), FORMAT), (dict(bits=2), FORMAT), (dict(bits=6), FORMAT),
    (dict(fmt=2), FORMAT),
    (dict(M=0), DIM), (dict(N=0), DIM), (dict(K=0), DIM), (dict(N=-3), DIM),
    (dict(K=100), BLOCK), (dict(bs=64), BLOCK), (dict(fmt=1, bs=32, wb=A), BLOCK),
    (dict(fmt=1, bs=256, K=256, wb=A), BLOCK), (dict(fmt=1, bs=64, K=96, wb=A), BLOCK),
    (dict(wq=None), NULL), (dict(ws=None), NULL), (dict(xq=None), NULL), (dict(xs=None), NULL),
    (dict(xsum=None), NULL), (dict(y=None), NULL), (dict(fmt=1, bs=64, wb=None), NULL),
    (dict(wq=MIS), ALIGN), (dict(xq=A + 8), ALIGN), (dict(y=MIS), ALIGN), (dict(xs=A + 2), ALIGN),
])
def test_matmul_validation(entry, kw, status):
    if entry == "q4_gemv" and "M" not in kw:
        kw = dict(kw, M=1)
    args = gemm_args(**kw)
    assert getattr(q4.lib(), entry)(*args) == status


@pytest.mark.parametrize("entry", ["q4_gemv", "q4_gemm"])
def test_code_width_guard(entry):
    # meTile PR #29: a decoder handed a width it does not decode must refuse it. Q4_0 is 4-bit only; the decode
    # GEMV decodes 4-bit codes only; widths other than 4, 6, 8 are refused everywhere (all before any launch).
    f = getattr(q4.lib(), entry)
    for bits in (2, 3, 5, 7, 16):
        assert f(*gemm_args(M=1, fmt=1, bs=64, wb=A, bits=bits)) == FORMAT
    assert f(*gemm_args(M=1, fmt=0, bits=8)) == FORMAT
    assert f(*gemm_args(M=1, fmt=0, bits=6)) == FORMAT
    if entry == "q4_gemv":
        assert f(*gemm_args(M=1, fmt=1, bs=64, wb=A, bits=8)) == FORMAT
        assert f(*gemm_args(M=1, fmt=1, bs=64, wb=A, bits=6)) == FORMAT


def test_gemv_requires_one_row():
    assert q4.lib().q4_gemv(*gemm_args(M=2)) == DIM


def test_gemv_fused_validation():
    f = q4.lib().q4_gemv_fused
    base = [1, 128, 8, 32, 0, 4, 0, A, A, A, None, A, None, None, None, None]
    assert f(*base[:5], 8, *base[6:]) == FORMAT             # bits
    args = list(base); args[6] = 5
    assert f(*args) == FORMAT                               # x dtype
    args = list(base); args[0] = 2
    assert f(*args) == DIM                                  # decode only
    args = list(base); args[1] = 65536
    assert f(*args) == DIM                                  # K beyond the LDS staging
    args = list(base); args[12] = A
    assert f(*args) == NULL                                 # partial set of code outputs
    args = list(base); args[7] = A + 4
    assert f(*args) == ALIGN
    args = list(base); args[12], args[13], args[14] = A + 8, A, A
    assert f(*args) == ALIGN


def test_quantize_act_validation():
    f = q4.lib().q4_quantize_act
    assert f(4, 128, 32, 0, None, A, A, A, None) == NULL
    assert f(4, 128, 32, 2, A, A, A, A, None) == FORMAT
    assert f(0, 128, 32, 0, A, A, A, A, None) == DIM
    assert f(4, 100, 32, 0, A, A, A, A, None) == BLOCK
    assert f(4, 128, 48, 0, A, A, A, A, None) == BLOCK
    assert f(4, 128, 32, 1, A + 4, A, A, A, None) == ALIGN
    assert f(4, 128, 32, 1, A, A + 1, A, A, None) == ALIGN


def test_debug_partials_validation():
    f = q4.lib().q4_debug_partials
    base = [1, 4, 128, 8, 32, 0, 4, A, A, A, 0, 4, A, None]
    assert f(*base[:6], 8, *base[7:]) == FORMAT          # bits
    assert f(3, *base[1:]) == FORMAT                     # path
    assert f(-1, *base[1:]) == FORMAT
    args = list(base); args[10], args[11] = 2, 2
    assert f(*args) == RANGE                             # empty range
    args = list(base); args[11] = 5
    assert f(*args) == RANGE                             # beyond M
    args = list(base); args[0] = 0
    assert f(*args) == RANGE                             # GEMV path needs one row
    args = list(base); args[12] = None
    assert f(*args) == NULL
    # few-row kernel: at most 64 rows
    big = [2, 80, 128, 8, 32, 0, 4, A, A, A, 0, 65, A, None]
    assert f(*big) == RANGE


def test_packed_sizes_and_validation():
    L = q4.lib()
    # 4096 x 14336, g128: 112 column tiles x 32 stages x 8 KB codes, 112 x 32 x 128 bf16 scales and biases
    assert L.q4_packed_bytes(4096, 14336, 128, 1) == 112 * 32 * 8192 + 2 * 112 * 32 * 256
    # ragged: N = 130 -> 2 tiles, K = 160 -> 2 stages, 5 groups of 32
    assert L.q4_packed_bytes(160, 130, 32, 0) == 2 * 2 * 8192 + 2 * 5 * 256
    assert L.q4_packed_bytes(160, 130, 32, 2) == 0
    assert L.q4_packed_bytes(100, 130, 32, 0) == 0
    assert L.q4_packed_bytes(160, 0, 32, 0) == 0
    assert L.q4_gemm_packed_work_bytes(3, 160, 32) == 512 + 2 * 256
    assert L.q4_gemm_packed_work_bytes(3, 100, 32) == 0
    p = L.q4_pack_weights
    assert p(8, 128, 32, 0, 8, A, A, None, A, None) == FORMAT
    assert p(8, 128, 64, 1, 4, A, A, None, A, None) == NULL
    assert p(8, 128, 32, 0, 4, A, A, None, None, None) == NULL
    assert p(8, 128, 32, 0, 4, A, A, None, A + 8, None) == ALIGN
    assert p(8, 100, 32, 0, 4, A, A, None, A, None) == BLOCK
    g = L.q4_gemm_packed
    base = [4, 128, 8, 32, 0, 4, 0, A, A, A, A, None]
    args = list(base); args[6] = 5
    assert g(*args) == FORMAT
    args = list(base); args[5] = 6
    assert g(*args) == FORMAT
    args = list(base); args[10] = None
    assert g(*args) == NULL
    args = list(base); args[10] = A + 4
    assert g(*args) == ALIGN
    args = list(base); args[0] = 0
    assert g(*args) == DIM


def test_backward_validation():
    L = q4.lib()
    assert L.q4_backward_work_bytes(1, 4096, 14336) > 0
    assert L.q4_backward_work_bytes(1, 4000, 14336) == 0
    assert L.q4_backward_work_bytes(0, 4096, 8) == 0
    f = L.q4k_gemm_backward
    assert f(1, 512, 8, None, A, A, A, None) == NULL
    assert f(1, 500, 8, A, A, A, A, None) == BLOCK
    assert f(1, 512, 0, A, A, A, A, None) == DIM
    assert f(1, 512, 8, A + 8, A, A, A, None) == ALIGN
    assert f(1, 512, 8, A, A, A, None, None) == NULL
    g = L.q4_gemm_backward
    assert g(1, 512, 8, 32, 0, 8, A, A, None, A, A, A, None) == FORMAT
    assert g(1, 512, 8, 32, 3, 4, A, A, None, A, A, A, None) == FORMAT
    assert g(1, 512, 8, 64, 0, 4, A, A, None, A, A, A, None) == BLOCK
    assert g(1, 96, 8, 32, 0, 4, A, A, None, A, A, A, None) == BLOCK          # K not a multiple of 256
    assert g(1, 512, 8, 64, 1, 4, A, A, None, A, A, A, None) == NULL          # affine needs biases
    assert g(1, 512, 8, 32, 0, 4, A, A + 1, None, A, A, A, None) == ALIGN


def test_q4k_validation():
    for f in (q4.lib().q4k_gemv, q4.lib().q4k_gemm):
        assert f(1, 4096, 8, None, A, A, None) == NULL
        assert f(1, 4000, 8, A, A, A, None) == BLOCK
        assert f(1, 4096, 0, A, A, A, None) == DIM
        assert f(1, 4096, 8, A + 8, A, A, None) == ALIGN
    assert q4.lib().q4k_gemv(2, 4096, 8, A, A, A, None) == DIM
    # 32-bit buffer offsets: the weight blocks and x must each stay below 2^31 bytes
    assert q4.lib().q4k_gemv(1, 32768, 460000, A, A, A, None) == DIM      # 460000 * 128 * 144 bytes
    assert q4.lib().q4k_gemm(16, 32768, 460000, A, A, A, None) == DIM
    assert q4.lib().q4k_gemm(20000, 32768, 8, A, A, A, None) == DIM       # 4 * M * K bytes of x


def test_weight_quantizer_validation():
    f = q4.lib().q4_quantize_weights
    assert f(8, 128, 32, 0, 8, 0, A, A, A, None, None) == FORMAT      # Q4_0 is 4-bit only
    assert f(8, 128, 64, 1, 5, 0, A, A, A, None, None) == FORMAT      # affine: 4, 6 or 8 bits
    assert f(8, 128, 32, 0, 4, 3, A, A, A, None, None) == FORMAT
    assert f(8, 128, 64, 1, 4, 1, A, A, A, None, None) == NULL
    assert f(8, 100, 32, 0, 4, 0, A, A, A, None, None) == BLOCK
    assert f(8, 128, 32, 0, 4, 0, A, A + 4, A, None, None) == ALIGN
    g = q4.lib().q4k_quantize_weights
    assert g(8, 300, A, A, None) == BLOCK
    assert g(8, 256, A, A + 16 + 8, None) == ALIGN


def test_binding_raises_with_message():
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only check")
    with pytest.raises(ValueError):
        q4.quantize_act(torch.zeros(2, 64), 32)   # host tensor: refused before any call


def test_noalloc_backward_validation():
    # shapes whose partial sums exceed the static 16 MiB buffer are refused before any launch
    f = q4.lib().q4k_gemm_backward_noalloc
    need = q4.lib().q4_backward_work_bytes(512, 14336, 4096)
    assert need > 16 << 20
    assert f(512, 14336, 4096, A, A, A, None) == SCRATCH
    assert f(0, 256, 8, A, A, A, None) == DIM
    assert f(4, 100, 8, A, A, A, None) == BLOCK
    assert f(4, 256, 8, None, A, A, None) == NULL
    assert f(4, 256, 8, MIS, A, A, None) == ALIGN
    assert "16 MiB" in q4.status_string(SCRATCH)


def test_q4k_gemm_work_validation():
    f = q4.lib().q4k_gemm_work
    assert q4.lib().q4k_gemm_work_bytes(16, 4096) == 16 * 1060 * 16
    assert q4.lib().q4k_gemm_work_bytes(17, 512) == 2 * 2 * 1060 * 16
    assert q4.lib().q4k_gemm_work_bytes(4, 100) == 0 and q4.lib().q4k_gemm_work_bytes(0, 256) == 0
    assert f(16, 256, 8, A, A, A, None, None) == NULL
    assert f(0, 256, 8, A, A, A, A, None) == DIM
    assert f(16, 300, 8, A, A, A, A, None) == BLOCK
    assert f(16, 256, 8, A, A, A, MIS, None) == ALIGN


def test_offset_limits_of_the_w4a8_entry_points():
    # Buffer loads address each operand with 32-bit byte offsets: weight codes of N * K * bits / 8 bytes and
    # activation codes of M * K bytes must each stay below 2^31, else Q4_ERR_DIM before any launch.
    L = q4.lib()
    for entry in (L.q4_gemm, L.q4_gemv):
        assert entry(*gemm_args(M=1, K=65536, N=65536)) == DIM                 # 2^31 bytes of 4-bit codes
    assert L.q4_gemm(*gemm_args(M=1, K=65536, N=43691, fmt=1, bs=64, wb=A, bits=6)) == DIM
    assert L.q4_gemm(*gemm_args(M=1, K=65536, N=32768, fmt=1, bs=64, wb=A, bits=8)) == DIM
    assert L.q4_gemm(*gemm_args(M=32768, K=65536, N=8)) == DIM                # 2^31 bytes of activation codes
    f = L.q4_debug_partials
    assert f(1, 1, 65536, 65536, 32, 0, 4, A, A, A, 0, 1, A, None) == DIM
    assert f(1, 32768, 65536, 8, 32, 0, 4, A, A, A, 0, 32768, A, None) == DIM
