"""Pins of the oracle's Q4_K super-block format and fused-dequant result.

C-Kernel-Engine gemm_kernels_q4k.c page: Q4_K holds 256 weights in 4.5 bits
per weight (144 bytes: fp16 d, fp16 dmin, twelve bytes of 6-bit sub-block
scales and mins, 128 bytes of codes). gemv_q4_k_ref maps chunk c of 64 weights
to qs[32c .. 32c+31], low nibbles first (sub-block 2c) then high nibbles
(sub-block 2c+1), and dequantizes as w = d * sc * q - dmin * m. gemm_q4_k_ref
computes the GEMM as one GEMV per activation row.
"""
import numpy as np
import pytest

import synth
from tests import _decode as dec


def _block(d=0x3C00, dmin=0, sc=None, mn=None, qs=None, orc=None):
    sc = np.ones(8, np.uint8) if sc is None else np.asarray(sc, np.uint8)
    mn = np.zeros(8, np.uint8) if mn is None else np.asarray(mn, np.uint8)
    qs = np.zeros(128, np.uint8) if qs is None else np.asarray(qs, np.uint8)
    raw = np.zeros(144, np.uint8)
    raw[0:2] = np.array([d], np.uint16).view(np.uint8)
    raw[2:4] = np.array([dmin], np.uint16).view(np.uint8)
    raw[4:16] = orc.q4k_pack_scales(sc, mn)
    raw[16:] = qs
    return raw


def test_scale_packing_roundtrip_all_values(orc):
    rng = np.random.default_rng(0)
    for f in range(16):
        for v in range(64):
            vals = rng.integers(0, 64, 16)
            vals[f] = v
            b = orc.q4k_pack_scales(vals[:8], vals[8:])
            sc, mn = orc.q4k_unpack_scales(b)
            assert list(sc) + list(mn) == list(vals)
            isc, imn = dec.q4k_fields(b)
            assert list(isc) + list(imn) == list(vals)


def test_unit_block_sums_x(orc):
    x = np.random.default_rng(1).integers(-50, 50, (1, 256)).astype(np.float32)
    blk = _block(qs=np.full(128, 0x11), orc=orc)
    assert orc.q4k_gemv(blk, x, 256, 1)[0] == x.sum()


def test_min_only_block(orc):
    x = np.random.default_rng(2).integers(-50, 50, (1, 256)).astype(np.float32)
    blk = _block(dmin=0x3C00, sc=np.zeros(8), mn=np.ones(8), orc=orc)
    assert orc.q4k_gemv(blk, x, 256, 1)[0] == -x.sum()


@pytest.mark.parametrize("s", range(8))
def test_sub_block_scale_probe(orc, s):
    # only sub-block s has a scale: the result sums x over weights 32s..32s+31
    x = np.random.default_rng(3 + s).integers(-50, 50, (1, 256)).astype(np.float32)
    sc = np.zeros(8); sc[s] = 1
    blk = _block(sc=sc, qs=np.full(128, 0x11), orc=orc)
    assert orc.q4k_gemv(blk, x, 256, 1)[0] == x[0, 32 * s:32 * s + 32].sum()


@pytest.mark.parametrize("byte,high", [(0, False), (0, True), (31, True), (32, False), (77, True), (127, False)])
def test_code_map_probe(orc, byte, high):
    # one nonzero nibble selects one weight: low nibble of qs[32c + l] is
    # weight 64c + l, its high nibble is weight 64c + 32 + l
    x = np.arange(256, dtype=np.float32).reshape(1, 256) + 1
    qs = np.zeros(128, np.uint8)
    qs[byte] = 0x10 if high else 0x01
    blk = _block(qs=qs, orc=orc)
    c, l = divmod(byte, 32)
    k = 64 * c + l + (32 if high else 0)
    assert orc.q4k_gemv(blk, x, 256, 1)[0] == x[0, k]


def test_quantizer_roundtrip(orc):
    wl = synth.workload("q4_k_gemv_1x4096x14336")
    w = synth.gen.weights(wl, N=16, K=512)
    blocks = orc.quantize_q4k(w)
    what = orc.q4k_dequant(blocks, 16, 512)
    assert np.array_equal(what, dec.q4k_dequant(blocks, 16, 512))
    b = blocks.reshape(16, 2, 144)
    d = dec.f16(b[:, :, 0:2].copy().view(np.uint16))[..., 0]           # [16, 2]
    dmin = dec.f16(b[:, :, 2:4].copy().view(np.uint16))[..., 0]
    # grid -dmin*m + d*sc*q: half a step inside the range, plus the overshoot
    # left by rounding the sub-block scale (<= 15 d/2) and min (<= dmin/2)
    sc = np.array([[dec.q4k_fields(b[n, j, 4:16])[0] for j in range(2)] for n in range(16)])
    step = d[..., None] * sc                                  # [16, 2, 8]
    bound = np.repeat((step / 2 + 7.5 * d[..., None] + dmin[..., None] / 2).reshape(16, 16), 32, axis=1)
    assert np.all(np.abs(what - w) <= bound * (1 + 1e-9))
    rel = np.sqrt(((what - w) ** 2).mean() / (w.astype(np.float64) ** 2).mean())
    assert rel < 0.15


@pytest.mark.parametrize("M,K,N", [(1, 256, 3), (2, 512, 5), (4, 768, 2)])
def test_brute_force_and_gemm_is_rows_of_gemv(orc, M, K, N):
    rng = np.random.default_rng(M * K + N)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    blocks = orc.quantize_q4k(w)
    y = orc.q4k_gemm(blocks, x, K, N)
    for m in range(M):
        assert np.array_equal(y[m], orc.q4k_gemv(blocks, x[m], K, N))
    what = dec.q4k_dequant(blocks, N, K)
    ref = x.astype(np.float64) @ what.T
    terms = np.abs(x.astype(np.float64)) @ np.abs(what).T
    assert np.all(np.abs(y - ref) <= np.abs(ref) * 2 ** -24 + 1e-12 * terms)
    ms = np.array([M - 1, 0]); ns = np.array([0, N - 1])
    assert np.array_equal(orc.q4k_gemm_sample(blocks, x, K, N, ms, ns), y[ms, ns])
