"""Pins of the oracle's affine 4-bit quantizer and W4A8 result.

MLX PR #4802: affine weights carry per-group scales and biases; x is quantized
to int8 and an int8 x int8 MMA runs on the original codes with the per-group
scale and bias applied in the kernel. The bias enters as bias * sum(x) over
the group; with int8 activations that sum is xs * sum(xq), so the result is
exactly dequant(W) . dequant(X). Section "Accuracy" gives the expected error
of the whole scheme against the float product.
"""
import json
import os

import numpy as np
import pytest

import synth
from tests import _decode as dec

FMT_AFFINE = 1
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mlx_affine_accuracy.json")


def test_quantizer_hand_group(orc):
    # min -1, max 0.875 -> scale (0.875 + 1)/15 = 0.125 and bias -1, both exact
    # in bf16; -0.9375 and -0.8125 sit on ties (0.5 and 1.5 steps) -> 0 and 2.
    codes = np.array([0, 15] + [(3 * j) % 16 for j in range(60)] + [0, 0])
    w = (-1.0 + 0.125 * codes).astype(np.float32)
    w[62] = -0.9375
    w[63] = -0.8125
    expect = codes.copy()
    expect[62], expect[63] = 0, 2
    wq, ws, wb = orc.quantize_affine(synth.bf16_bits(w.reshape(1, 64)), 64)
    assert ws[0, 0] == 0x3E00 and wb[0, 0] == 0xBF80    # bf16(0.125), bf16(-1.0)
    assert np.array_equal(dec.codes_from_planes(wq, 64)[0], expect)


def test_quantizer_constant_group(orc):
    w = np.full((1, 128), 0.03125, dtype=np.float32)
    wq, ws, wb = orc.quantize_affine(synth.bf16_bits(w), 128)
    assert ws[0, 0] == 0 and dec.bf16(wb)[0, 0] == 0.03125 and np.all(wq == 0)


@pytest.mark.parametrize("g", [64, 128])
def test_quantizer_roundtrip(orc, g):
    wl = synth.workload("affine_g64_1024x4096x4096")
    wb16 = synth.gen.weights(wl, N=32, K=512)
    w = dec.bf16(wb16)
    wq, ws, wb = orc.quantize_affine(wb16, g)
    q = dec.codes_from_planes(wq, 512)
    s = np.repeat(dec.bf16(ws), g, axis=1)
    b = np.repeat(dec.bf16(wb), g, axis=1)
    what = s * q + b
    rng_ = np.repeat(w.reshape(32, -1, g).max(2) - w.reshape(32, -1, g).min(2), g, axis=1)
    assert np.all(np.abs(what - w) <= s / 2 * (1 + 1e-6) + rng_ * 2 ** -7)
    assert np.array_equal(b, np.repeat(w.reshape(32, -1, g).min(2), g, axis=1))


def test_zero_scale_bias_only_closed_form(orc):
    M, K, N, g = 3, 256, 4, 128
    rng = np.random.default_rng(5)
    xq, xs, xsum = orc.quantize_act(rng.standard_normal((M, K)).astype(np.float32), g)
    wq = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    ws = np.zeros((N, K // g), dtype=np.uint16)
    wb = synth.bf16_bits(rng.standard_normal((N, K // g)).astype(np.float32))
    y = orc.q4_gemm(wq, ws, wb, xq, xs, xsum, K, N, g, FMT_AFFINE)
    expect = np.einsum("ng,mg,mg->mn", dec.bf16(wb), xs.astype(np.float64), xsum.astype(np.float64))
    assert np.array_equal(y, expect.astype(np.float32))


def test_scale_one_bias_zero(orc):
    M, K, N, g = 2, 128, 3, 64
    rng = np.random.default_rng(6)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    xs = np.ones((M, K // g), dtype=np.float32)
    xsum = xq.reshape(M, -1, g).astype(np.int32).sum(2)
    codes = rng.integers(0, 16, (N, K))
    wq = dec.planes_from_codes(codes)
    ws = np.full((N, K // g), 0x3F80, dtype=np.uint16)
    wb = np.zeros((N, K // g), dtype=np.uint16)
    y = orc.q4_gemm(wq, ws, wb, xq, xs, xsum, K, N, g, FMT_AFFINE)
    assert np.array_equal(y, (xq.astype(np.int64) @ codes.T).astype(np.float32))


@pytest.mark.parametrize("M,K,N,g", [(1, 64, 1, 64), (3, 256, 5, 64), (2, 384, 7, 128), (4, 512, 3, 128)])
def test_brute_force_dequant_matmul(orc, M, K, N, g):
    rng = np.random.default_rng(M + K + N + g)
    xb = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    wb16 = synth.bf16_bits((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    xq, xs, xsum = orc.quantize_act(xb, g)
    wq, ws, wb = orc.quantize_affine(wb16, g)
    y = orc.q4_gemm(wq, ws, wb, xq, xs, xsum, K, N, g, FMT_AFFINE)
    what = np.repeat(dec.bf16(ws), g, 1) * dec.codes_from_planes(wq, K) + np.repeat(dec.bf16(wb), g, 1)
    xhat = np.repeat(xs.astype(np.float64), g, 1) * xq
    ref = xhat @ what.T
    terms = np.abs(xhat) @ np.abs(what).T
    assert np.all(np.abs(y - ref) <= np.abs(ref) * 2 ** -24 + 1e-12 * terms)
    p = orc.q4_partials(wq, xq, K, N, g, FMT_AFFINE)
    brute = np.einsum("nbj,mbj->mnb", dec.codes_from_planes(wq, K).reshape(N, -1, g),
                      xq.astype(np.int64).reshape(M, -1, g))
    assert np.array_equal(p, brute)


@pytest.mark.parametrize("g,key", [(64, "affine4_gs64"), (128, "affine4_gs128")])
def test_quantization_quality_matches_published_level(orc, g, key):
    # A sample of 16 rows of the M=1024, K=N=4096 normal bf16 workload; the
    # error of the whole scheme relative to the float32 product should sit near
    # the published level (a nibble-order or bit-width bug gives O(1) error).
    ref = json.load(open(GOLDEN))["rel_rms_error"][key]
    wl = synth.workload("affine_g64_1024x4096x4096")
    xb = synth.gen.activations(wl, M=16)
    wb16 = synth.gen.weights(wl)
    xq, xs, xsum = orc.quantize_act(xb, g)
    wq, ws, wb = orc.quantize_affine(wb16, g)
    y = orc.q4_gemm(wq, ws, wb, xq, xs, xsum, 4096, 4096, g, FMT_AFFINE).astype(np.float64)
    exact = dec.bf16(xb) @ dec.bf16(wb16).T
    rel = np.sqrt(((y - exact) ** 2).mean()) / np.sqrt((exact ** 2).mean())
    assert abs(rel - ref) < 0.05 * ref, (rel, ref)
