"""Pins of the oracle's affine 6- and 8-bit weights (MLX PR #4802: the int8
x int8 kernel serves 4, 6 and 8 bit weights with group size 64 or more).

The code layouts are this project's own (written out in tests/_decode.py and
include/q4.h); the pins decode them with numpy independently of the oracle,
check the quantizer's round trip and code range, the integer partials and the
float result by brute force, and the error of the whole scheme against the
levels the page publishes for 6 and 8 bits.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from tests import _decode as dec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mlx_affine_accuracy.json")
FMT_AFFINE = oracle.FMT_AFFINE


def _w(N, K, seed, scale=0.02):
    return synth.bf16_bits((scale * np.random.default_rng(seed).standard_normal((N, K))).astype(np.float32))


@pytest.mark.parametrize("bits", [6, 8])
@pytest.mark.parametrize("g", [64, 128])
def test_quantizer_roundtrip_and_code_range(bits, g):
    N, K = 7, 512
    wb16 = _w(N, K, bits * g)
    wq, ws, wb = oracle.quantize_affine(wb16, g, bits)
    assert wq.size == N * K * bits // 8
    codes = dec.codes_from_bits(wq, N, K, bits)
    assert codes.min() >= 0 and codes.max() <= 2 ** bits - 1
    assert codes.max() == 2 ** bits - 1          # the group maximum reaches the top code somewhere
    s = np.repeat(dec.bf16(ws), g, axis=1)
    b = np.repeat(dec.bf16(wb), g, axis=1)
    w = dec.bf16(wb16)
    what = s * codes + b
    # rounding to the nearest code, computed with the rounded scale and bias
    assert np.all(np.abs(what - w) <= s / 2 * (1 + 2 ** -7) + np.abs(b) * 2 ** -8)


@pytest.mark.parametrize("bits", [6, 8])
def test_code_accessor_matches_decoder(bits):
    N, K = 5, 256
    wq, _, _ = oracle.quantize_affine(_w(N, K, 3), 64, bits)
    codes = dec.codes_from_bits(wq, N, K, bits)
    for n, k in [(0, 0), (0, 15), (0, 16), (1, 31), (2, 32), (3, 100), (4, 255)]:
        assert oracle.get_code(wq, K, n, k, bits=bits, N=N) == codes[n, k]


def test_six_bit_layout_by_hand():
    # one row, one 32-code block with code c = c: low nibbles c & 15, high bits c >> 4
    N, K = 1, 32
    codes = np.arange(32)
    lo = dec.planes_from_codes((codes & 15)[None, :])
    hp = np.zeros(8, dtype=np.uint8)
    for j in range(32):
        h, c = j // 16, j % 16
        hp[4 * h + c % 4] |= ((codes[j] >> 4) & 3) << (2 * (c // 4))
    wq = np.concatenate([lo.reshape(-1), hp])
    assert np.array_equal(dec.codes_from_bits(wq, N, K, 6)[0], codes)
    assert [oracle.get_code(wq, K, 0, k, bits=6, N=1) for k in range(32)] == list(range(32))
    # code 63 everywhere: every bit set
    wq63 = np.full(24, 0xFF, dtype=np.uint8)
    assert np.all(dec.codes_from_bits(wq63, 1, 32, 6) == 63)


def test_constant_group_gives_zero_scale():
    w = np.full((1, 64), 0x3F80, dtype=np.uint16)   # bf16 1.0
    wq, ws, wb = oracle.quantize_affine(w, 64, 8)
    assert ws[0, 0] == 0 and wb[0, 0] == 0x3F80 and np.all(wq == 0)


@pytest.mark.parametrize("bits", [6, 8])
@pytest.mark.parametrize("M,K,N,g", [(1, 64, 1, 64), (3, 256, 5, 64), (2, 384, 4, 128)])
def test_brute_force_dequant_matmul(bits, M, K, N, g):
    rng = np.random.default_rng(M + K + N + bits)
    x = rng.standard_normal((M, K)).astype(np.float32)
    wq, ws, wb = oracle.quantize_affine(_w(N, K, K + bits), g, bits)
    xq, xs, xsum = oracle.quantize_act(x, g)
    y = oracle.q4_gemm(wq, ws, wb, xq, xs, xsum, K, N, g, FMT_AFFINE, bits=bits)
    codes = dec.codes_from_bits(wq, N, K, bits)
    what = np.repeat(dec.bf16(ws), g, axis=1) * codes + np.repeat(dec.bf16(wb), g, axis=1)
    xhat = xq.astype(np.float64) * np.repeat(xs.astype(np.float64), g, axis=1)
    ref = xhat @ what.T
    terms = np.abs(xhat) @ np.abs(what).T
    assert np.all(np.abs(y - ref) <= np.abs(ref) * 2 ** -24 + 1e-12 * terms)
    p = oracle.q4_partials(wq, xq, K, N, g, FMT_AFFINE, bits=bits)
    brute = np.einsum("nbj,mbj->mnb", codes.reshape(N, -1, g), xq.astype(np.int64).reshape(M, -1, g))
    assert np.array_equal(p, brute)
    ys = oracle.q4_gemm_sample(wq, ws, wb, xq, xs, xsum, K, N, g, FMT_AFFINE,
                               np.array([M - 1, 0]), np.array([0, N - 1]), bits=bits)
    assert ys[0] == y[M - 1, 0] and ys[1] == y[0, N - 1]


def test_bit_width_is_honoured():
    # the same bytes decoded at another width give another product: the width is not ignored
    N, K, g = 3, 128, 64
    wq8, ws, wb = oracle.quantize_affine(_w(N, K, 5), g, 8)
    xq, xs, xsum = oracle.quantize_act(np.random.default_rng(2).standard_normal((1, K)).astype(np.float32), g)
    p8 = oracle.q4_partials(wq8, xq, K, N, g, FMT_AFFINE, bits=8)
    p4 = oracle.q4_partials(wq8.reshape(-1)[:N * K // 2].reshape(N, K // 2), xq, K, N, g, FMT_AFFINE, bits=4)
    assert not np.array_equal(p8, p4)
    with pytest.raises(ValueError):
        oracle.q4_partials(wq8, xq, K, N, g, FMT_AFFINE, bits=5)
    with pytest.raises(ValueError):
        oracle.q4_partials(wq8, xq, K, N, 32, oracle.FMT_Q4_0, bits=8)   # Q4_0 is 4-bit only


@pytest.mark.parametrize("bits,g,key", [(6, 64, "affine6_gs64"), (8, 64, "affine8_gs64"), (8, 128, "affine8_gs128")])
def test_quantization_quality_matches_published_level(bits, g, key):
    # 16 rows of the M=1024, K=N=4096 normal bf16 workload, as for 4 bits. At 6
    # and 8 bits the activation rounding is a visible share of the error, and
    # the page does not say how qqmm groups x; so the scheme's error must lie
    # between the page's weight-only level (quantized_matmul, bf16 x) and its
    # int8-x level (qqmm), within 5% either way. (At 4 bits the two columns
    # coincide and the 4-bit test pins the level itself.)
    gold = json.load(open(GOLDEN))
    hi, lo = gold["rel_rms_error"][key], gold["quantized_matmul_column"][key]
    wl = synth.workload("affine_g64_1024x4096x4096")
    xb = synth.gen.activations(wl, M=16)
    wb16 = synth.gen.weights(wl)
    xq, xs, xsum = oracle.quantize_act(xb, g)
    wq, ws, wb = oracle.quantize_affine(wb16, g, bits)
    y = oracle.q4_gemm(wq, ws, wb, xq, xs, xsum, 4096, 4096, g, FMT_AFFINE, bits=bits).astype(np.float64)
    exact = dec.bf16(xb) @ dec.bf16(wb16).T
    rel = np.sqrt(((y - exact) ** 2).mean()) / np.sqrt((exact ** 2).mean())
    assert 0.95 * lo <= rel <= 1.05 * hi, (rel, lo, hi)
