"""Pins of the oracle's Q4_0 weight quantizer and W4A8 result.

tract PR #2432, section "The kernel": Q4_0 weights (4-bit codes, N x K, one
scale per 32-weight block) times int8 per-block activations; each block's
integer dot is exact and the per-block scale is applied afterwards in float,
giving an f32 output. Codes 0..15 mean d * (q - 8) with d = (signed extreme)/-8
stored as fp16 (the Q4_0 workload's description).
"""
import numpy as np
import pytest

import synth
from tests import _decode as dec

FMT_Q4_0 = 0
FMT_AFFINE = 1


def _hand_block():
    # w_j = (j - 16) / 4: extreme -4 at j = 0 -> d = 0.5 -> q = rne((j-16)/2) + 8,
    # ties to even, the +8 end clamped to 15 (worked by hand).
    w = ((np.arange(32) - 16) * 0.25).astype(np.float32)
    q = [0, 0, 1, 2, 2, 2, 3, 4, 4, 4, 5, 6, 6, 6, 7, 8,
         8, 8, 9, 10, 10, 10, 11, 12, 12, 12, 13, 14, 14, 14, 15, 15]
    return w, np.array(q)


def test_quantizer_hand_block(orc):
    w, q = _hand_block()
    wq, wd = orc.quantize_q4_0(w.reshape(1, 32))
    assert wd[0, 0] == 0x3800                      # fp16(0.5)
    assert np.array_equal(dec.codes_from_planes(wq, 32)[0], q)
    assert wq[0, 0] == (0 | (8 << 4)) and wq[0, 15] == (8 | (15 << 4))


def test_quantizer_roundtrip_and_extreme(orc):
    wl = synth.workload("q4_0_minilm_64x384x1536")
    w = synth.gen.weights(wl, N=64, K=384).astype(np.float64)
    wq, wd = orc.quantize_q4_0(w.astype(np.float32))
    q = dec.codes_from_planes(wq, 384)
    d = np.repeat(dec.f16(wd), 32, axis=1)
    what = d * (q - 8)
    err = np.abs(what - w)
    clamped = q == 15
    assert np.all(err[~clamped] <= np.abs(d[~clamped]) / 2 * (1 + 1e-6) + 1e-12)
    # the signed extreme of each block is code 0 and is reproduced to fp16 rounding of d
    wb = w.reshape(64, 12, 32)
    qb = q.reshape(64, 12, 32)
    i = np.argmax(np.abs(wb), axis=2)
    assert np.all(np.take_along_axis(qb, i[..., None], 2) == 0)
    db = dec.f16(wd)
    assert np.all(np.abs(-8 * db - np.take_along_axis(wb, i[..., None], 2)[..., 0])
                  <= np.abs(db) * 8 * 2 ** -11)


def test_quantizer_zero_block(orc):
    # 0 / -8 is -0.0 under IEEE 754, so the stored fp16 scale is 0x8000
    wq, wd = orc.quantize_q4_0(np.zeros((2, 64), dtype=np.float32))
    assert np.all(wd == 0x8000) and np.all(wq == 0x88)


def _random_case(M, K, N, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    return x, w


def test_all_codes_eight_gives_zero(orc):
    M, K, N = 3, 96, 5
    rng = np.random.default_rng(3)
    xq, xs, xsum = orc.quantize_act(rng.standard_normal((M, K)).astype(np.float32), 32)
    wq = np.full((N, K // 2), 0x88, dtype=np.uint8)
    wd = orc.f32_to_f16(rng.standard_normal((N, K // 32)).astype(np.float32))
    y = orc.q4_gemm(wq, wd, None, xq, xs, xsum, K, N, 32, FMT_Q4_0)
    assert np.all(y == 0)


def test_all_codes_zero_closed_form(orc):
    M, K, N = 2, 128, 3
    rng = np.random.default_rng(4)
    xq, xs, xsum = orc.quantize_act(rng.standard_normal((M, K)).astype(np.float32), 32)
    wq = np.zeros((N, K // 2), dtype=np.uint8)
    wd = orc.f32_to_f16(rng.standard_normal((N, K // 32)).astype(np.float32))
    y = orc.q4_gemm(wq, wd, None, xq, xs, xsum, K, N, 32, FMT_Q4_0)
    d = dec.f16(wd)
    expect = -8.0 * np.einsum("nb,mb,mb->mn", d, xs.astype(np.float64), xsum.astype(np.float64))
    assert np.array_equal(y, expect.astype(np.float32))


@pytest.mark.parametrize("j0,q", [(0, 0), (5, 15), (16, 3), (31, 9)])
def test_single_lane_scale_one(orc, j0, q):
    rng = np.random.default_rng(j0)
    xq = rng.integers(-127, 128, (1, 32)).astype(np.int8)
    xs = np.ones((1, 1), dtype=np.float32)
    xsum = xq.sum(axis=1, keepdims=True).astype(np.int32)
    codes = np.full((1, 32), 8)
    codes[0, j0] = q
    wq = dec.planes_from_codes(codes)
    wd = np.array([[0x3C00]], dtype=np.uint16)      # fp16(1.0)
    y = orc.q4_gemm(wq, wd, None, xq, xs, xsum, 32, 1, 32, FMT_Q4_0)
    assert y[0, 0] == (q - 8) * int(xq[0, j0])


def test_scale_one_sums_partials(orc):
    M, K, N = 3, 160, 4
    rng = np.random.default_rng(9)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    xs = np.ones((M, K // 32), dtype=np.float32)
    xsum = xq.reshape(M, K // 32, 32).astype(np.int32).sum(axis=2)
    codes = rng.integers(0, 16, (N, K))
    wq = dec.planes_from_codes(codes)
    wd = np.full((N, K // 32), 0x3C00, dtype=np.uint16)
    y = orc.q4_gemm(wq, wd, None, xq, xs, xsum, K, N, 32, FMT_Q4_0)
    expect = xq.astype(np.int64) @ (codes - 8).T
    assert np.array_equal(y, expect.astype(np.float32))


def test_partials_invariant_and_definition(orc):
    M, K, N = 4, 256, 6
    x, w = _random_case(M, K, N, 11)
    xq, xs, xsum = orc.quantize_act(x, 32)
    wq, wd = orc.quantize_q4_0(w)
    p0 = orc.q4_partials(wq, xq, K, N, 32, FMT_Q4_0)
    p1 = orc.q4_partials(wq, xq, K, N, 32, FMT_AFFINE)
    # P = sum q*xq - 8*xsum on every block
    assert np.array_equal(p0, p1 - 8 * xsum[:, None, :])
    # and P is sum (q-8)*xq by brute force
    q = dec.codes_from_planes(wq, K).reshape(N, K // 32, 32)
    xb = xq.astype(np.int64).reshape(M, K // 32, 32)
    brute = np.einsum("nbj,mbj->mnb", q - 8, xb)
    assert np.array_equal(p0, brute)
    # row ranges
    assert np.array_equal(orc.q4_partials(wq, xq, K, N, 32, FMT_Q4_0, 1, 3), p0[1:3])


@pytest.mark.parametrize("M,K,N", [(1, 32, 1), (2, 64, 8), (4, 96, 7), (3, 384, 5)])
def test_brute_force_dequant_matmul(orc, M, K, N):
    x, w = _random_case(M, K, N, M * 1000 + K + N)
    xq, xs, xsum = orc.quantize_act(x, 32)
    wq, wd = orc.quantize_q4_0(w)
    y = orc.q4_gemm(wq, wd, None, xq, xs, xsum, K, N, 32, FMT_Q4_0)
    what = np.repeat(dec.f16(wd), 32, axis=1) * (dec.codes_from_planes(wq, K) - 8)
    xhat = np.repeat(xs.astype(np.float64), 32, axis=1) * xq
    ref = xhat @ what.T
    terms = np.abs(xhat) @ np.abs(what).T
    assert np.all(np.abs(y - ref) <= np.abs(ref) * 2 ** -24 + 1e-12 * terms)
    # and the quantized product approximates the float product
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.sqrt(((y - exact) ** 2).sum() / (exact ** 2).sum()) < 0.2


def test_sample_matches_full(orc):
    M, K, N = 5, 128, 9
    x, w = _random_case(M, K, N, 21)
    xq, xs, xsum = orc.quantize_act(x, 32)
    wq, wd = orc.quantize_q4_0(w)
    y = orc.q4_gemm(wq, wd, None, xq, xs, xsum, K, N, 32, FMT_Q4_0)
    ms = np.array([0, 4, 2, 3]); ns = np.array([8, 0, 5, 5])
    ys = orc.q4_gemm_sample(wq, wd, None, xq, xs, xsum, K, N, 32, FMT_Q4_0, ms, ns)
    assert np.array_equal(ys, y[ms, ns])


def test_rejects_bad_block_size(orc):
    with pytest.raises(ValueError):
        orc.q4_partials(np.zeros((1, 32), np.uint8), np.zeros((1, 64), np.int8), 64, 1, 64, FMT_Q4_0)
