"""Pins of the oracle's input gradient with frozen weights.

C-Kernel-Engine gemm_kernels_q4k.c, section "Backward Pass: Gradient w.r.t.
Input": dL/dX = W^T . dL/dY with the weights dequantized on the fly and no
weight gradient; the batched form is one such product per activation row.
With W [N][K] and dY [M][N] this is dX [M][K] = dY . dequant(W).

The pins do not reuse the oracle's arithmetic: the weights are decoded by the
independent numpy decoders of tests/_decode.py and multiplied with numpy; the
adjoint identity ties the backward to the oracle's own forward product; and
closed forms on hand-built blocks fix the code map and the sign conventions.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _decode


def _ulp_close(a, ref64):
    """a (float32) equals ref64 (float64) rounded to float32, within one unit in the last place."""
    r = ref64.astype(np.float32)
    return np.all(np.abs(a.astype(np.float64) - r.astype(np.float64)) <= np.spacing(np.abs(r)).astype(np.float64) + 1e-30)


def _q4k_case(N, K, seed):
    rng = np.random.default_rng(seed)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    return oracle.quantize_q4k(w)


@pytest.mark.parametrize("M,K,N", [(1, 256, 1), (3, 512, 37), (2, 768, 64)])
def test_q4k_backward_is_dy_times_decoded_weights(M, K, N):
    blocks = _q4k_case(N, K, M + K + N)
    dy = np.random.default_rng(7 * N).standard_normal((M, N)).astype(np.float32)
    ref = dy.astype(np.float64) @ _decode.q4k_dequant(blocks, N, K)
    dx = oracle.q4k_backward(blocks, dy, K, N)
    assert dx.shape == (M, K)
    assert _ulp_close(dx, ref)


def _w4_case(fmt, bs, N, K, seed):
    rng = np.random.default_rng(seed)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    if fmt == "q4_0":
        wq, wd = oracle.quantize_q4_0(w)
        codes = _decode.codes_from_planes(wq, K)
        d = np.repeat(_decode.f16(wd), 32, axis=1)
        return (wq, wd, None), d * (codes - 8)
    wq, ws, wb = oracle.quantize_affine(synth.bf16_bits(w), bs)
    codes = _decode.codes_from_planes(wq, K)
    return (wq, ws, wb), np.repeat(_decode.bf16(ws), bs, axis=1) * codes + np.repeat(_decode.bf16(wb), bs, axis=1)


@pytest.mark.parametrize("fmt,bs,M,K,N", [("q4_0", 32, 1, 32, 1), ("q4_0", 32, 3, 160, 33), ("affine", 64, 2, 192, 17),
                                          ("affine", 128, 4, 384, 9)])
def test_q4_backward_is_dy_times_decoded_weights(fmt, bs, M, K, N):
    wts, what = _w4_case(fmt, bs, N, K, 5 * K + N)
    dy = np.random.default_rng(K).standard_normal((M, N)).astype(np.float32)
    ref = dy.astype(np.float64) @ what
    f = oracle.FMT_Q4_0 if fmt == "q4_0" else oracle.FMT_AFFINE
    dx = oracle.q4_backward(*wts, dy, K, N, bs, f)
    assert _ulp_close(dx, ref)


def test_q4k_backward_is_adjoint_of_forward():
    # <dY, W x> = <W^T dY, x>: ties the backward's indexing to the forward product
    M, K, N = 3, 512, 45
    blocks = _q4k_case(N, K, 99)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((M, K)).astype(np.float32)
    dy = rng.standard_normal((M, N)).astype(np.float32)
    y = oracle.q4k_gemm(blocks, x, K, N)
    dx = oracle.q4k_backward(blocks, dy, K, N)
    lhs = float((dy.astype(np.float64) * y.astype(np.float64)).sum())
    rhs = float((dx.astype(np.float64) * x.astype(np.float64)).sum())
    assert abs(lhs - rhs) <= 1e-5 * (abs(lhs) + 1.0)


@pytest.mark.parametrize("fmt,bs", [("q4_0", 32), ("affine", 64), ("affine", 128)])
def test_q4_backward_is_adjoint_of_forward(fmt, bs):
    # the W4A8 forward computes dequant(W) . xhat with xhat = xs * xq exactly, so
    # <dY, y> = <dX, xhat> up to the float32 rounding of y and dx
    M, K, N = 2, 256, 40
    wts, _ = _w4_case(fmt, bs, N, K, 17)
    rng = np.random.default_rng(11)
    xq, xs, xsum = oracle.quantize_act(rng.standard_normal((M, K)).astype(np.float32), bs)
    xhat = xq.astype(np.float64) * np.repeat(xs.astype(np.float64), bs, axis=1)
    f = oracle.FMT_Q4_0 if fmt == "q4_0" else oracle.FMT_AFFINE
    y = oracle.q4_gemm(*wts, xq, xs, xsum, K, N, bs, f)
    dy = rng.standard_normal((M, N)).astype(np.float32)
    dx = oracle.q4_backward(*wts, dy, K, N, bs, f)
    lhs = float((dy.astype(np.float64) * y.astype(np.float64)).sum())
    rhs = float((dx.astype(np.float64) * xhat).sum())
    assert abs(lhs - rhs) <= 1e-5 * (abs(lhs) + 1.0)


def test_q4_0_code_eight_gives_zero_gradient():
    K, N = 64, 5
    wq = np.full((N, K // 2), 0x88, dtype=np.uint8)      # every code 8: d * (8 - 8) = 0
    wd = np.full((N, K // 32), 0x3C00, dtype=np.uint16)   # d = 1.0
    dy = np.random.default_rng(1).standard_normal((2, N)).astype(np.float32)
    assert np.all(oracle.q4_backward(wq, wd, None, dy, K, N, 32, oracle.FMT_Q4_0) == 0.0)


def test_affine_zero_scale_gives_bias_sums():
    # s = 0: every weight of group g equals its bias b[n, g]; dx[m, k] = sum_n dy[m, n] * b[n, g(k)]
    K, N, g = 128, 3, 64
    wq = np.random.default_rng(2).integers(0, 256, (N, K // 2), dtype=np.uint8)
    ws = np.zeros((N, K // g), dtype=np.uint16)
    b = np.array([[1.0, -2.0], [0.5, 4.0], [-1.0, 0.25]], dtype=np.float32)
    wb = (b.view(np.uint32) >> 16).astype(np.uint16)       # exact in bf16
    dy = np.array([[1.0, 2.0, 3.0]], dtype=np.float32)
    dx = oracle.q4_backward(wq, ws, wb, dy, K, N, g, oracle.FMT_AFFINE)
    expect = (dy @ b)[0]                                   # [1*1 + 2*0.5 + 3*-1, 1*-2 + 2*4 + 3*0.25]
    assert np.array_equal(dx[0, :64], np.full(64, expect[0], dtype=np.float32))
    assert np.array_equal(dx[0, 64:], np.full(64, expect[1], dtype=np.float32))


def _q4k_block(d=0x3C00, dmin=0, sc=(1,) * 8, mn=(0,) * 8, q=1):
    blk = np.zeros(144, dtype=np.uint8)
    blk[0:2] = np.array([d], dtype=np.uint16).view(np.uint8)
    blk[2:4] = np.array([dmin], dtype=np.uint16).view(np.uint8)
    blk[4:16] = oracle.q4k_pack_scales(np.array(sc, dtype=np.uint8), np.array(mn, dtype=np.uint8))
    blk[16:] = (q & 0xF) | ((q & 0xF) << 4)
    return blk


def test_q4k_unit_blocks_give_column_sums():
    # d = 1, dmin = 0, every sc = 1, every q = 1: every weight is 1, so dx[m, k] = sum_n dy[m, n]
    N, K = 4, 256
    blocks = np.stack([_q4k_block() for _ in range(N)])
    dy = np.array([[1.0, 2.0, -3.0, 5.0], [0.0, 1.0, 1.0, 1.0]], dtype=np.float32)
    dx = oracle.q4k_backward(blocks, dy, K, N)
    assert np.all(dx[0] == 5.0) and np.all(dx[1] == 3.0)


@pytest.mark.parametrize("s", range(8))
def test_q4k_sub_block_probe(s):
    # only sub-block s has sc = 1: the gradient is nonzero exactly on the 32 k of that sub-block
    sc = [0] * 8
    sc[s] = 1
    blocks = _q4k_block(sc=sc, q=3)[None, :]
    dx = oracle.q4k_backward(blocks, np.array([[2.0]], dtype=np.float32), 256, 1)[0]
    nz = np.nonzero(dx)[0]
    assert np.array_equal(nz, np.arange(32 * s, 32 * s + 32))
    assert np.all(dx[nz] == 6.0)          # 2 * (1 * 1 * 3 - 0)


def test_q4k_min_only_gives_negative_sums():
    # q = 0, dmin = 1, m = 1: every weight is -1
    blocks = _q4k_block(d=0x3C00, dmin=0x3C00, mn=(1,) * 8, q=0)[None, :]
    dx = oracle.q4k_backward(blocks, np.array([[4.0]], dtype=np.float32), 256, 1)
    assert np.all(dx == -4.0)


def test_backward_samples_match_full():
    M, K, N = 3, 512, 21
    blocks = _q4k_case(N, K, 5)
    dy = np.random.default_rng(9).standard_normal((M, N)).astype(np.float32)
    full = oracle.q4k_backward(blocks, dy, K, N)
    ms = np.array([0, 2, 1, 2], dtype=np.int32)
    ks = np.array([0, 511, 300, 17], dtype=np.int32)
    assert np.array_equal(oracle.q4k_backward_sample(blocks, dy, K, N, ms, ks), full[ms, ks])
    wts, _ = _w4_case("affine", 64, N, K, 6)
    full = oracle.q4_backward(*wts, dy, K, N, 64, oracle.FMT_AFFINE)
    assert np.array_equal(oracle.q4_backward_sample(*wts, dy, K, N, 64, oracle.FMT_AFFINE, ms, ks), full[ms, ks])
