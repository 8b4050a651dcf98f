"""The oracle's thread partition over output columns changes no bit of a result."""
import numpy as np
import pytest

import synth


@pytest.fixture
def threads(orc):
    yield orc.set_threads
    orc.set_threads(1)


@pytest.mark.parametrize("T", [2, 3, 8, 64])
def test_threaded_products_bit_identical(orc, threads, T):
    rng = np.random.default_rng(T)
    M, K, N = 3, 512, 37
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    act32 = orc.quantize_act(x, 32)
    act128 = orc.quantize_act(x, 128)
    wq, wd = orc.quantize_q4_0(w)
    a6 = orc.quantize_affine(synth.bf16_bits(w), 128, bits=6)
    blocks = orc.quantize_q4k(w)
    outs = []
    for t in (1, T):
        assert threads(t) == t
        outs.append([
            orc.q4_gemm(wq, wd, None, *act32, K, N, 32, orc.FMT_Q4_0),
            orc.q4_gemm(a6[0], a6[1], a6[2], *act128, K, N, 128, orc.FMT_AFFINE, bits=6),
            orc.q4k_gemm(blocks, x, K, N),
            orc.q4k_gemv(blocks, x[1], K, N),
        ])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_more_threads_than_columns(orc, threads):
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, 256)).astype(np.float32)
    blocks = orc.quantize_q4k((0.02 * rng.standard_normal((3, 256))).astype(np.float32))
    ref = orc.q4k_gemm(blocks, x, 256, 3)
    threads(16)
    assert np.array_equal(orc.q4k_gemm(blocks, x, 256, 3).view(np.uint32), ref.view(np.uint32))
