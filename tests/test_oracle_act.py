"""Pins of the oracle's per-block int8 activation quantizer.

tract PR #2432 (pipeline figure, "activation -> int8, per-block") and MLX PR
#4802 ("x is quantized to int8") quantize activations per block to int8. The
scale is amax / 127 and codes round half to even (the Q4_0 workload's
description); the same rule is read for the affine workloads' 64- and
128-groups.
"""
import numpy as np
import pytest

import synth


def test_scale_one_block_pins_round_half_even(orc):
    # amax = 127 -> xs = 1.0 exactly -> q = rne(v): ties go to the even code.
    v = [127.0, 0.5, 1.5, 2.5, -2.5, 126.5, -0.5, 3.5, -126.5, 0.49999997]
    expect = [127, 0, 2, 2, -2, 126, 0, 4, -126, 0]
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :len(v)] = v
    xq, xs, xsum = orc.quantize_act(x, 32)
    assert xs[0, 0] == np.float32(1.0)
    assert list(xq[0, :len(v)]) == expect
    assert xsum[0, 0] == sum(expect)


def test_zero_block(orc):
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, 32:] = 3.0
    xq, xs, xsum = orc.quantize_act(x, 32)
    assert xs[0, 0] == 0 and xs[0, 1] == 0 and xs[1, 0] == 0
    assert np.all(xq[0] == 0) and np.all(xq[1, :32] == 0)
    assert np.all(xq[1, 32:] == 127) and xsum[1, 1] == 127 * 32


@pytest.mark.parametrize("bs", [32, 64, 128])
def test_random_blocks_invariants(orc, bs):
    rng = np.random.default_rng(bs)
    x = (rng.standard_normal((8, 4 * bs)) * 3).astype(np.float32)
    x[3, :bs] = 0.0
    xq, xs, xsum = orc.quantize_act(x, bs)
    nb = x.shape[1] // bs
    xb = x.reshape(8, nb, bs).astype(np.float64)
    qb = xq.reshape(8, nb, bs).astype(np.int64)
    # block sums
    assert np.array_equal(qb.sum(axis=2), xsum)
    # codes are symmetric int8: never -128
    assert xq.min() >= -127
    for m in range(8):
        for b in range(nb):
            blk, q, s = xb[m, b], qb[m, b], float(xs[m, b])
            amax = np.abs(blk).max()
            if amax == 0:
                assert s == 0 and np.all(q == 0)
                continue
            # scale is amax/127 within float32 rounding
            assert abs(s - amax / 127) <= 2 ** -23 * amax / 127
            # the extreme element maps to +-127
            i = int(np.argmax(np.abs(blk)))
            assert q[i] == (127 if blk[i] > 0 else -127)
            # every code is a nearest integer of v/xs (rounding error <= half a step)
            assert np.all(np.abs(blk / s - q) <= 0.5 + 1e-5)


def test_negation_and_power_of_two_invariance(orc):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    xq, xs, xsum = orc.quantize_act(x, 32)
    nq, nxs, nsum = orc.quantize_act(-x, 32)
    assert np.array_equal(nq, -xq) and np.array_equal(nxs, xs) and np.array_equal(nsum, -xsum)
    for k in (-20, -3, 5, 40):
        sq, sxs, ssum = orc.quantize_act(x * np.float32(2.0 ** k), 32)
        assert np.array_equal(sq, xq)
        assert np.array_equal(sxs, xs * np.float32(2.0 ** k))


def test_bf16_input_matches_f32_of_same_values(orc):
    w = synth.workload("affine_g64_1024x4096x4096")
    xb = synth.gen.activations(w, M=4, K=256)
    xf = synth.bf16_bits_to_f32(xb)
    a = orc.quantize_act(xb, 64)
    b = orc.quantize_act(xf, 64)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_outlier_workload_codes(orc):
    # The decode workload scales 1% of entries x20: their blocks get a large
    # scale and the outlier itself the extreme code.
    w = synth.workload("q4_0_decode_4096")
    x = synth.gen.activations(w)
    xq, xs, xsum = orc.quantize_act(x, 32)
    big = np.abs(x[0]) > 10
    assert big.sum() > 10
    assert np.all(np.abs(xq[0][big]) >= 64)
