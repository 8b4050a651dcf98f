"""Pins of the oracle's per-block int8 activation quantizer.

tract PR #2432 (pipeline figure, "activation -> int8, per-block") and MLX PR
#4802 ("x is quantized to int8") quantize activations per block to int8. The
scale is amax / 127 and codes round half to even (the Q4_0 workload's
description); the same rule is read for the affine workloads' 64- and
128-groups.
"""
from fractions import Fraction

import numpy as np
import pytest

import synth

from ._exact import act_code, act_scale, bits, f32, quantize_block, rne_f32, rne_int


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


# ---- exact pins of the scale and the code rounding ----------------------------------
#
# The reading: xs = amax / 127 correctly rounded to binary32, and each code is
# round-half-even of the correctly rounded binary32 quotient v / xs (clamped to
# +-127). The expected values below come from exact rational arithmetic
# (tests/_exact.py). Each fixture is chosen so that the plausible other
# readings give a different result on at least one element:
#   scale  amax * f32(1/127)            (a reciprocal multiply)
#   code   v * f32(127 / amax)          (no division by the stored scale)
#          v * f32(1 / xs)              (a reciprocal of the stored scale)
#          round(v / xs) of the exact rational (no float32 quotient)
#          round half away from zero


def alt_scale_recip(amax):
    return rne_f32(Fraction(float(amax)) * Fraction(float(rne_f32(Fraction(1, 127)))))


def _clamp(q):
    return max(-127, min(127, q))


def alt_code_127_over_amax(v, amax):
    r = rne_f32(Fraction(float(v)) * Fraction(float(rne_f32(Fraction(127) / Fraction(float(amax))))))
    return _clamp(rne_int(Fraction(float(r))))


def alt_code_rcp_scale(v, xs):
    r = rne_f32(Fraction(float(v)) * Fraction(float(rne_f32(1 / Fraction(float(xs))))))
    return _clamp(rne_int(Fraction(float(r))))


def alt_code_exact_quotient(v, xs):
    return _clamp(rne_int(Fraction(float(v)) / Fraction(float(xs))))


def alt_code_half_away(v, xs):
    r = Fraction(float(rne_f32(Fraction(float(v)) / Fraction(float(xs)))))
    a = abs(r) + Fraction(1, 2)
    q = a.numerator // a.denominator
    return _clamp(q if r >= 0 else -q)


def separating_scales(count, seed=2432):
    """Seeded amax values whose correctly rounded amax/127 differs from amax*f32(1/127)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        a = np.float32(rng.uniform(0.25, 64.0))
        if act_scale(a) != alt_scale_recip(a):
            out.append(a)
    return out


def near_tie_blocks(bs, nblocks, seed):
    """Blocks whose first element is the block's amax (one that separates the
    two scale readings) and whose other elements sit within two ulps of
    (half-integer) * xs, with random signs: the cases where the readings of
    the code rounding differ."""
    rng = np.random.default_rng(seed)
    out = []
    for a in separating_scales(nblocks, seed):
        xs = act_scale(a)
        row = [a]
        halves = rng.choice(np.arange(1, 254, 2), size=bs - 1, replace=bs - 1 > 127)
        for t2 in halves:
            v0 = rne_f32(Fraction(int(t2), 2) * Fraction(float(xs)))
            v = f32(bits(v0) + int(rng.integers(-2, 3)))
            v = min(v, a)
            row.append(v if rng.random() < 0.5 else -v)
        out.append(row)
    return np.array(out, dtype=np.float32)


def check_exact_codes(quantize, bs, nblocks, seed):
    """quantize(x [M][K], bs) -> (xq, xs, xsum). Returns the list of failures
    against the exact reading (empty when it holds)."""
    x = near_tie_blocks(bs, nblocks, seed)
    xq, xs, xsum = quantize(x.reshape(1, -1), bs)
    fails = []
    for b in range(nblocks):
        q, s, t = quantize_block(x[b])
        if bits(xs[0, b]) != bits(s):
            fails.append(("scale", b, bits(xs[0, b]), bits(s)))
        got = [int(c) for c in xq[0, b * bs:(b + 1) * bs]]
        for j in range(bs):
            if got[j] != q[j]:
                fails.append(("code", b, j, got[j], q[j]))
        if int(xsum[0, b]) != t:
            fails.append(("sum", b, int(xsum[0, b]), t))
    return fails


def test_exact_helpers_agree_with_ieee_division():
    # numpy's float32 division is IEEE correctly rounded: the helper must agree on
    # random operands, subnormal quotients included
    rng = np.random.default_rng(5)
    a = rng.standard_normal(400).astype(np.float32) * np.float32(3.0)
    b = (rng.standard_normal(400).astype(np.float32) + np.float32(0.1)) * np.float32(2.0 ** 60)
    b[:40] = np.float32(127.0)
    for u, v in zip(a, b):
        if v == 0:
            continue
        want = np.float32(u) / np.float32(v)
        assert bits(rne_f32(Fraction(float(u)) / Fraction(float(v)))) == bits(want)
    # ties at the halfway point between two floats go to the even significand
    assert bits(rne_f32(Fraction(1) + Fraction(1, 2 ** 24))) == bits(np.float32(1.0))
    assert bits(rne_f32(Fraction(1) + Fraction(3, 2 ** 24))) == bits(np.float32(1.0)) + 2
    assert rne_int(Fraction(5, 2)) == 2 and rne_int(Fraction(-5, 2)) == -2 and rne_int(Fraction(7, 2)) == 4


def test_scale_is_correctly_rounded_quotient(orc):
    # 2048 seeded amax values over 2^-140 .. 2^120, plus the separating ones:
    # the stored scale must be the correctly rounded amax / 127, bit for bit
    rng = np.random.default_rng(127)
    amax = (rng.uniform(1.0, 2.0, 2048) * 2.0 ** rng.integers(-140, 120, 2048)).astype(np.float32)
    amax = np.concatenate([amax, np.array(separating_scales(64), dtype=np.float32)])
    x = np.zeros((amax.size, 32), dtype=np.float32)
    x[:, 5] = amax
    x[1::2, 5] *= -1
    _, xs, _ = orc.quantize_act(x, 32)
    want = np.array([act_scale(a) for a in amax], dtype=np.float32)
    assert np.array_equal(xs[:, 0].view(np.uint32), want.view(np.uint32))
    # the fixture separates the reciprocal-multiply reading
    alt = np.array([alt_scale_recip(a) for a in amax], dtype=np.float32)
    assert (alt.view(np.uint32) != want.view(np.uint32)).sum() >= 64


@pytest.mark.parametrize("bs,nblocks,seed", [(32, 24, 1), (64, 8, 2), (128, 4, 3)])
def test_near_tie_codes_are_exact(orc, bs, nblocks, seed):
    assert check_exact_codes(orc.quantize_act, bs, nblocks, seed) == []


def test_near_tie_fixture_separates_the_other_readings():
    # every alternative reading gives another code on at least one element of
    # the 32-blocks above, so a quantizer that took it fails the pin
    x = near_tie_blocks(32, 24, 1)
    diff = {"127/amax": 0, "rcp(xs)": 0, "exact quotient": 0, "half away": 0, "scale": 0}
    for row in x:
        q, xs, _ = quantize_block(row)
        a = abs(float(row[0]))
        diff["scale"] += bits(alt_scale_recip(a)) != bits(xs)
        for v, c in zip(row, q):
            diff["127/amax"] += alt_code_127_over_amax(v, a) != c
            diff["rcp(xs)"] += alt_code_rcp_scale(v, xs) != c
            diff["exact quotient"] += alt_code_exact_quotient(v, xs) != c
            diff["half away"] += alt_code_half_away(v, xs) != c
    assert all(n > 0 for n in diff.values()), diff


def test_hand_block_near_ties(orc):
    # One block written out: amax = 0x427325a7 (60.786770), whose scale
    # 60.786770/127 rounds to 0x3ef50fc7 while amax * f32(1/127) gives
    # 0x3ef50fc6; the other values sit next to (half-integer) * xs.
    amax = f32(0x427325A7)
    vals = [amax, f32(0x4161EA8B), f32(0x41AE3937), f32(0x41F325A7), f32(0x4236D6C5),
            f32(0x42594CFD), f32(0x3F37CBD5), f32(0x3FD66DCE), f32(0x4009D8E0), f32(0x40471CD2)]
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :len(vals)] = vals
    x[0, 16:16 + len(vals) - 1] = [-v for v in vals[1:]]
    xq, xs, xsum = orc.quantize_act(x, 32)
    q, s, t = quantize_block(x[0])
    assert bits(s) == 0x3EF50FC7 and bits(alt_scale_recip(amax)) == 0x3EF50FC6
    assert bits(xs[0, 0]) == bits(s)
    assert [int(c) for c in xq[0]] == q and int(xsum[0, 0]) == t
    # codes of the values next to 29.5, 45.5, 63.5, 95.5, 113.5, 1.5, 3.5, 4.5, 6.5 times xs
    assert q[1:10] == [30, 46, 64, 96, 114, 2, 4, 4, 6]
    assert q[16:25] == [-30, -46, -64, -96, -114, -2, -4, -4, -6]
