"""Planted mistakes in copies of the oracle's activation quantizer must fail its pins.

Each mutant is the oracle source with one plausible other reading of the
quantizer written in (a reciprocal-multiply scale, codes from v * 127 / amax
or v * (1 / xs), a quotient rounded only once to an integer, ties away from
zero). The copy is compiled on the CPU into a temporary directory and run
through the exact pins of tests/test_oracle_act.py; an unchanged copy, built
the same way, passes them. The oracle itself is not modified.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle

from .test_oracle_act import check_exact_codes

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

SCALE = "float s = amax / 127.0f;"
QUOT = "float r = load_x(x, xdt, base + j) / s;"
ROUND = "q = (int)nearbyintf(r);"

MUTANTS = {
    "scale by reciprocal": [(SCALE, "float s = amax * (1.0f / 127.0f);")],
    "codes by 127/amax": [(QUOT, "float r = load_x(x, xdt, base + j) * (127.0f / amax);")],
    "codes by rcp(xs)": [(QUOT, "float r = load_x(x, xdt, base + j) * (1.0f / s);")],
    "exact quotient": [(QUOT, "double r = (double)load_x(x, xdt, base + j) / (double)s;"),
                       (ROUND, "q = (int)nearbyint(r);")],
    "ties away from zero": [(ROUND, "q = (int)roundf(r);")],
}


def _build(tmp_path, name, edits):
    text = open(SRC).read()
    for old, new in edits:
        assert text.count(old) == 1, f"the oracle no longer contains {old!r}"
        text = text.replace(old, new)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(text)
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(c), "-o", str(so), "-lm"])
    L = ctypes.CDLL(str(so))
    L.or_quantize_act.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 4
    return L


def _quantizer(L):
    def quantize(x, bs):
        x = np.ascontiguousarray(x, dtype=np.float32)
        M, K = x.shape
        xq = np.empty((M, K), dtype=np.int8)
        xs = np.empty((M, K // bs), dtype=np.float32)
        xsum = np.empty((M, K // bs), dtype=np.int32)
        p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
        assert L.or_quantize_act(M, K, bs, 0, p(x), p(xq), p(xs), p(xsum)) == 0
        return xq, xs, xsum
    return quantize


def _fails(quantize):
    n = 0
    for bs, nb, seed in ((32, 24, 1), (64, 8, 2), (128, 4, 3)):
        n += len(check_exact_codes(quantize, bs, nb, seed))
    # the scale-one block: ties go to the even code
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :6] = [127.0, 0.5, 1.5, 2.5, -2.5, 126.5]
    xq, _, _ = quantize(x, 32)
    n += list(xq[0, :6]) != [127, 0, 2, 2, -2, 126]
    return n


def test_unchanged_copy_passes(tmp_path):
    assert _fails(_quantizer(_build(tmp_path, "control", []))) == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_the_pins(tmp_path, name):
    L = _build(tmp_path, name.replace(" ", "_").replace("/", "_"), MUTANTS[name])
    assert _fails(_quantizer(L)) > 0, f"the pins do not catch the reading '{name}'"
