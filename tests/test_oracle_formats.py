"""Pins of the oracle's number-format converters against library routines.

binary16 follows IEEE 754 (numpy's float16 is the library routine); bfloat16
is the upper half of binary32 with round-half-even (torch's bfloat16 is the
library routine). The C-Kernel-Engine gemm_kernels_q4k.c page converts the
Q4_K fp16 fields d and dmin to float before use.
"""
import numpy as np
import torch


def test_f16_decode_exhaustive(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = orc.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_roundtrip_exhaustive(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = orc.f16_to_f32(h)
    keep = ~np.isnan(f)
    back = orc.f32_to_f16(f[keep])
    assert np.array_equal(back, h[keep])


def _f16_edge_values():
    vals = [0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 1e6, 2.0 ** -24, 2.0 ** -25,
            1.5 * 2.0 ** -25, 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -11),
            1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0, -0.5 - 2.0 ** -12]
    # every midpoint between consecutive positive finite halves (ties go to even)
    h = np.arange(0, 0x7BFF, dtype=np.uint32).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mids = ((lo + hi) / 2).astype(np.float32)
    return np.concatenate([np.array(vals, dtype=np.float32), mids, -mids])


def test_f16_encode_matches_numpy(orc):
    rng = np.random.default_rng(1)
    rand = rng.standard_normal(200000).astype(np.float32) * np.float32(2.0) ** rng.integers(
        -30, 18, 200000).astype(np.float32)
    x = np.concatenate([_f16_edge_values(), rand]).astype(np.float32)
    mine = orc.f32_to_f16(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_encode_matches_torch(orc):
    rng = np.random.default_rng(2)
    rand = rng.standard_normal(200000).astype(np.float32) * np.float32(2.0) ** rng.integers(
        -60, 60, 200000).astype(np.float32)
    # exact ties: low half == 0x8000 with odd and even upper halves
    u = rng.integers(0, 0x7F00, 5000).astype(np.uint32) << 16 | np.uint32(0x8000)
    ties = u.view(np.float32)
    x = np.concatenate([rand, ties, -ties, np.float32([3.4e38, -3.4e38, 1e-40])])
    mine = orc.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_decode(orc):
    b = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], dtype=np.uint16)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(orc.bf16_to_f32(b), ref)
