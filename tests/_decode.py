"""Independent numpy decoders of the packed layouts, used by brute-force pins.

Code layout: block b of a weight row is 16 bytes at offset 16*b; byte j holds
k = 32*b + j in its low nibble and k = 32*b + 16 + j in its high nibble.
Q4_K block: fp16 d, fp16 dmin, 12 bytes of sixteen 6-bit fields (sc[0..7],
m[0..7], little-endian, field f at bits 6f..6f+5), then qs[128] where chunk c
of 64 weights takes the low nibbles of qs[32c..32c+31] (sub-block 2c) and then
their high nibbles (sub-block 2c+1).
"""
import numpy as np


def codes_from_planes(wq: np.ndarray, K: int) -> np.ndarray:
    N = wq.shape[0]
    blk = wq.reshape(N, K // 32, 16).astype(np.int64)
    out = np.empty((N, K // 32, 32), dtype=np.int64)
    out[:, :, :16] = blk & 0xF
    out[:, :, 16:] = blk >> 4
    return out.reshape(N, K)


def planes_from_codes(codes: np.ndarray) -> np.ndarray:
    N, K = codes.shape
    c = codes.reshape(N, K // 32, 32).astype(np.uint8)
    return (c[:, :, :16] | (c[:, :, 16:] << 4)).reshape(N, K // 2).astype(np.uint8)


def f16(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def q4k_fields(b12: np.ndarray):
    bits = 0
    for i, v in enumerate(np.asarray(b12, dtype=np.uint8).tolist()):
        bits |= int(v) << (8 * i)
    vals = [(bits >> (6 * f)) & 0x3F for f in range(16)]
    return np.array(vals[:8]), np.array(vals[8:])


def q4k_dequant(blocks: np.ndarray, N: int, K: int) -> np.ndarray:
    nb = K // 256
    out = np.empty((N, K), dtype=np.float64)
    b = blocks.reshape(N, nb, 144)
    for n in range(N):
        for j in range(nb):
            raw = b[n, j]
            d = f16(raw[0:2].view(np.uint16))[0]
            dmin = f16(raw[2:4].view(np.uint16))[0]
            sc, mn = q4k_fields(raw[4:16])
            qs = raw[16:].astype(np.int64)
            w = np.empty(256)
            for c in range(4):
                lo = qs[32 * c:32 * c + 32] & 0xF
                hi = qs[32 * c:32 * c + 32] >> 4
                w[64 * c:64 * c + 32] = d * sc[2 * c] * lo - dmin * mn[2 * c]
                w[64 * c + 32:64 * c + 64] = d * sc[2 * c + 1] * hi - dmin * mn[2 * c + 1]
            out[n, 256 * j:256 * j + 256] = w
    return out


def codes_from_bits(wq: np.ndarray, N: int, K: int, bits: int) -> np.ndarray:
    """Codes [N][K] of a 4-, 6- or 8-bit affine code array.
    8 bits: one byte per code. 6 bits: the 4-bit layout holds the low 4 bits
    (N*K/2 bytes), then the high 2 bits follow as N*K/4 bytes: block b of row n
    is 8 bytes at 8*b, two little-endian words; word h holds code 32b + 16h + c
    in byte c % 4, bits 2*(c // 4) and 2*(c // 4) + 1."""
    flat = np.ascontiguousarray(wq).reshape(-1)
    if bits == 8:
        return flat.reshape(N, K).astype(np.int64)
    lo = codes_from_planes(flat[:N * K // 2].reshape(N, K // 2), K)
    if bits == 4:
        return lo
    hp = flat[N * K // 2:].reshape(N, K // 32, 2, 4).astype(np.int64)   # [n][block][word h][byte]
    c = np.arange(16)
    hi = (hp[:, :, :, c % 4] >> (2 * (c // 4))) & 3                       # [n][block][h][c]
    return lo | (hi.reshape(N, K) << 4)
