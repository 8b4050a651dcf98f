"""Counter-based random draws and the workload recipes.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014). Draw i of a stream with seed s mixes the
state s + (i + 1) * GAMMA (mod 2**64), which is exactly the sequence the
sequential generator produces, so draws can be taken in vectorised chunks.

* uniform: u = ((z >> 11) + 0.5) * 2**-53, strictly inside (0, 1).
* normal: Box-Muller on consecutive uniform pairs (u1, u2);
  r = sqrt(-2 ln u1), outputs r cos(2 pi u2) then r sin(2 pi u2).
* Student-t with 4 degrees of freedom: z0 / sqrt((z1^2+z2^2+z3^2+z4^2)/4)
  from five consecutive normals.
* index subsets: partial Fisher-Yates (Durstenfeld) shuffle of range(K).

Values are computed in float64 and rounded once to float32 (and, where the
workload is bfloat16, once more to bfloat16 with round-half-even).
"""
from __future__ import annotations

import dataclasses
import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Draws start .. start+count-1 of the SplitMix64 stream `seed` (uint64)."""
    idx = np.arange(start + 1, start + 1 + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform(seed: int, start: int, count: int) -> np.ndarray:
    z = splitmix64(seed, start, count)
    return ((z >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def normal(seed: int, count: int, start_pair: int = 0) -> np.ndarray:
    """`count` standard normals (float64), Box-Muller pairs from pair `start_pair`."""
    out = np.empty(count, dtype=np.float64)
    npairs = (count + 1) // 2
    done = 0
    p = 0
    while p < npairs:
        n = min(_CHUNK, npairs - p)
        u = uniform(seed, 2 * (start_pair + p), 2 * n)
        r = np.sqrt(-2.0 * np.log(u[0::2]))
        t = 2.0 * np.pi * u[1::2]
        z = np.empty(2 * n, dtype=np.float64)
        z[0::2] = r * np.cos(t)
        z[1::2] = r * np.sin(t)
        take = min(2 * n, count - done)
        out[done:done + take] = z[:take]
        done += take
        p += n
    return out


def student_t4(seed: int, count: int) -> np.ndarray:
    z = normal(seed, 5 * count).reshape(count, 5)
    return z[:, 0] / np.sqrt((z[:, 1:] ** 2).sum(axis=1) / 4.0)


def choose_subset(seed: int, k_range: int, count: int) -> np.ndarray:
    """`count` distinct indices of range(k_range), in draw order (partial Fisher-Yates)."""
    arr = np.arange(k_range, dtype=np.int64)
    draws = splitmix64(seed, 0, count)
    for i in range(count):
        j = i + int(draws[i] % np.uint64(k_range - i))
        arr[i], arr[j] = arr[j], arr[i]
    return arr[:count].copy()


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-half-even; inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def seed_for(workload_id: int, variant: int, stream: int) -> int:
    """Seed = 1000*(id+1) + 100*variant + stream; streams: 0 weights,
    1 activations, 2 index selection, 3 heavy-tail draws."""
    return 1000 * (workload_id + 1) + 100 * variant + stream


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # workload id (seed family)
    variant: int        # seed variant
    M: int
    K: int
    N: int
    fmt: str            # "q4_0" | "affine" | "q4_k"
    bs: int             # block / group size along K (256 for q4_k super-blocks)
    xdtype: str         # "f32" | "bf16" (activation storage)
    wdtype: str         # "f32" | "bf16" (unquantized weight storage)
    outlier_frac: float = 0.0   # fraction of x entries scaled x20 (M == 1 workloads)
    tail_frac: float = 0.0      # fraction of K columns drawn Student-t(4)
    weight_variant: int | None = None  # seed variant of the weights, if shared


WORKLOADS = {
    "q4_0_minilm_64x384x1536": Workload("q4_0_minilm_64x384x1536", 0, 0, 64, 384, 1536, "q4_0", 32, "f32", "f32"),
    "q4_0_decode_4096": Workload("q4_0_decode_4096", 1, 0, 1, 4096, 4096, "q4_0", 32, "f32", "f32", outlier_frac=0.01),
    "affine_g64_1024x4096x4096": Workload("affine_g64_1024x4096x4096", 2, 0, 1024, 4096, 4096, "affine", 64, "bf16", "bf16"),
    "affine_g128_4096x4096x14336": Workload("affine_g128_4096x4096x14336", 3, 0, 4096, 4096, 14336, "affine", 128, "bf16", "bf16", tail_frac=0.05),
    "affine_g128_4096x14336x4096": Workload("affine_g128_4096x14336x4096", 3, 1, 4096, 14336, 4096, "affine", 128, "bf16", "bf16", tail_frac=0.05),
    "q4_k_gemv_1x4096x14336": Workload("q4_k_gemv_1x4096x14336", 4, 0, 1, 4096, 14336, "q4_k", 256, "f32", "f32", weight_variant=0),
    "q4_k_gemm_16x4096x14336": Workload("q4_k_gemm_16x4096x14336", 4, 1, 16, 4096, 14336, "q4_k", 256, "f32", "f32", weight_variant=0),
}


def _round_f32(a: np.ndarray) -> np.ndarray:
    return a.astype(np.float32)


def weights(w: Workload, N: int | None = None, K: int | None = None) -> np.ndarray:
    """Unquantized weights [N][K]: N(0, 0.02^2); float32, or bfloat16 bits (uint16)."""
    N = w.N if N is None else N
    K = w.K if K is None else K
    wv = w.variant if w.weight_variant is None else w.weight_variant
    vals = _round_f32(0.02 * normal(seed_for(w.wid, wv, 0), N * K)).reshape(N, K)
    return bf16_bits(vals) if w.wdtype == "bf16" else vals


def activations(w: Workload, M: int | None = None, K: int | None = None) -> np.ndarray:
    """Activations [M][K]: N(0,1) with the workload's outlier or heavy-tail structure;
    float32, or bfloat16 bits (uint16)."""
    M = w.M if M is None else M
    K = w.K if K is None else K
    x = normal(seed_for(w.wid, w.variant, 1), M * K).reshape(M, K)
    if w.outlier_frac > 0.0:
        cnt = int(round(w.outlier_frac * M * K))
        idx = choose_subset(seed_for(w.wid, w.variant, 2), M * K, cnt)
        flat = x.reshape(-1)
        flat[idx] *= 20.0
    if w.tail_frac > 0.0:
        cnt = int(round(w.tail_frac * K))
        cols = np.sort(choose_subset(seed_for(w.wid, w.variant, 2), K, cnt))
        t = student_t4(seed_for(w.wid, w.variant, 3), M * cnt).reshape(M, cnt)
        x[:, cols] = t
    x32 = _round_f32(x)
    return bf16_bits(x32) if w.xdtype == "bf16" else x32


def workload(name: str) -> Workload:
    return WORKLOADS[name]
