"""GPU parity: the HIP kernels through the C ABI against the C oracle.

Integer artefacts (activation codes, scales as bit patterns, code sums,
per-block int32 partials, quantized weight bytes) must be identical; float32
outputs must be within 1e-5 relative RMS of the oracle. Shapes cover the five
workloads of the pages at full size (sampled outputs where the oracle would be
too slow element by element) and ragged sizes spanning several tiles with
tails in M, N and K.
"""
import numpy as np
import pytest
import torch

import block_quantized_bit_amd as q4
import oracle
import synth
from tests._gpu import TOL, rel_rms, sample_pairs, to_dev, to_np, workload_data

pytestmark = pytest.mark.gpu

FMT = {"q4_0": oracle.FMT_Q4_0, "affine": oracle.FMT_AFFINE}


def _sync():
    torch.cuda.synchronize()


def _wts_dev(fmt, wts):
    if fmt == "q4_0":
        wq, wd = wts
        return to_dev(wq), to_dev(wd, torch.float16), None
    wq, ws, wb = wts
    return to_dev(wq), to_dev(ws, torch.bfloat16), to_dev(wb, torch.bfloat16)


def _oracle_y(fmt, wts, act, K, N, bs, rows=None):
    wq, ws = wts[0], wts[1]
    wb = wts[2] if fmt == "affine" else None
    xq, xs, xsum = act
    if rows is not None:
        xq, xs, xsum = xq[rows], xs[rows], xsum[rows]
    return oracle.q4_gemm(wq, ws, wb, xq, xs, xsum, K, N, bs, FMT[fmt])


def _oracle_y_sample(fmt, wts, act, K, N, bs, ms, ns):
    wq, ws = wts[0], wts[1]
    wb = wts[2] if fmt == "affine" else None
    return oracle.q4_gemm_sample(wq, ws, wb, *act, K, N, bs, FMT[fmt], ms, ns)


# ---------------------------------------------------------------- activations

ALL = ["q4_0_minilm_64x384x1536", "q4_0_decode_4096", "affine_g64_1024x4096x4096",
       "affine_g128_4096x4096x14336", "affine_g128_4096x14336x4096"]


@pytest.mark.parametrize("name", ALL)
def test_quantize_act_bit_exact_workloads(name):
    print(f"case quantize_act {name}", flush=True)
    wl, x, _, act, _ = workload_data(name)
    gx = to_dev(x)
    gq, gs, gsum = q4.quantize_act(gx, wl.bs)
    _sync()
    assert np.array_equal(to_np(gq), act[0])
    assert np.array_equal(to_np(gs).view(np.uint32), act[1].view(np.uint32))
    assert np.array_equal(to_np(gsum), act[2])


@pytest.mark.parametrize("bs", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_act_edge_cases(bs, dtype):
    print(f"case quantize_act edges bs={bs} {dtype}", flush=True)
    rng = np.random.default_rng(bs)
    M, K = 7, 3 * 128
    x = (rng.standard_normal((M, K)) * 10.0 ** rng.integers(-6, 6, (M, 1))).astype(np.float32)
    x[0] = 0.0                                   # all-zero row: xs = 0, codes 0
    x[1, :bs] = 127.0 * np.sign(rng.standard_normal(bs))
    x[1, 1:6] = [0.5, 1.5, 2.5, -2.5, 126.5]      # ties: round half to even
    x[2, 5] = 1e30                               # one huge entry per block
    x[3] = -x[3]
    if dtype == "bf16":
        xin = synth.bf16_bits(x)
        gx = to_dev(xin)
    else:
        xin = x
        gx = to_dev(x)
    ref = oracle.quantize_act(xin, bs)
    got = q4.quantize_act(gx, bs)
    _sync()
    assert np.array_equal(to_np(got[0]), ref[0])
    assert np.array_equal(to_np(got[1]).view(np.uint32), ref[1].view(np.uint32))
    assert np.array_equal(to_np(got[2]), ref[2])


# ---------------------------------------------------------------- weight quantizers

@pytest.mark.parametrize("name", ["q4_0_minilm_64x384x1536", "q4_0_decode_4096", "affine_g64_1024x4096x4096",
                                  "affine_g128_4096x14336x4096"])
def test_quantize_weights_bit_exact(name):
    print(f"case quantize_weights {name}", flush=True)
    wl, _, w, _, wts = workload_data(name)
    gw = to_dev(w)
    got = q4.quantize_weights(gw, wl.fmt, wl.bs)
    _sync()
    assert np.array_equal(to_np(got[0]), wts[0])
    assert np.array_equal(to_np(got[1]), wts[1])
    if wl.fmt == "affine":
        assert np.array_equal(to_np(got[2]), wts[2])


def test_quantize_weights_edge_blocks():
    print("case quantize_weights edges", flush=True)
    rng = np.random.default_rng(3)
    w = (0.02 * rng.standard_normal((5, 256))).astype(np.float32)
    w[0, :32] = 0.0                          # zero block: d = -0, codes 8
    w[1, :32] = 0.01                         # constant block
    w[2, :32] = w[2, :32] * 0 + np.float32(-0.5)
    w[2, 7] = 0.5                            # tie of |extremes|: first index wins
    w[3, 32:64] = 1e-7                       # fp16 subnormal scale
    ref = oracle.quantize_q4_0(w)
    got = q4.quantize_weights(to_dev(w), "q4_0", 32)
    _sync()
    assert np.array_equal(to_np(got[0]), ref[0]) and np.array_equal(to_np(got[1]), ref[1])
    wb = synth.bf16_bits(w)
    for g in (64, 128):
        ref = oracle.quantize_affine(wb, g)
        got = q4.quantize_weights(to_dev(wb), "affine", g)
        _sync()
        for a, b in zip(got, ref):
            assert np.array_equal(to_np(a), b)


def test_q4k_quantize_weights_bit_exact():
    print("case q4k quantize_weights", flush=True)
    wl, _, w, _, blocks = workload_data("q4_k_gemv_1x4096x14336")
    got = q4.q4k_quantize_weights(to_dev(w))
    _sync()
    assert np.array_equal(to_np(got), blocks)
    rng = np.random.default_rng(4)
    e = (0.02 * rng.standard_normal((3, 512))).astype(np.float32)
    e[0, :256] = 0.0
    e[1, :32] = np.abs(e[1, :32])            # sub-block with min >= 0
    e[2, 256:] = -np.abs(e[2, 256:])         # all-negative super-block
    got = q4.q4k_quantize_weights(to_dev(e))
    _sync()
    assert np.array_equal(to_np(got), oracle.quantize_q4k(e))


# ---------------------------------------------------------------- integer partials

def _partials_case(fmt, bs, M, K, N, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    if fmt == "q4_0":
        wts = oracle.quantize_q4_0((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    else:
        wts = oracle.quantize_affine(synth.bf16_bits((0.02 * rng.standard_normal((N, K))).astype(np.float32)), bs)
    act = oracle.quantize_act(x, bs)
    return wts, act


@pytest.mark.parametrize("fmt,bs,M,K,N", [
    ("q4_0", 32, 1, 32, 1), ("q4_0", 32, 3, 96, 33), ("q4_0", 32, 65, 160, 31), ("q4_0", 32, 130, 384, 129),
    ("q4_0", 32, 129, 4096, 257), ("affine", 64, 1, 64, 1), ("affine", 64, 5, 192, 65),
    ("affine", 64, 131, 320, 130), ("affine", 128, 2, 128, 1537), ("affine", 128, 67, 384, 63),
    ("affine", 128, 128, 1152, 256),
])
def test_gemm_partials_bit_exact_ragged(fmt, bs, M, K, N):
    print(f"case gemm partials {fmt} bs={bs} M={M} K={K} N={N}", flush=True)
    wts, act = _partials_case(fmt, bs, M, K, N, M * 7 + K + N)
    ref = oracle.q4_partials(wts[0], act[0], K, N, bs, FMT[fmt])
    got = q4.debug_partials("gemm", fmt, bs, to_dev(wts[0]), to_dev(act[0]), to_dev(act[2]))
    _sync()
    assert np.array_equal(to_np(got), ref)
    if M > 2:
        sub = q4.debug_partials("gemm", fmt, bs, to_dev(wts[0]), to_dev(act[0]), to_dev(act[2]), 1, M - 1)
        _sync()
        assert np.array_equal(to_np(sub), ref[1:M - 1])


@pytest.mark.parametrize("fmt,bs,K,N", [("q4_0", 32, 32, 1), ("q4_0", 32, 4096, 4096), ("q4_0", 32, 8224, 37),
                                        ("affine", 64, 4096, 100), ("affine", 128, 4096, 65),
                                        ("affine", 128, 14336, 33)])
def test_gemv_partials_equal_gemm_partials(fmt, bs, K, N):
    # tract PR #2432: the lane-mapped GEMM kernel is bit-exact with the GEMV path
    print(f"case gemv/gemm partials {fmt} bs={bs} K={K} N={N}", flush=True)
    wts, act = _partials_case(fmt, bs, 1, K, N, K + N)
    ref = oracle.q4_partials(wts[0], act[0], K, N, bs, FMT[fmt])
    args = (to_dev(wts[0]), to_dev(act[0]), to_dev(act[2]))
    pv = q4.debug_partials("gemv", fmt, bs, *args)
    pm = q4.debug_partials("gemm", fmt, bs, *args)
    _sync()
    assert np.array_equal(to_np(pv), ref)
    assert np.array_equal(to_np(pm), ref)


@pytest.mark.parametrize("name,rows", [("q4_0_minilm_64x384x1536", None), ("q4_0_decode_4096", None),
                                       ("affine_g64_1024x4096x4096", (0, 3)),
                                       ("affine_g64_1024x4096x4096", (1021, 1024)),
                                       ("affine_g128_4096x4096x14336", (4094, 4096)),
                                       ("affine_g128_4096x14336x4096", (0, 2))])
def test_partials_workloads(name, rows):
    print(f"case partials {name} rows={rows}", flush=True)
    wl, _, _, act, wts = workload_data(name)
    m0, m1 = rows if rows else (0, wl.M)
    ref = oracle.q4_partials(wts[0], act[0], wl.K, wl.N, wl.bs, FMT[wl.fmt], m0, m1)
    got = q4.debug_partials("gemm", wl.fmt, wl.bs, to_dev(wts[0]), to_dev(act[0]), to_dev(act[2]), m0, m1)
    _sync()
    assert np.array_equal(to_np(got), ref)
    if wl.M == 1:
        gv = q4.debug_partials("gemv", wl.fmt, wl.bs, to_dev(wts[0]), to_dev(act[0]), to_dev(act[2]))
        _sync()
        assert np.array_equal(to_np(gv), ref)


# ---------------------------------------------------------------- float outputs

def test_gemv_decode_workload():
    print("case gemv q4_0 decode 1x4096x4096", flush=True)
    wl, _, _, act, wts = workload_data("q4_0_decode_4096")
    g = _wts_dev("q4_0", wts)
    y = q4.gemv("q4_0", 32, *g, *[to_dev(a) for a in act])
    _sync()
    ref = _oracle_y("q4_0", wts, act, wl.K, wl.N, 32)
    assert rel_rms(to_np(y), ref) <= TOL


@pytest.mark.parametrize("fmt,bs,K,N", [("q4_0", 32, 32, 1), ("q4_0", 32, 96, 129), ("q4_0", 32, 8224, 65),
                                        ("affine", 64, 64, 3), ("affine", 64, 4096, 4096),
                                        ("affine", 128, 14336, 257)])
def test_gemv_ragged(fmt, bs, K, N):
    print(f"case gemv {fmt} bs={bs} K={K} N={N}", flush=True)
    wts, act = _partials_case(fmt, bs, 1, K, N, 3 * K + N)
    y = q4.gemv(fmt, bs, *_wts_dev(fmt, wts), *[to_dev(a) for a in act])
    _sync()
    assert rel_rms(to_np(y), _oracle_y(fmt, wts, act, K, N, bs)) <= TOL


@pytest.mark.parametrize("fmt,bs,M,K,N", [
    ("q4_0", 32, 1, 32, 1), ("q4_0", 32, 3, 96, 33), ("q4_0", 32, 65, 160, 1537), ("q4_0", 32, 257, 416, 130),
    ("affine", 64, 1, 64, 5), ("affine", 64, 129, 320, 255), ("affine", 128, 200, 384, 131),
    ("affine", 128, 65, 4224, 64),
    # 33..64 rows with N > 8192: the tiled kernel (the few-row one above 32 rows takes N <= 8192)
    ("q4_0", 32, 48, 256, 8224),
    # few tiles and at least 8 K stages: K split over two wavefront groups per workgroup
    ("affine", 64, 65, 2048, 129), ("q4_0", 32, 200, 1024, 100),
])
def test_gemm_ragged(fmt, bs, M, K, N):
    print(f"case gemm {fmt} bs={bs} M={M} K={K} N={N}", flush=True)
    wts, act = _partials_case(fmt, bs, M, K, N, 5 * M + K + N)
    y = q4.gemm(fmt, bs, *_wts_dev(fmt, wts), *[to_dev(a) for a in act])
    _sync()
    assert rel_rms(to_np(y), _oracle_y(fmt, wts, act, K, N, bs)) <= TOL


@pytest.mark.parametrize("M", [1, 8, 65])
def test_gemm_large_scales(M):
    # affine scales and biases times 2^90 (bf16 exponent field + 90): the tiled
    # kernel (M = 65) takes each group's integer sum into float through an
    # exponent bias and needs |scale| < 2^104; the few-row kernels (M = 1, 8)
    # convert directly. All three against the oracle, with finite outputs.
    print(f"case gemm large scales M={M}", flush=True)
    K, N = 512, 130
    (wq, ws, wb), act = _partials_case("affine", 128, M, K, N, 777 + M)

    def up(bits):
        bits = bits.copy()
        nz = (bits & 0x7FFF) != 0
        bits[nz] = bits[nz] + np.uint16(90 << 7)
        return bits
    wts = (wq, up(ws), up(wb))
    y = q4.gemm("affine", 128, *_wts_dev("affine", wts), *[to_dev(a) for a in act])
    _sync()
    got = to_np(y)
    assert np.all(np.isfinite(got))
    assert rel_rms(got, _oracle_y("affine", wts, act, K, N, 128)) <= TOL


def test_gemm_minilm_workload_full():
    print("case gemm q4_0 64x384x1536", flush=True)
    wl, _, _, act, wts = workload_data("q4_0_minilm_64x384x1536")
    y = q4.gemm("q4_0", 32, *_wts_dev("q4_0", wts), *[to_dev(a) for a in act])
    _sync()
    assert rel_rms(to_np(y), _oracle_y("q4_0", wts, act, wl.K, wl.N, 32)) <= TOL


@pytest.mark.parametrize("name", ["affine_g64_1024x4096x4096", "affine_g128_4096x4096x14336",
                                  "affine_g128_4096x14336x4096"])
def test_gemm_large_workloads_sampled(name):
    print(f"case gemm sampled {name}", flush=True)
    wl, x, _, _, wts = workload_data(name)
    gx = to_dev(x)
    gq, gs, gsum = q4.quantize_act(gx, wl.bs)        # the path as timed: quantize, then GEMM
    y = q4.gemm(wl.fmt, wl.bs, *_wts_dev(wl.fmt, wts), gq, gs, gsum)
    _sync()
    act = (to_np(gq), to_np(gs), to_np(gsum))
    ms, ns = sample_pairs(wl.M, wl.N, 2000, wl.K + wl.N)
    ref = _oracle_y_sample(wl.fmt, wts, act, wl.K, wl.N, wl.bs, ms, ns)
    yh = to_np(y)
    assert rel_rms(yh[ms, ns], ref) <= TOL
    # whole rows at the tile edges against the oracle as well
    rows = np.array([0, 127, 128, wl.M - 1])
    ref_rows = _oracle_y(wl.fmt, wts, act, wl.K, wl.N, wl.bs, rows=rows)
    assert rel_rms(yh[rows], ref_rows) <= TOL


def test_gemm_deterministic():
    print("case gemm determinism", flush=True)
    wl, _, _, act, wts = workload_data("affine_g64_1024x4096x4096")
    g = _wts_dev("affine", wts)
    a = [to_dev(v) for v in act]
    y1 = q4.gemm("affine", 64, *g, *a)
    y2 = q4.gemm("affine", 64, *g, *a)
    _sync()
    assert torch.equal(y1, y2)


# ---------------------------------------------------------------- few-row GEMM (M <= 64)

SMALL_CASES = [("q4_0", 32, 2, 416, 37), ("q4_0", 32, 16, 96, 17), ("q4_0", 32, 17, 4096, 33),
               ("q4_0", 32, 32, 8224, 16), ("affine", 64, 5, 320, 31), ("affine", 64, 32, 4096, 48),
               ("affine", 128, 3, 14336, 21), ("affine", 128, 24, 384, 129),
               # 33 to 64 rows: four 16-row tiles; 512-wide K chunks (Q4_0, g64) and 1024-wide (g128),
               # ragged last chunk, rows and columns
               ("q4_0", 32, 33, 544, 20), ("q4_0", 32, 64, 1632, 33), ("affine", 64, 48, 1088, 37),
               ("affine", 64, 64, 4096, 17), ("affine", 128, 40, 2176, 70), ("affine", 128, 64, 1024, 16),
               # 1 and 2 rows: the GEMV-shaped kernel (several K passes, pass tails, ragged N, N
               # smaller than a workgroup's rows); 3 and 4 rows: the matrix-core weight stream with
               # the 8-row activation load, long rows (four quads in flight) and tiny K
               ("affine", 64, 4, 4160, 45), ("affine", 128, 1, 8320, 19), ("q4_0", 32, 3, 12320, 7),
               ("affine", 128, 2, 256, 3), ("q4_0", 32, 4, 32, 9),
               # 5 to 8 rows at N >= 4096 (the 8-row activation load; ragged K, N one past a
               # workgroup's rows; long K with four quads in flight per wavefront)
               ("q4_0", 32, 5, 4192, 4099), ("affine", 64, 8, 2048, 4096), ("affine", 128, 7, 14336, 4100),
               ("q4_0", 32, 6, 8192, 4096), ("q4_0", 32, 8, 16384, 4096)]


@pytest.mark.parametrize("fmt,bs,M,K,N", SMALL_CASES)
def test_small_partials_bit_exact(fmt, bs, M, K, N):
    print(f"case small partials {fmt} bs={bs} M={M} K={K} N={N}", flush=True)
    wts, act = _partials_case(fmt, bs, M, K, N, 7 * M + K + N)
    ref = oracle.q4_partials(wts[0], act[0], K, N, bs, FMT[fmt])
    got = q4.debug_partials("small", fmt, bs, to_dev(wts[0]), to_dev(act[0]), to_dev(act[2]))
    _sync()
    assert np.array_equal(to_np(got), ref)


@pytest.mark.parametrize("fmt,bs,M,K,N", SMALL_CASES)
def test_small_gemm_ragged(fmt, bs, M, K, N):
    print(f"case small gemm {fmt} bs={bs} M={M} K={K} N={N}", flush=True)
    wts, act = _partials_case(fmt, bs, M, K, N, 7 * M + K + N)
    y = q4.gemm(fmt, bs, *_wts_dev(fmt, wts), *[to_dev(a) for a in act])   # M <= 64: the few-row kernel
    _sync()
    assert rel_rms(to_np(y), _oracle_y(fmt, wts, act, K, N, bs)) <= TOL


@pytest.mark.parametrize("M", [2, 4, 6, 8, 16, 32, 64])
def test_small_gemm_decode_rows(M):
    # the decode workload's weights against M rows drawn like its activation vector
    print(f"case small gemm q4_0 decode rows M={M}", flush=True)
    wl, _, _, _, wts = workload_data("q4_0_decode_4096")
    x = synth.gen.activations(wl, M=M)
    act = oracle.quantize_act(x, 32)
    gq, gs, gsum = q4.quantize_act(to_dev(x), 32)
    y = q4.gemm("q4_0", 32, *_wts_dev("q4_0", wts), gq, gs, gsum)
    _sync()
    assert np.array_equal(to_np(gq), act[0]) and np.array_equal(to_np(gs).view(np.uint32), act[1].view(np.uint32))
    assert rel_rms(to_np(y), _oracle_y("q4_0", wts, act, wl.K, wl.N, 32)) <= TOL


def test_small_gemm_dispatch_boundary():
    # 64 rows take the few-row kernel (four 16-row tiles), 65 the tiled one, 32 and
    # 33 the two- and four-tile few-row kernels; all against the oracle
    print("case small/tiled boundary M=32,33,64,65", flush=True)
    wts, act = _partials_case("affine", 64, 65, 1024, 200, 4242)
    g = _wts_dev("affine", wts)
    ref = _oracle_y("affine", wts, act, 1024, 200, 64)
    for m in (32, 33, 64, 65):
        y = q4.gemm("affine", 64, *g, *[to_dev(a[:m]) for a in act])
        _sync()
        assert rel_rms(to_np(y), ref[:m]) <= TOL, m


@pytest.mark.parametrize("M", [2, 3, 16, 40, 100])
def test_gemm_activation_row_extremes(M):
    # An all-zero activation row (scale 0, codes 0) must give exact zeros, and
    # rows scaled by 1e-30 and 1e30 must match the oracle, on every q4_gemm path
    # at N = 4096: 2 rows take the register GEMV-shaped kernel, 3 and 16 the
    # weight-streaming matrix-core kernel, 40 the staged few-row MFMA kernel and
    # 100 the tiled kernel.
    print(f"case gemm activation row extremes M={M}", flush=True)
    K, N = 512, 4096
    rng = np.random.default_rng(9000 + M)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[0] = 0.0
    x[1] *= np.float32(1e-30)
    if M > 2:
        x[2] *= np.float32(1e30)
    act = oracle.quantize_act(x, 32)
    wts = oracle.quantize_q4_0((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    y = q4.gemm("q4_0", 32, *_wts_dev("q4_0", wts), *[to_dev(a) for a in act])
    _sync()
    got = to_np(y)
    ref = _oracle_y("q4_0", wts, act, K, N, 32)
    assert np.all(np.isfinite(got))
    assert np.all(got[0] == 0.0)
    for m in range(1, M):
        assert rel_rms(got[m], ref[m]) <= TOL, m


def test_small_gemm_kernel_boundaries():
    # at N = 4096: 2 rows take the register GEMV-shaped kernel, 3 to 32 the
    # weight-streaming matrix-core kernel (one 16-row tile up to 16 rows, two
    # from 17), 33 the staged few-row MFMA kernel; K = 16416 at 8 rows gives
    # each wavefront more than four quads (four in flight). All against the oracle.
    print("case small kernel boundaries M=2,3,16,17,32,33", flush=True)
    wts, act = _partials_case("affine", 128, 33, 1024, 4096, 4343)
    g = _wts_dev("affine", wts)
    ref = _oracle_y("affine", wts, act, 1024, 4096, 128)
    for m in (2, 3, 16, 17, 32, 33):
        y = q4.gemm("affine", 128, *g, *[to_dev(a[:m]) for a in act])
        _sync()
        assert rel_rms(to_np(y), ref[:m]) <= TOL, m
    wts, act = _partials_case("q4_0", 32, 8, 16416, 4096, 4344)
    y = q4.gemm("q4_0", 32, *_wts_dev("q4_0", wts), *[to_dev(a) for a in act])
    _sync()
    assert rel_rms(to_np(y), _oracle_y("q4_0", wts, act, 16416, 4096, 32)) <= TOL


@pytest.mark.parametrize("fmt,bs,M,N", [("q4_0", 32, 32, 16), ("affine", 64, 17, 20)])
def test_small_gemm_max_k(fmt, bs, M, N):
    # K = 32768: the longest rows, many quads per wavefront
    print(f"case small gemm max K {fmt} M={M} N={N}", flush=True)
    K = 32768
    wts, act = _partials_case(fmt, bs, M, K, N, 99 + M)
    y = q4.gemm(fmt, bs, *_wts_dev(fmt, wts), *[to_dev(a) for a in act])
    p = q4.debug_partials("small", fmt, bs, to_dev(wts[0]), to_dev(act[0]), to_dev(act[2]))
    _sync()
    assert rel_rms(to_np(y), _oracle_y(fmt, wts, act, K, N, bs)) <= TOL
    assert np.array_equal(to_np(p), oracle.q4_partials(wts[0], act[0], K, N, bs, FMT[fmt]))


@pytest.mark.parametrize("fmt,bs,K,N", [("q4_0", 32, 4096, 4096), ("affine", 128, 14336, 33)])
def test_small_partials_equal_gemv_partials(fmt, bs, K, N):
    print(f"case small/gemv partials {fmt} bs={bs} K={K} N={N}", flush=True)
    wts, act = _partials_case(fmt, bs, 1, K, N, K + 3 * N)
    args = (to_dev(wts[0]), to_dev(act[0]), to_dev(act[2]))
    ps = q4.debug_partials("small", fmt, bs, *args)
    pv = q4.debug_partials("gemv", fmt, bs, *args)
    _sync()
    assert torch.equal(ps, pv)
    assert np.array_equal(to_np(ps), oracle.q4_partials(wts[0], act[0], K, N, bs, FMT[fmt]))


def test_small_gemm_deterministic():
    print("case small gemm determinism", flush=True)
    wts, act = _partials_case("q4_0", 32, 24, 4096, 300, 5150)
    g = _wts_dev("q4_0", wts)
    a = [to_dev(v) for v in act]
    y1 = q4.gemm("q4_0", 32, *g, *a)
    y2 = q4.gemm("q4_0", 32, *g, *a)
    _sync()
    assert torch.equal(y1, y2)


# ---------------------------------------------------------------- affine 6- and 8-bit codes

def _bits_case(bits, g, M, K, N, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w16 = synth.bf16_bits((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    wq, ws, wb = oracle.quantize_affine(w16, g, bits)
    return w16, (wq, ws, wb), oracle.quantize_act(x, g)


BITS_CASES = [(6, 64, 3, 320, 37), (6, 128, 130, 384, 131), (6, 64, 17, 4096, 65), (8, 64, 2, 192, 33),
              (8, 128, 129, 512, 257), (8, 64, 32, 4096, 48), (8, 128, 200, 1152, 64), (6, 64, 40, 1024, 70),
              # four-tile few-row kernel: 8-bit codes in 512- (g64) and 1024-wide (g128) K chunks
              (8, 64, 56, 640, 40), (8, 128, 64, 1152, 24), (6, 128, 36, 2304, 33)]


@pytest.mark.parametrize("bits,g", [(6, 64), (6, 128), (8, 64), (8, 128)])
def test_quantize_weights_bits_bit_exact(bits, g):
    print(f"case quantize affine {bits}-bit g={g}", flush=True)
    w16, (wq, ws, wb), _ = _bits_case(bits, g, 1, 1024, 77, bits * g)
    gq, gs, gb = q4.quantize_weights(to_dev(w16, torch.bfloat16), "affine", g, bits=bits)
    _sync()
    assert np.array_equal(to_np(gq).reshape(-1), wq.reshape(-1))
    assert np.array_equal(to_np(gs), ws) and np.array_equal(to_np(gb), wb)


@pytest.mark.parametrize("bits,g,M,K,N", BITS_CASES)
def test_bits_partials_bit_exact(bits, g, M, K, N):
    print(f"case partials {bits}-bit g={g} M={M} K={K} N={N}", flush=True)
    _, (wq, ws, wb), act = _bits_case(bits, g, M, K, N, M + K + N + bits)
    ref = oracle.q4_partials(wq, act[0], K, N, g, FMT["affine"], bits=bits)
    args = (to_dev(wq), to_dev(act[0]), to_dev(act[2]))
    got = q4.debug_partials("gemm", "affine", g, *args, bits=bits)
    _sync()
    assert np.array_equal(to_np(got), ref)
    if M <= 64:
        gs_ = q4.debug_partials("small", "affine", g, *args, bits=bits)
        _sync()
        assert np.array_equal(to_np(gs_), ref)


@pytest.mark.parametrize("bits,g,M,K,N", BITS_CASES)
def test_bits_gemm_ragged(bits, g, M, K, N):
    print(f"case gemm {bits}-bit g={g} M={M} K={K} N={N}", flush=True)
    _, (wq, ws, wb), act = _bits_case(bits, g, M, K, N, 3 * M + K + N + bits)
    y = q4.gemm("affine", g, to_dev(wq), to_dev(ws, torch.bfloat16), to_dev(wb, torch.bfloat16),
                *[to_dev(a) for a in act], bits=bits)
    _sync()
    ref = oracle.q4_gemm(wq, ws, wb, *act, K, N, g, FMT["affine"], bits=bits)
    assert rel_rms(to_np(y), ref) <= TOL


@pytest.mark.parametrize("bits,g,name", [(6, 64, "affine_g64_1024x4096x4096"), (8, 64, "affine_g64_1024x4096x4096"),
                                        (8, 128, "affine_g64_1024x4096x4096"),
                                        (6, 128, "affine_g128_4096x4096x14336"),
                                        (8, 128, "affine_g128_4096x4096x14336")])
def test_bits_gemm_workload_sampled(bits, g, name):
    # a bf16 workload with its weights quantized at 6 or 8 bits (the widths bench.py times)
    print(f"case gemm {bits}-bit g={g} {name} sampled", flush=True)
    wl, x, w16, _, _ = workload_data(name)
    wq, ws, wb = oracle.quantize_affine(w16, g, bits)
    gq, gs, gsum = q4.quantize_act(to_dev(x), g)
    y = q4.gemm("affine", g, to_dev(wq), to_dev(ws, torch.bfloat16), to_dev(wb, torch.bfloat16), gq, gs, gsum,
                bits=bits)
    _sync()
    act = (to_np(gq), to_np(gs), to_np(gsum))
    ms, ns = sample_pairs(wl.M, wl.N, 1500, bits * 100 + g)
    ref = oracle.q4_gemm_sample(wq, ws, wb, *act, wl.K, wl.N, g, FMT["affine"], ms, ns, bits=bits)
    assert rel_rms(to_np(y)[ms, ns], ref) <= TOL


# ---------------------------------------------------------------- packed weights, fused quantize + GEMM

def _pack_reference(wq, ws, wb, K, N, bs):
    """The packed layout of include/q4.h written out with numpy reshapes."""
    T, S, ng = -(-N // 128), -(-K // 128), K // bs
    wpad = np.zeros((T * 128, S * 64), np.uint8)
    wpad[:N, :K // 2] = wq
    codes = wpad.reshape(T, 128, S, 64).transpose(0, 2, 1, 3)      # [t][s][r][64 bytes]
    parts = [np.ascontiguousarray(codes).tobytes()]
    for a in (ws, wb):
        if a is None:
            continue
        pad = np.zeros((T * 128, ng), np.uint16)
        pad[:N] = a
        parts.append(np.ascontiguousarray(pad.reshape(T, 128, ng).transpose(0, 2, 1)).tobytes())  # [t][g][r]
    return np.frombuffer(b"".join(parts), dtype=np.uint8)


PACK_CASES = [("q4_0", 32, 3, 160, 130), ("q4_0", 32, 130, 416, 257), ("affine", 64, 65, 320, 129),
              ("affine", 128, 200, 384, 131), ("affine", 128, 33, 1152, 256)]


@pytest.mark.parametrize("fmt,bs,M,K,N", PACK_CASES)
def test_pack_weights_layout(fmt, bs, M, K, N):
    print(f"case pack {fmt} bs={bs} K={K} N={N}", flush=True)
    wts, _ = _partials_case(fmt, bs, 1, K, N, 11 * K + N)
    g = _wts_dev(fmt, wts)
    packed = q4.pack_weights(fmt, bs, *g)
    _sync()
    ref = _pack_reference(wts[0], wts[1], wts[2] if fmt == "affine" else None, K, N, bs)
    assert packed.numel() == ref.size == q4.packed_bytes(K, N, bs, fmt)
    assert np.array_equal(to_np(packed), ref)


@pytest.mark.parametrize("fmt,bs,M,K,N", PACK_CASES)
def test_gemm_packed_ragged(fmt, bs, M, K, N):
    print(f"case gemm packed {fmt} bs={bs} M={M} K={K} N={N}", flush=True)
    rng = np.random.default_rng(13 * M + K + N)
    x = rng.standard_normal((M, K)).astype(np.float32)
    if fmt == "affine":
        x = synth.bf16_bits(x)
        xd = to_dev(x, torch.bfloat16)
    else:
        xd = to_dev(x)
    wts, _ = _partials_case(fmt, bs, 1, K, N, 17 * K + N)
    g = _wts_dev(fmt, wts)
    packed = q4.pack_weights(fmt, bs, *g)
    y, (xq, xs_gm, xsum_gm) = q4.gemm_packed(fmt, bs, xd, packed, N)
    _sync()
    act = oracle.quantize_act(x, bs)
    # the codes the call used: bit-identical to the quantizer's, scales transposed
    assert np.array_equal(to_np(xq), act[0])
    assert np.array_equal(to_np(xs_gm).T.view(np.uint32), act[1].view(np.uint32))
    assert np.array_equal(to_np(xsum_gm).T, act[2])
    assert rel_rms(to_np(y), _oracle_y(fmt, wts, act, K, N, bs)) <= TOL
    if M > 64:
        # same tiled kernel arithmetic as the unpacked GEMM (which takes the tiled kernel above 64 rows)
        yu = q4.gemm(fmt, bs, *g, xq, *[to_dev(a) for a in act[1:]])
        _sync()
        assert torch.equal(y, yu)


@pytest.mark.parametrize("name", ["affine_g128_4096x4096x14336", "affine_g128_4096x14336x4096",
                                  "affine_g64_1024x4096x4096", "q4_0_minilm_64x384x1536"])
def test_gemm_packed_workload_sampled(name):
    # every prefill workload bench.py times on packed weights; above 64 rows q4_gemm
    # runs the same tiled kernel on the unpacked layout, so the outputs are identical
    print(f"case gemm packed sampled {name}", flush=True)
    wl, x, _, _, wts = workload_data(name)
    g = _wts_dev(wl.fmt, wts)
    packed = q4.pack_weights(wl.fmt, wl.bs, *g)
    xd = to_dev(x)
    y, (xq, xs_gm, xsum_gm) = q4.gemm_packed(wl.fmt, wl.bs, xd, packed, wl.N)
    gq, gs, gsum = q4.quantize_act(xd, wl.bs)
    yu = q4.gemm(wl.fmt, wl.bs, *g, gq, gs, gsum)
    _sync()
    assert torch.equal(xq, gq) and torch.equal(xs_gm.t(), gs) and torch.equal(xsum_gm.t(), gsum)
    if wl.M > 64:
        assert torch.equal(y, yu)
    else:  # the few-row kernel sums in another order
        assert rel_rms(to_np(y), to_np(yu).astype(np.float64)) <= TOL
    act = (to_np(gq), to_np(gs), to_np(gsum))
    ms, ns = sample_pairs(wl.M, wl.N, 1000, wl.K + 7)
    ref = _oracle_y_sample(wl.fmt, wts, act, wl.K, wl.N, wl.bs, ms, ns)
    assert rel_rms(to_np(y)[ms, ns], ref) <= TOL


# ---------------------------------------------------------------- input gradient, frozen weights

BWD_SHAPES = [(1, 256, 1), (3, 512, 70), (16, 1024, 129), (17, 768, 200), (33, 256, 64),
              # up to 4 rows: the weight-stream kernel, with two K slices (the second partial) and ragged N
              (2, 2304, 45), (4, 4352, 19), (1, 4096, 300),
              # 3 and 5 passes per wavefront (odd counts: the second load slot's last pass is skipped),
              # the last pass partly filled
              (1, 2048, 18000), (3, 2048, 9000), (4, 2048, 17000)]


@pytest.mark.parametrize("M,K,N", BWD_SHAPES)
def test_q4k_backward_ragged(M, K, N):
    print(f"case q4k backward M={M} K={K} N={N}", flush=True)
    rng = np.random.default_rng(M * 31 + K + N)
    blocks = oracle.quantize_q4k((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    dy = rng.standard_normal((M, N)).astype(np.float32)
    dx = q4.q4k_gemm_backward(to_dev(blocks), to_dev(dy), K)
    _sync()
    assert rel_rms(to_np(dx), oracle.q4k_backward(blocks, dy, K, N)) <= TOL


@pytest.mark.parametrize("fmt,bs", [("q4_0", 32), ("affine", 64), ("affine", 128)])
@pytest.mark.parametrize("M,K,N", BWD_SHAPES)
def test_q4_backward_ragged(fmt, bs, M, K, N):
    print(f"case backward {fmt} bs={bs} M={M} K={K} N={N}", flush=True)
    wts, _ = _partials_case(fmt, bs, 1, K, N, 19 * M + K + N)
    dy = np.random.default_rng(K + 3 * N).standard_normal((M, N)).astype(np.float32)
    dx = q4.gemm_backward(fmt, bs, *_wts_dev(fmt, wts), to_dev(dy))
    _sync()
    wb = wts[2] if fmt == "affine" else None
    ref = oracle.q4_backward(wts[0], wts[1], wb, dy, K, N, bs, FMT[fmt])
    assert rel_rms(to_np(dx), ref) <= TOL


@pytest.mark.parametrize("M", [1, 16])
def test_q4k_backward_workload(M):
    # the Q4_K workload's weights (N=14336, K=4096); dY drawn N(0,1)
    print(f"case q4k backward workload M={M}", flush=True)
    wl, _, _, _, blocks = workload_data("q4_k_gemv_1x4096x14336")
    dy = np.random.default_rng(4242 + M).standard_normal((M, wl.N)).astype(np.float32)
    gb, gdy = to_dev(blocks), to_dev(dy)
    dx = q4.q4k_gemm_backward(gb, gdy, wl.K)
    dx2 = q4.q4k_gemm_backward(gb, gdy, wl.K)
    _sync()
    assert torch.equal(dx, dx2)
    ms, ks = sample_pairs(M, wl.K, 400, 77 + M)
    ref = oracle.q4k_backward_sample(blocks, dy, wl.K, wl.N, ms, ks)
    assert rel_rms(to_np(dx)[ms, ks], ref) <= TOL
    # adjoint of the GPU forward product at full size: <dY, W x> = <dX, x>
    x = np.random.default_rng(5 + M).standard_normal((M, wl.K)).astype(np.float32)
    y = q4.q4k_gemm(gb, to_dev(x), wl.N) if M > 1 else q4.q4k_gemv(gb, to_dev(x), wl.N)
    _sync()
    lhs = float((dy.astype(np.float64) * to_np(y).astype(np.float64)).sum())
    rhs = float((to_np(dx).astype(np.float64) * x.astype(np.float64)).sum())
    assert abs(lhs - rhs) <= 1e-4 * np.sqrt(M * wl.N) * np.abs(to_np(y)).mean()


@pytest.mark.parametrize("M", [16, 40])
def test_q4_backward_workload(M):
    # the Q4_K workload's weights (N=14336, K=4096) quantized as Q4_0; above 4 dY
    # rows the f16 matrix-core kernel (hi/lo halves of dY and of d * (q - 8))
    print(f"case q4_0 backward workload M={M}", flush=True)
    wl = synth.workload("q4_k_gemv_1x4096x14336")
    wts = oracle.quantize_q4_0(synth.gen.weights(wl))
    dy = np.random.default_rng(5151 + M).standard_normal((M, wl.N)).astype(np.float32)
    g = _wts_dev("q4_0", wts)
    gdy = to_dev(dy)
    dx = q4.gemm_backward("q4_0", 32, *g, gdy)
    dx2 = q4.gemm_backward("q4_0", 32, *g, gdy)
    _sync()
    assert torch.equal(dx, dx2)
    ms, ks = sample_pairs(M, wl.K, 400, 31 + M)
    ref = oracle.q4_backward_sample(wts[0], wts[1], None, dy, wl.K, wl.N, 32, FMT["q4_0"], ms, ks)
    assert rel_rms(to_np(dx)[ms, ks], ref) <= TOL


def test_q4_backward_scale_extremes():
    # Q4_0 block scales from about 1e-4 to 6e4 in one weight matrix: every
    # block column of the f16 kernel is brought to its own range, so the large
    # scales do not overflow f16 and the small ones keep their precision
    print("case q4_0 backward scale extremes", flush=True)
    M, K, N = 16, 512, 200
    rng = np.random.default_rng(77)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    w[::7] *= np.float32(2e6)     # d up to about 6e4 (beyond 65504 / 8)
    w[3::11] *= np.float32(1e-2)  # d about 1e-4
    w[:, 64:96] *= np.float32(1e-3)  # one block column much smaller than the rest
    wts = oracle.quantize_q4_0(w)
    assert np.abs(wts[1].view(np.float16).astype(np.float32)).max() > 8192
    dy = rng.standard_normal((M, N)).astype(np.float32)
    dx = q4.gemm_backward("q4_0", 32, *_wts_dev("q4_0", wts), to_dev(dy))
    _sync()
    got = to_np(dx)
    ref = oracle.q4_backward(wts[0], wts[1], None, dy, K, N, 32, FMT["q4_0"])
    assert np.all(np.isfinite(got))
    assert rel_rms(got, ref) <= TOL
    assert rel_rms(got[:, 64:96], ref[:, 64:96]) <= TOL


def test_q4_backward_decode_workload_sampled():
    print("case backward q4_0 decode weights M=4", flush=True)
    wl, _, _, _, wts = workload_data("q4_0_decode_4096")
    dy = np.random.default_rng(808).standard_normal((4, wl.N)).astype(np.float32)
    dx = q4.gemm_backward("q4_0", 32, *_wts_dev("q4_0", wts), to_dev(dy))
    _sync()
    ms, ks = sample_pairs(4, wl.K, 400, 9)
    ref = oracle.q4_backward_sample(wts[0], wts[1], None, dy, wl.K, wl.N, 32, FMT["q4_0"], ms, ks)
    assert rel_rms(to_np(dx)[ms, ks], ref) <= TOL


# ---------------------------------------------------------------- Q4_K

def test_q4k_gemv_workload():
    print("case q4k gemv 1x4096x14336", flush=True)
    wl, x, _, _, blocks = workload_data("q4_k_gemv_1x4096x14336")
    y = q4.q4k_gemv(to_dev(blocks), to_dev(x), wl.N)
    _sync()
    ms, ns = sample_pairs(1, wl.N, 3000, 11)
    ref = oracle.q4k_gemm_sample(blocks, x, wl.K, wl.N, ms, ns)
    assert rel_rms(to_np(y)[ms, ns], ref) <= TOL


def test_q4k_gemm_row_magnitudes():
    # The GEMM takes activations through the f16 matrix cores as scaled hi/lo
    # halves, with a power-of-two scale per row and super-block: rows far
    # outside the f16 range (1e20, 1e-20, 1e-33), near its top (3e4), and a row
    # whose super-blocks differ by 1e12 must each match the oracle on their own.
    # A row of zeros (its largest magnitude, taken over the bit patterns, is 0 and
    # the scale exponent is clamped) must give exact zeros, and a row whose first
    # super-block is zero must match the oracle.
    print("case q4k gemm row magnitudes", flush=True)
    K, N = 768, 70
    rng = np.random.default_rng(4321)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    blocks = oracle.quantize_q4k(w)
    scales = np.array([1e-20, 1e-5, 1.0, 3e4, 1e5, 1e20, 7.0, 1e-33, 0.0, 1.0], dtype=np.float64)
    x = (rng.standard_normal((10, K)) * scales[:, None]).astype(np.float32)
    x[6, 256:512] *= np.float32(1e12)   # super-block 1 of row 6: 1e12 x the others
    x[9, 0:256] = 0.0                   # super-block 0 of row 9: zeros
    ref = oracle.q4k_gemm(blocks, x, K, N)
    y = q4.q4k_gemm(to_dev(blocks), to_dev(x), N)
    _sync()
    got = to_np(y)
    assert np.all(np.isfinite(got))
    assert np.all(got[8] == 0.0) and np.all(ref[8] == 0.0)
    for m in (0, 1, 2, 3, 4, 5, 6, 7, 9):
        assert rel_rms(got[m], ref[m]) <= TOL, m


def test_q4k_gemm_workload():
    print("case q4k gemm 16x4096x14336", flush=True)
    wl = synth.workload("q4_k_gemm_16x4096x14336")
    _, _, _, _, blocks = workload_data("q4_k_gemv_1x4096x14336")   # one weight set for both
    x = synth.gen.activations(wl)
    y = q4.q4k_gemm(to_dev(blocks), to_dev(x), wl.N)
    _sync()
    ms, ns = sample_pairs(16, wl.N, 3000, 12)
    ref = oracle.q4k_gemm_sample(blocks, x, wl.K, wl.N, ms, ns)
    assert rel_rms(to_np(y)[ms, ns], ref) <= TOL


# The M = 1 cases cover 1 to 4 chunks per lane (K up to 8192), a partly
# filled last chunk pass (K = 2304: 72 of 128 lanes), the long-row kernel
# (K > 8192), N = 4099, where the GEMV grid leaves some wavefronts with no
# rows (they still take part in the workgroup's activation staging), and
# N = 14339 at K = 256, where each wavefront walks 3 rows in two 2-row passes
# (the second half empty).
@pytest.mark.parametrize("M,K,N", [(1, 256, 1), (1, 768, 70), (1, 2304, 3), (1, 4096, 4099), (1, 256, 14339),
                                   (1, 6144, 9),
                                   (1, 8192, 130), (1, 12288, 33), (1, 20480, 5), (3, 512, 63),
                                   (16, 256, 64), (17, 1024, 65), (40, 2048, 130)])
def test_q4k_ragged(M, K, N):
    print(f"case q4k M={M} K={K} N={N}", flush=True)
    rng = np.random.default_rng(M + K + N)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    blocks = oracle.quantize_q4k(w)
    ref = oracle.q4k_gemm(blocks, x, K, N)
    gb, gx = to_dev(blocks), to_dev(x)
    y = q4.q4k_gemm(gb, gx, N)
    _sync()
    assert rel_rms(to_np(y), ref) <= TOL
    if M == 1:
        yv = q4.q4k_gemv(gb, gx, N)
        _sync()
        assert rel_rms(to_np(yv), ref) <= TOL


# ---------------------------------------------------------------- guard

def test_bit_width_guard_on_device():
    print("case bit-width guard", flush=True)
    # Q4_0 is 4-bit only: with a code array sized for 8-bit codes the binding passes the
    # call through and the library's own width guard must reject it
    wts, act = _partials_case("q4_0", 32, 1, 64, 4, 1)
    wq, wd, wb = _wts_dev("q4_0", wts)
    wq8 = torch.zeros(q4.code_shape(4, 64, 8), dtype=torch.uint8, device=wq.device)
    with pytest.raises(q4.Q4Error) as e:
        q4.gemm("q4_0", 32, wq8, wd, wb, *[to_dev(a) for a in act], bits=8)
    assert e.value.status == 4


# ---------------------------------------------------------------- fused decode step

def _near_tie_activations(M, K, bs, seed):
    """Blocks whose quotients v / xs sit within a few ulps of half-integers:
    the rounding of each code is decided by the last bits of the division."""
    rng = np.random.default_rng(seed)
    x = np.zeros((M, K), dtype=np.float32)
    for m in range(M):
        for b in range(K // bs):
            amax = np.float32(rng.uniform(0.5, 2.0) * 10.0 ** rng.integers(-3, 3))
            s = np.float32(amax / np.float32(127.0))
            k = rng.integers(-126, 126, bs).astype(np.float64) + 0.5
            v = (k * np.float64(s)).astype(np.float32)
            ulps = rng.integers(-3, 4, bs).astype(np.int32)
            v = (v.view(np.int32) + ulps).view(np.float32)
            v[0] = amax                      # fixes the block maximum
            v = np.clip(v, -amax, amax)
            x[m, b * bs:(b + 1) * bs] = v
    return x


@pytest.mark.parametrize("bs", [32, 64, 128])
def test_quantize_act_near_ties(bs):
    print(f"case quantize_act near ties bs={bs}", flush=True)
    x = _near_tie_activations(16, 4096, bs, bs + 100)
    ref = oracle.quantize_act(x, bs)
    got = q4.quantize_act(to_dev(x), bs)
    _sync()
    for a, b in zip(got, ref):
        assert np.array_equal(to_np(a).view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("fmt,bs,xdt", [("q4_0", 32, "f32"), ("q4_0", 32, "bf16"), ("affine", 64, "bf16"),
                                        ("affine", 128, "f32"), ("affine", 128, "bf16")])
def test_gemv_fused_decode(fmt, bs, xdt):
    print(f"case gemv_fused {fmt} bs={bs} x={xdt}", flush=True)
    if fmt == "q4_0":
        wl, x, _, _, wts = workload_data("q4_0_decode_4096")
        if xdt == "bf16":
            x = synth.bf16_bits(synth.bf16_bits_to_f32(synth.bf16_bits(x)))
    else:
        rng = np.random.default_rng(bs)
        x32 = rng.standard_normal((1, 4096)).astype(np.float32)
        x = synth.bf16_bits(x32) if xdt == "bf16" else x32
        wts = oracle.quantize_affine(synth.bf16_bits((0.02 * rng.standard_normal((1000, 4096))).astype(np.float32)),
                                     bs)
    K, N = 4096, wts[0].shape[0]
    act = oracle.quantize_act(x, bs)
    gx = to_dev(x)
    out = (torch.empty((1, K), dtype=torch.int8, device=gx.device),
           torch.empty((1, K // bs), dtype=torch.float32, device=gx.device),
           torch.empty((1, K // bs), dtype=torch.int32, device=gx.device))
    y = q4.gemv_fused(fmt, bs, gx, *_wts_dev(fmt, wts), act_out=out)
    y2 = q4.gemv_fused(fmt, bs, gx, *_wts_dev(fmt, wts))
    _sync()
    for a, b in zip(out, act):
        assert np.array_equal(to_np(a).view(np.uint8), b.view(np.uint8))
    ref = _oracle_y(fmt, wts, act, K, N, bs)
    assert rel_rms(to_np(y), ref) <= TOL
    assert torch.equal(y, y2)


@pytest.mark.parametrize("fmt,bs,xdt,K,N", [("q4_0", 32, "f32", 32768, 70), ("affine", 128, "bf16", 32768, 33),
                                            ("affine", 64, "bf16", 14336, 129), ("q4_0", 32, "bf16", 14336, 5)])
def test_gemv_fused_long_k(fmt, bs, xdt, K, N):
    # past 16 activations per thread the quantizer loops over the rest of x; K = 14336 ends
    # with a partial pass of weight loads, K = 32768 is the largest K the GEMV takes
    print(f"case gemv_fused long K {fmt} bs={bs} x={xdt} K={K} N={N}", flush=True)
    rng = np.random.default_rng(K + N)
    x32 = rng.standard_normal((1, K)).astype(np.float32)
    x = synth.bf16_bits(x32) if xdt == "bf16" else x32
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    wts = oracle.quantize_q4_0(w) if fmt == "q4_0" else oracle.quantize_affine(synth.bf16_bits(w), bs)
    act = oracle.quantize_act(x, bs)
    gx = to_dev(x)
    out = (torch.empty((1, K), dtype=torch.int8, device=gx.device),
           torch.empty((1, K // bs), dtype=torch.float32, device=gx.device),
           torch.empty((1, K // bs), dtype=torch.int32, device=gx.device))
    y = q4.gemv_fused(fmt, bs, gx, *_wts_dev(fmt, wts), act_out=out)
    _sync()
    for a, b in zip(out, act):
        assert np.array_equal(to_np(a).view(np.uint8), b.view(np.uint8))
    assert rel_rms(to_np(y), _oracle_y(fmt, wts, act, K, N, bs)) <= TOL


@pytest.mark.parametrize("fmt,bs", [("q4_0", 32), ("affine", 64), ("affine", 128)])
def test_gemv_fused_activation_extremes(fmt, bs):
    # the quantization inside the decode kernel at its edges: blocks of zeros
    # (scale 0, codes 0), blocks scaled by 1e-30 and 1e30, one huge entry in a
    # block; then an all-zero vector, whose output must be exact zeros
    print(f"case gemv_fused activation extremes {fmt} bs={bs}", flush=True)
    K, N = 4096, 300
    rng = np.random.default_rng(bs + 17)
    x = rng.standard_normal((1, K)).astype(np.float32)
    x[0, 0:bs] = 0.0
    x[0, bs:2 * bs] *= np.float32(1e-30)
    x[0, 2 * bs:3 * bs] *= np.float32(1e30)
    x[0, 3 * bs + 5] = np.float32(3e35)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    wts = oracle.quantize_q4_0(w) if fmt == "q4_0" else oracle.quantize_affine(synth.bf16_bits(w), bs)
    g = _wts_dev(fmt, wts)
    for xv in (x, np.zeros_like(x)):
        act = oracle.quantize_act(xv, bs)
        gx = to_dev(xv)
        out = (torch.empty((1, K), dtype=torch.int8, device=gx.device),
               torch.empty((1, K // bs), dtype=torch.float32, device=gx.device),
               torch.empty((1, K // bs), dtype=torch.int32, device=gx.device))
        y = q4.gemv_fused(fmt, bs, gx, *g, act_out=out)
        _sync()
        for a, b in zip(out, act):
            assert np.array_equal(to_np(a).view(np.uint8), b.view(np.uint8))
        got = to_np(y)
        assert np.all(np.isfinite(got))
        if not xv.any():
            assert np.all(got == 0.0)
        else:
            assert rel_rms(got, _oracle_y(fmt, wts, act, K, N, bs)) <= TOL


def test_gemv_fused_near_ties_and_ragged():
    print("case gemv_fused near ties, ragged N", flush=True)
    x = _near_tie_activations(1, 8192, 32, 5)
    rng = np.random.default_rng(6)
    wts = oracle.quantize_q4_0((0.02 * rng.standard_normal((77, 8192))).astype(np.float32))
    act = oracle.quantize_act(x, 32)
    gx = to_dev(x)
    out = (torch.empty((1, 8192), dtype=torch.int8, device=gx.device),
           torch.empty((1, 256), dtype=torch.float32, device=gx.device),
           torch.empty((1, 256), dtype=torch.int32, device=gx.device))
    y = q4.gemv_fused("q4_0", 32, gx, *_wts_dev("q4_0", wts), act_out=out)
    _sync()
    for a, b in zip(out, act):
        assert np.array_equal(to_np(a).view(np.uint8), b.view(np.uint8))
    assert rel_rms(to_np(y), _oracle_y("q4_0", wts, act, 8192, 77, 32)) <= TOL


@pytest.mark.parametrize("bs,nblocks,seed", [(32, 24, 1), (64, 8, 2), (128, 4, 3)])
def test_quantize_act_exact_reading(bs, nblocks, seed):
    # the near-tie blocks of the oracle's exact pins, checked against exact
    # rational arithmetic directly (not only against the oracle): the
    # standalone quantizer and the fused decode GEMV's codes
    from tests.test_oracle_act import check_exact_codes
    print(f"case exact activation codes bs={bs}", flush=True)

    def standalone(x, bs):
        got = q4.quantize_act(to_dev(x), bs)
        _sync()
        return [to_np(t) for t in got]

    def fused(x, bs):
        K = x.shape[1]
        fmt = "q4_0" if bs == 32 else "affine"
        rng = np.random.default_rng(bs)
        w = (0.02 * rng.standard_normal((40, K))).astype(np.float32)
        wts = oracle.quantize_q4_0(w) if fmt == "q4_0" else oracle.quantize_affine(synth.bf16_bits(w), bs)
        gx = to_dev(x)
        out = (torch.empty((1, K), dtype=torch.int8, device=gx.device),
               torch.empty((1, K // bs), dtype=torch.float32, device=gx.device),
               torch.empty((1, K // bs), dtype=torch.int32, device=gx.device))
        q4.gemv_fused(fmt, bs, gx, *_wts_dev(fmt, wts), act_out=out)
        _sync()
        return [to_np(t) for t in out]

    assert check_exact_codes(standalone, bs, nblocks, seed) == []
    assert check_exact_codes(fused, bs, nblocks, seed) == []


@pytest.mark.parametrize("fmt,bs,xdt,K,N", [("q4_0", 32, "f32", 4096, 4096), ("q4_0", 32, "bf16", 4096, 4096),
                                            ("q4_0", 32, "f32", 8224, 37), ("affine", 64, "bf16", 4096, 1000),
                                            ("affine", 128, "f32", 14336, 33), ("affine", 128, "bf16", 128, 17)])
def test_gemv_fused_partials_bit_exact(fmt, bs, xdt, K, N):
    # the production fused decode kernel (each workgroup quantizes x into its
    # own LDS copy) with the partials store: every workgroup's integer path
    print(f"case fused gemv partials {fmt} bs={bs} x={xdt} K={K} N={N}", flush=True)
    if fmt == "q4_0" and K == 4096 and N == 4096:
        wl, x, _, _, wts = workload_data("q4_0_decode_4096")
        if xdt == "bf16":
            x = synth.bf16_bits(x)
    else:
        rng = np.random.default_rng(K + N)
        x32 = (rng.standard_normal((1, K)) * 2.0).astype(np.float32)
        x32[0, rng.integers(0, K, max(1, K // 100))] *= 20.0
        x = synth.bf16_bits(x32) if xdt == "bf16" else x32
        w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
        wts = oracle.quantize_q4_0(w) if fmt == "q4_0" else oracle.quantize_affine(synth.bf16_bits(w), bs)
    act = oracle.quantize_act(x, bs)
    ref = oracle.q4_partials(wts[0], act[0], K, N, bs, FMT[fmt])[0]
    got = q4.debug_partials_fused(fmt, bs, to_dev(x), to_dev(wts[0]))
    _sync()
    assert np.array_equal(to_np(got), ref)


@pytest.mark.parametrize("M,K,N", [(16, 4096, 14336), (1, 256, 7), (17, 512, 301), (33, 1280, 64)])
def test_q4k_gemm_work_matches_q4k_gemm(M, K, N):
    # the presplit path does the same arithmetic as q4k_gemm: bit-identical outputs, and within the
    # tolerance of the oracle (sampled at the full 16 x 4096 x 14336 workload)
    print(f"case q4k_gemm_work M={M} K={K} N={N}", flush=True)
    if (M, K, N) == (16, 4096, 14336):
        wl, x, _, _, blocks = workload_data("q4_k_gemm_16x4096x14336")
    else:
        rng = np.random.default_rng(M + K + N)
        x = rng.standard_normal((M, K)).astype(np.float32)
        x[M // 2] *= np.float32(1e-20)
        blocks = oracle.quantize_q4k((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    gb, gx = to_dev(blocks), to_dev(x)
    y0 = q4.q4k_gemm(gb, gx, N)
    y1 = q4.q4k_gemm_work(gb, gx, N)
    _sync()
    a, b = to_np(y0), to_np(y1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    if M * N <= 20000:
        ref = oracle.q4k_gemm(blocks, x, K, N)
        assert rel_rms(b, ref) <= TOL
    else:
        ms, ns = sample_pairs(M, N, 400, 5)
        ref = oracle.q4k_gemm_sample(blocks, x, K, N, ms, ns)
        assert rel_rms(b[ms, ns], ref) <= TOL
