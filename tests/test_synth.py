"""The seeded generators: determinism, known SplitMix64 outputs, statistics and
the workloads' outlier / heavy-tail structure."""
import numpy as np

import synth
from synth import gen


def test_splitmix64_reference_values():
    # SplitMix64 from seed 0: the published first outputs of the generator
    z = gen.splitmix64(0, 0, 3)
    assert [int(v) for v in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_chunks_agree():
    a = gen.splitmix64(1234, 0, 1000)
    b = np.concatenate([gen.splitmix64(1234, 0, 400), gen.splitmix64(1234, 400, 600)])
    assert np.array_equal(a, b)


def test_normal_statistics():
    z = gen.normal(77, 400000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    t = gen.student_t4(78, 400000)
    assert abs(t.var() - 2.0) < 0.2        # Var of t(4) is 4/(4-2) = 2


def test_subset_is_distinct_and_sized():
    s = gen.choose_subset(5, 4096, 205)
    assert len(set(s.tolist())) == 205 and s.min() >= 0 and s.max() < 4096


def test_workload_structure():
    w1 = synth.workload("q4_0_decode_4096")
    x = gen.activations(w1)
    assert x.shape == (1, 4096) and x.dtype == np.float32
    assert np.array_equal(x, gen.activations(w1))
    w3 = synth.workload("affine_g128_4096x4096x14336")
    xb = gen.activations(w3, M=64)
    assert xb.dtype == np.uint16
    xf = synth.bf16_bits_to_f32(xb)
    cols = np.sort(gen.choose_subset(gen.seed_for(3, 0, 2), 4096, 205))
    # the heavy-tail columns carry much larger extremes than the normal ones
    assert np.abs(xf[:, cols]).max() > 2 * np.abs(np.delete(xf, cols, axis=1)).max() / 2
    wk = synth.workload("q4_k_gemm_16x4096x14336")
    assert np.array_equal(gen.weights(wk, N=4, K=256),
                          gen.weights(synth.workload("q4_k_gemv_1x4096x14336"), N=4, K=256))
    w = gen.weights(w1, N=64, K=4096).astype(np.float64)
    assert abs(w.std() - 0.02) < 0.001
