"""The input gradient's no-allocation entry point (static per-device scratch)
against the entry point that takes a caller workspace, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input (the buffer
keeps the first call's contents); each must equal the workspace entry point
bit for bit, and both must be within the float tolerance of the oracle.
"""
import numpy as np
import pytest
import torch

import block_quantized_bit_amd as q4
import oracle
from tests._gpu import TOL, rel_rms, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shapes", [((16, 4096, 2048), (3, 1024, 700)), ((40, 2048, 1500), (16, 512, 64))])
def test_noalloc_backward_matches_workspace_entry(shapes):
    for i, (M, K, N) in enumerate(shapes):
        print(f"case noalloc backward call {i} M={M} K={K} N={N}", flush=True)
        rng = np.random.default_rng(M * 131 + K + N)
        blocks = oracle.quantize_q4k((0.02 * rng.standard_normal((N, K))).astype(np.float32))
        dy = rng.standard_normal((M, N)).astype(np.float32)
        gb, gdy = to_dev(blocks), to_dev(dy)
        dx_na = torch.full((M, K), float("nan"), dtype=torch.float32, device=gdy.device)
        q4.q4k_gemm_backward_noalloc(gb, gdy, K, dx_na)
        dx_ws = q4.q4k_gemm_backward(gb, gdy, K)
        torch.cuda.synchronize()
        a, b = to_np(dx_na), to_np(dx_ws)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        assert rel_rms(a, oracle.q4k_backward(blocks, dy, K, N)) <= TOL
