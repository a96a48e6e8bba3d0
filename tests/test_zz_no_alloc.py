"""w4a16_matmul_noalloc (the entry point for callers that cannot allocate) against w4a16_matmul
with a caller workspace, through the C ABI, on the GPU.

Two calls in a row share the library's per-GPU scratch array; the second is smaller, so it runs
over what the first left there.  Each must equal w4a16_matmul's result bit for bit (the same
kernels and split order) and pass the element-wise check against the oracle's product.
"""
import numpy as np
import pytest
import torch

import gemm_w4a16_amd as w
import oracle
import refcheck
import workloads
from test_gpu_parity import G128, BF16, NAN16, bf16_f32, dev, gpu_pack, host, say

pytestmark = pytest.mark.gpu


def _noalloc(x_bits, packed, N, K):
    M = x_bits.shape[0]
    y = torch.full((M, N), NAN16, dtype=torch.int16, device="cuda")
    w.w4a16_matmul_noalloc(G128, BF16, dev(x_bits), M, *packed, N, K, y)
    return host(y, np.uint16)


def _with_workspace(x_bits, packed, N, K):
    M = x_bits.shape[0]
    y = torch.full((M, N), NAN16, dtype=torch.int16, device="cuda")
    ws, nb = w.alloc_workspace(G128, M, N, K)
    w.w4a16_matmul(G128, BF16, dev(x_bits), M, *packed, N, K, y, ws, nb)
    return host(y, np.uint16)


def test_noalloc_matches_matmul_on_two_calls_in_a_row():
    # first: 3 x 1 tiles of 128 x 256 split 32 ways (9.8 MB of partials); second, smaller:
    # 2 x 2 tiles of 128 x 128 split 16 ways (1.7 MB); then a GEMV-sized call (no scratch), and
    # two small-M calls with K split over blocks (N = 4096: 4 splits), the second smaller
    cases = [(300, 256, 4096, 201), (130, 200, 2048, 202), (5, 300, 1024, 203), (6, 4096, 8192, 206),
             (2, 4096, 8192, 207)]
    for M, N, K, seed in cases:
        need = w.w4a16_gemm_workspace_bytes(G128, M, N, K)
        say(f"noalloc M={M} N={N} K={K}: {need} B of split-K partials")
        assert need <= w.w4a16_matmul_noalloc_max_scratch_bytes()
        assert (need > 0) == (M > 100 or N == 4096)
        W = workloads.weights(N, K, outliers=True, seed=seed)
        x = workloads.activations(M, K, "bf16", seed=seed + 1)
        packed = gpu_pack(G128, W)
        y = _noalloc(x, packed, N, K)
        np.testing.assert_array_equal(y, _with_workspace(x, packed, N, K))
        refcheck.check(bf16_f32(y), refcheck.g128(x, *oracle.quantize_g128(W)), "bf16", f"noalloc M={M}")


def test_noalloc_refuses_shapes_beyond_its_scratch():
    M, N, K = 2048, 520, 1024        # 8 splits x 2048 x 520 fp32 partials: 34 MB > 16 MiB
    assert w.w4a16_gemm_workspace_bytes(G128, M, N, K) > w.w4a16_matmul_noalloc_max_scratch_bytes()
    packed = gpu_pack(G128, workloads.weights(N, K, seed=204))
    y = torch.full((M, N), NAN16, dtype=torch.int16, device="cuda")
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_matmul_noalloc(G128, BF16, dev(workloads.activations(M, K, "bf16", seed=205)), M, *packed, N, K, y)
    assert e.value.status == w.W4A16_ERR_UNSUPPORTED
    assert np.all(host(y, np.uint16) == 0xFFFF)           # nothing was launched
