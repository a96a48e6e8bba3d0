"""W4A8 on the GPU (through the C ABI) against the CPU oracle.

Bars: the activation quantizer (int8 codes, row scales, group sums) bit-exact; the product held to
the checks of tests/refcheck.py against the oracle's fp64 product of the same quantized activations
and 4-bit weights (relative L2 error 5e-3 over all outputs and an element-wise bound: the integer
sums are exact, the scales are applied in fp32 and the output is rounded to bf16).  Outputs are
filled with NaN before every launch, so an output a kernel never writes fails.
"""
import numpy as np
import pytest
import torch

import gemm_w4a16_amd as w
import oracle
import refcheck
import workloads
from test_gpu_parity import G128, NAN16, TOL, bf16_f32, dev, gpu_pack, host, rel_err, say

pytestmark = pytest.mark.gpu


def gpu_quantize(x_bits: np.ndarray):
    M, K = x_bits.shape
    xq, a, xs = w.alloc_act_i8(M, K)
    w.w4a16_quantize_act_i8(dev(x_bits), M, K, xq, a, xs)
    return xq, a, xs


def gpu_w4a8(xq, a, xs, packed, M, N, K) -> np.ndarray:
    codes, scales, mins = packed
    y = torch.full((M, N), NAN16, dtype=torch.int16, device="cuda")
    w.w4a16_gemm_w4a8(G128, xq, a, xs, M, codes, scales, mins, N, K, y)
    return host(y, np.uint16)


def _activation_rows(M, K, seed):
    """Random bf16 rows plus a zero row, a row with exact .5 ties (scale 1) and a row whose largest
    magnitude is negative."""
    x = workloads.activations(M, K, "bf16", seed=seed)
    x[1] = 0
    ties = np.array([0.5, 1.5, 2.5, -2.5, 126.5, -0.5], dtype=np.float32)
    row = np.zeros(K, dtype=np.float32)
    row[:len(ties)] = ties
    row[-1] = 127.0
    x[2] = (row.view(np.uint32) >> 16).astype(np.uint16)      # all exactly bf16
    x[3, 5] = 0xC2C8                                          # -100.0: the row's largest magnitude
    return x


@pytest.mark.parametrize("M,K", [(37, 1152), (5, 128), (300, 4096), (6, 12288), (1, 8192)])
def test_quantize_act_i8_bit_exact(M, K):
    say(f"quantize_act_i8 M={M} K={K}")
    x = _activation_rows(M, K, seed=91) if M >= 4 else workloads.activations(M, K, "bf16", seed=91)
    xq, a, xs = gpu_quantize(x)
    rq, ra, rs = oracle.quantize_act_i8(x)
    np.testing.assert_array_equal(host(xq, np.int8), rq)
    np.testing.assert_array_equal(host(a, np.float32), ra)
    np.testing.assert_array_equal(host(xs, np.float32), rs)


@pytest.mark.parametrize("M,N,K", [(1, 256, 128), (37, 260, 1152), (128, 128, 4096), (130, 500, 640),
                                   (257, 132, 384), (64, 4, 256), (3, 1028, 2048)])
def test_gemm_w4a8_parity(M, N, K):
    """The GEMM alone, fed the oracle's own quantized activations; several tiles and ragged tails
    in M and N (N % 4 == 0), one group (K = 128) to 32."""
    say(f"gemm_w4a8 M={M} N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=92)
    x = _activation_rows(M, K, seed=93) if M >= 4 else workloads.activations(M, K, "bf16", seed=93)
    rq, ra, rs = oracle.quantize_act_i8(x)
    packed = gpu_pack(G128, W)
    y = gpu_w4a8(dev(rq), dev(ra), dev(rs), packed, M, N, K)
    rp = oracle.quantize_g128(W)
    assert rel_err(bf16_f32(y), oracle.matmul_w4a8(rq, ra, *rp)) <= TOL
    err, _ = refcheck.check(bf16_f32(y), refcheck.w4a8(rq, ra, *rp), "bf16")
    say(f"  rel err {err:.3e}")
    if M >= 4:
        np.testing.assert_array_equal(y[1], 0)   # the zero row: a = 1, every code 0, y exactly 0


@pytest.mark.parametrize("M,N,K", [(1, 4, 128), (2, 4100, 4224), (4, 1028, 512), (5, 68, 8192), (16, 1156, 1024),
                                   (16, 20, 384), (7, 132, 4096), (17, 260, 640), (33, 1156, 4224),
                                   (50, 68, 1024), (64, 516, 256), (65, 260, 640)])
def test_gemm_w4a8_few_rows_parity(M, N, K):
    """Up to 64 rows (the weight-streaming kernel, 16 rows per block: one row in the last block at
    17 and 33): one and several 4096-k passes, groups past K in the last pass (4224, 8192), ragged N
    down to 4 columns; 65 rows, the first 128-row-tile shape, beside them.  Full comparison with the oracle on its own quantized activations, then the GPU
    quantizer's codes through the same product, bit for bit against the first."""
    say(f"gemm_w4a8 few rows M={M} N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=102)
    x = _activation_rows(M, K, seed=103) if M >= 4 else workloads.activations(M, K, "bf16", seed=103)
    rq, ra, rs = oracle.quantize_act_i8(x)
    packed = gpu_pack(G128, W)
    y = gpu_w4a8(dev(rq), dev(ra), dev(rs), packed, M, N, K)
    err, _ = refcheck.check(bf16_f32(y), refcheck.w4a8(rq, ra, *oracle.quantize_g128(W)), "bf16")
    say(f"  rel err {err:.3e}")
    if M >= 4:
        np.testing.assert_array_equal(y[1], 0)
    y2 = gpu_w4a8(*gpu_quantize(x), packed, M, N, K)
    np.testing.assert_array_equal(y2, y)


def test_w4a8_decode_full_size():
    """The decode shape (M=1, K=4096, N=14336) in the launch bench.py times: every output
    against the oracle."""
    wl = workloads.DECODE
    M, N, K = wl.M, wl.N, wl.K
    say(f"w4a8 decode M={M} N={N} K={K}")
    W = workloads.weights(N, K, wl.outliers, wl.seed_w)
    x = workloads.activations(M, K, "bf16", seed=wl.seed_x)
    packed = gpu_pack(G128, W)
    y = bf16_f32(gpu_w4a8(*gpu_quantize(x), packed, M, N, K))
    rq, ra, _ = oracle.quantize_act_i8(x)
    rp = oracle.quantize_g128(W)
    assert rel_err(y, oracle.matmul_w4a8(rq, ra, *rp)) <= TOL
    refcheck.check(y, refcheck.w4a8(rq, ra, *rp), "bf16", "w4a8 decode")


@pytest.mark.parametrize("N,K", [(4, 128), (260, 1152), (4100, 4224), (68, 8192), (14336, 4096)])
def test_matmul_w4a8_fused_one_row(N, K):
    """The fused one-row entry point: bit for bit the two-call result (same codes, scales and
    sums, same order of the fp32 epilogue), and within tolerance of the oracle; one and several
    4096-k passes, groups past K, a zero row, a row whose largest magnitude ties an exact .5."""
    say(f"matmul_w4a8 fused M=1 N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=104)
    packed = gpu_pack(G128, W)
    rows = [workloads.activations(1, K, "bf16", seed=105), np.zeros((1, K), dtype=np.uint16),
            _activation_rows(4, K, seed=106)[2:3]]
    for x in rows:
        y2 = gpu_w4a8(*gpu_quantize(x), packed, 1, N, K)
        y1 = torch.full((1, N), NAN16, dtype=torch.int16, device="cuda")
        w.w4a16_matmul_w4a8(G128, dev(x), 1, *packed, N, K, y1)
        y1 = host(y1, np.uint16)
        np.testing.assert_array_equal(y1, y2)
        rq, ra, _ = oracle.quantize_act_i8(x)
        refcheck.check(bf16_f32(y1), refcheck.w4a8(rq, ra, *oracle.quantize_g128(W)), "bf16")


@pytest.mark.parametrize("M,N,K", [(1024, 4096, 256), (257, 11268, 128), (520, 8196, 640)])
def test_gemm_w4a8_wide_tiles(M, N, K):
    """Shapes that take the 128 x 256 tiles (at least 128 of them): ragged M and N (N % 8 == 4 in
    the last), one to five groups.  Sampled outputs against the oracle's own sums, all outputs
    against its product."""
    say(f"gemm_w4a8 wide M={M} N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=99)
    x = _activation_rows(M, K, seed=100)
    packed = gpu_pack(G128, W)
    xq, a, xs = gpu_quantize(x)
    y = bf16_f32(gpu_w4a8(xq, a, xs, packed, M, N, K))
    rq, ra, _ = oracle.quantize_act_i8(x)
    rng = np.random.default_rng(101)
    rows = np.concatenate([rng.integers(0, M, 600), [M - 1] * 4, [0, 1, 2, 3]])
    cols = np.concatenate([rng.integers(0, N, 600), [N - 1, N - 2, N - 3, N - 4], [N - 1] * 4])
    rp = oracle.quantize_g128(W)
    ref = oracle.matmul_w4a8_at(rq, ra, *rp, rows, cols)
    assert rel_err(y[rows, cols], ref) <= TOL
    refcheck.check(y, refcheck.w4a8(rq, ra, *rp), "bf16", "w4a8 wide tiles")
    np.testing.assert_array_equal(y[1], 0)


def test_w4a8_end_to_end_and_repeatable():
    """Quantize on the GPU, then the GEMM: equal to the oracle chain, and bit-identical run to run."""
    M, N, K = 96, 384, 1024
    W = workloads.weights(N, K, seed=94)
    x = workloads.activations(M, K, "bf16", seed=95)
    packed = gpu_pack(G128, W)
    q = gpu_quantize(x)
    y1 = gpu_w4a8(*q, packed, M, N, K)
    y2 = gpu_w4a8(*q, packed, M, N, K)
    np.testing.assert_array_equal(y1, y2)
    rq, ra, _ = oracle.quantize_act_i8(x)
    ref = oracle.matmul_w4a8(rq, ra, *oracle.quantize_g128(W))
    assert rel_err(bf16_f32(y1), ref) <= TOL
    # the activation rounding against the W4A16 product of the same weights: small, not zero
    y16 = oracle.matmul_g128(x, *oracle.quantize_g128(W))
    assert 1e-4 < rel_err(bf16_f32(y1), y16) < 2e-2


def test_w4a8_prefill_full_size():
    """The prefill shape (M=1024, K=4096, N=14336) in the launch bench.py times: sampled outputs
    against the oracle's own sums, all outputs against its product, element by element."""
    wl = workloads.PREFILL
    M, N, K = wl.M, wl.N, wl.K
    say(f"w4a8 prefill M={M} N={N} K={K}")
    W = workloads.weights(N, K, wl.outliers, wl.seed_w)
    x = workloads.activations(M, K, "bf16", seed=wl.seed_x)
    packed = gpu_pack(G128, W)
    xq, a, xs = gpu_quantize(x)
    y = bf16_f32(gpu_w4a8(xq, a, xs, packed, M, N, K))
    rq, ra, _ = oracle.quantize_act_i8(x)
    np.testing.assert_array_equal(host(xq, np.int8), rq)
    rng = np.random.default_rng(96)
    rows, cols = rng.integers(0, M, 256), rng.integers(0, N, 256)
    ref = oracle.matmul_w4a8_at(rq, ra, *oracle.quantize_g128(W), rows, cols)
    samp = y[rows, cols].astype(np.float64)
    assert rel_err(samp, ref) <= TOL
    err, worst = refcheck.check(y, refcheck.w4a8(rq, ra, *oracle.quantize_g128(W)), "bf16", "w4a8 prefill")
    say(f"w4a8 prefill rel err {err:.3e}, worst element at {worst:.2f} of its bound")


def test_w4a8_graph_replays_match_eager():
    M, N, K = 200, 520, 1024
    W = workloads.weights(N, K, seed=97)
    packed = gpu_pack(G128, W)
    xd = dev(workloads.activations(M, K, "bf16", seed=98))
    xq, a, xs = w.alloc_act_i8(M, K)

    def step(y):
        w.w4a16_quantize_act_i8(xd, M, K, xq, a, xs)
        w.w4a16_gemm_w4a8(G128, xq, a, xs, M, *packed, N, K, y)

    y_eager = torch.empty((M, N), dtype=torch.int16, device="cuda")
    step(y_eager)
    ref = host(y_eager, np.uint16).copy()
    y = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(y)
    junk = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for r in range(3):
        y.fill_(0)
        xq.zero_()
        junk.normal_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y, np.uint16), ref, err_msg=f"replay {r}")


def test_w4a8_fused_graph_replays_match_eager():
    """The fused one-row product (its LDS-only barrier included) captured in a HIP graph: every
    replay, with other work and synchronizations in between, equals the eager result bit for bit."""
    N, K = 1028, 4224
    W = workloads.weights(N, K, seed=107)
    packed = gpu_pack(G128, W)
    xd = dev(workloads.activations(1, K, "bf16", seed=108))
    y_eager = torch.empty((1, N), dtype=torch.int16, device="cuda")
    w.w4a16_matmul_w4a8(G128, xd, 1, *packed, N, K, y_eager)
    ref = host(y_eager, np.uint16).copy()
    y = torch.zeros((1, N), dtype=torch.int16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w.w4a16_matmul_w4a8(G128, xd, 1, *packed, N, K, y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w.w4a16_matmul_w4a8(G128, xd, 1, *packed, N, K, y)
    junk = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for r in range(3):
        y.fill_(0)
        junk.normal_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y, np.uint16), ref, err_msg=f"replay {r}")

