"""Parity of the HIP path (called through the C ABI) with the CPU oracle, on the GPU.

Bars: packing and dequantized weights bit-exact; every matmul output checked against the
oracle's fp64 product with the same 4-bit weights (tests/refcheck.py): a relative error
||y - y_ref||_2 / ||y_ref||_2 <= 5e-3 over all outputs, and an element-wise bound derived from
the arithmetic (output rounding, bf16-rounded weights, fp32 cancellation in the factored forms).
The outputs are filled with NaN before every launch, so an output a kernel never writes fails.
Sizes span several tiles with ragged tails; the full-size workloads (decode, the batch sweep,
prefill, Q4) are compared in full.
"""
import numpy as np
import pytest
import torch

import gemm_w4a16_amd as w
import oracle
import refcheck
import workloads

pytestmark = pytest.mark.gpu

G128, Q4, ZP = w.W4A16_FMT_G128_ASYM_BF16, w.W4A16_FMT_Q4_B32_SYM_FP16, w.W4A16_FMT_G128_ZP_FP16
W8 = w.W4A16_FMT_W8_ROW_FP32
BF16, F16, F32 = w.W4A16_BF16, w.W4A16_FP16, w.W4A16_FP32
TOL = 5e-3


def say(*a):
    print(*a, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    view = {np.dtype(np.uint32): np.int32, np.dtype(np.uint16): np.int16}.get(a.dtype)
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(view) if view else a).cuda()


def host(t: torch.Tensor, dtype) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy().view(dtype)


def rel_err(y, ref) -> float:
    return float(np.linalg.norm(np.asarray(y, np.float64) - ref) / np.linalg.norm(ref))


def bf16_f32(bits):
    return workloads.bits_to_f32(bits, "bf16")


def gpu_pack(fmt, W: np.ndarray):
    N, K = W.shape
    codes, scales, mins = w.alloc_packed(fmt, N, K)
    w.w4a16_quantize_pack(fmt, dev(W), N, K, codes, scales, mins)
    return codes, scales, mins


NAN16 = -1  # 0xFFFF: a NaN in both bf16 and fp16


def run_matmul(fn, fmt, x_bits, packed, N, K, act):
    """y (16-bit patterns) of one call; y is filled with NaN first, so unwritten outputs show."""
    codes, scales, mins = packed
    M = x_bits.shape[0]
    xd = dev(x_bits)
    y = torch.full((M, N), NAN16, dtype=torch.int16, device="cuda")
    if fn is w.w4a16_gemv:
        fn(fmt, act, xd, M, codes, scales, mins, N, K, y)
    else:
        ws, nb = w.alloc_workspace(fmt, M, N, K)
        fn(fmt, act, xd, M, codes, scales, mins, N, K, y, ws, nb)
    return host(y, np.uint16)


# ---------------------------------------------------------------------------------------------
# Quantize/pack and dequant: bit-exact.
# ---------------------------------------------------------------------------------------------

G128_SHAPES = [(256, 512), (1, 128), (3, 256), (65, 384), (200, 1024), (130, 128)]
Q4_SHAPES = [(1, 32), (3, 96), (65, 1024), (130, 4096), (7, 160)]


@pytest.mark.parametrize("N,K", G128_SHAPES)
def test_pack_g128_bit_exact(N, K):
    say(f"pack_g128 N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=N + K)
    W[0, :128] = 0.25                     # a degenerate group (scale 1.0)
    W[-1, -128:] = -0.0
    c, s, m = gpu_pack(G128, W)
    rc, rs, rm = oracle.quantize_g128(W)
    np.testing.assert_array_equal(host(c, np.uint32), rc)
    np.testing.assert_array_equal(host(s, np.uint16), rs)
    np.testing.assert_array_equal(host(m, np.uint16), rm)


def test_pack_g128_rounding_ties_bit_exact():
    """Exact code midpoints over a grid of (scale, min): round-half-to-even, IEEE division."""
    rng = np.random.default_rng(21)
    rows = []
    for s_exp in range(-12, 2):
        for m_val in (-3.0, -0.125, 0.0, 0.4375):
            s = 2.0 ** s_exp * 1.5
            vals = [m_val, m_val + 15 * s] + [m_val + (j + 0.5) * s for j in range(15)]
            vals += list(m_val + rng.integers(0, 31, size=128 - len(vals)) * 0.5 * s)
            rows.append(np.array(vals, dtype=np.float32))
    W = np.stack(rows)
    c, s_, m_ = gpu_pack(G128, W)
    rc, rs, rm = oracle.quantize_g128(W)
    np.testing.assert_array_equal(host(c, np.uint32), rc)
    np.testing.assert_array_equal(host(s_, np.uint16), rs)
    np.testing.assert_array_equal(host(m_, np.uint16), rm)


@pytest.mark.parametrize("N,K", Q4_SHAPES)
def test_pack_q4_bit_exact(N, K):
    say(f"pack_q4 N={N} K={K}")
    W = workloads.weights(N, K, seed=N * 7 + K)
    W[0, :32] = 0.0                       # a zero block (scale 1.0)
    W[-1, -32:] = 1e-7                    # subnormal fp16 scale
    c, s, _ = gpu_pack(Q4, W)
    rc, rs = oracle.quantize_q4b32(W)
    np.testing.assert_array_equal(host(c, np.uint8), rc)
    np.testing.assert_array_equal(host(s, np.uint16), rs)


@pytest.mark.parametrize("dtype,kind,np_t", [(BF16, "bf16", np.uint16), (F32, "f32", np.float32)])
def test_dequant_g128_bit_exact(dtype, kind, np_t):
    W = workloads.weights(130, 384, outliers=True, seed=3)
    c, s, m = gpu_pack(G128, W)
    out = torch.empty((130, 384), dtype=torch.float32 if dtype == F32 else torch.int16, device="cuda")
    w.w4a16_dequant(G128, c, s, m, 130, 384, dtype, out)
    rc, rs, rm = oracle.quantize_g128(W)
    np.testing.assert_array_equal(host(out, np_t), oracle.dequant_g128(rc, rs, rm, kind))


@pytest.mark.parametrize("dtype,kind,np_t", [(F16, "f16", np.uint16), (BF16, "bf16", np.uint16),
                                             (F32, "f32", np.float32)])
def test_dequant_q4_bit_exact(dtype, kind, np_t):
    W = workloads.weights(65, 1024, seed=5)
    c, s, _ = gpu_pack(Q4, W)
    out = torch.empty((65, 1024), dtype=torch.float32 if dtype == F32 else torch.int16, device="cuda")
    w.w4a16_dequant(Q4, c, s, None, 65, 1024, dtype, out)
    rc, rs = oracle.quantize_q4b32(W)
    np.testing.assert_array_equal(host(out, np_t), oracle.dequant_q4b32(rc, rs, kind))


# ---------------------------------------------------------------------------------------------
# Matmul parity at sizes the oracle runs in full.
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("M", [1, 2, 3, 4, 6, 8])
@pytest.mark.parametrize("N,K", [(256, 512), (1, 128), (63, 256), (65, 384), (1000, 2048), (300, 4224)])
def test_gemv_g128_parity(M, N, K):
    say(f"gemv_g128 M={M} N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=11)
    x = workloads.activations(M, K, "bf16", seed=12)
    packed = gpu_pack(G128, W)
    y = run_matmul(w.w4a16_gemv, G128, x, packed, N, K, BF16)
    refcheck.check(bf16_f32(y), refcheck.g128(x, *oracle.quantize_g128(W)), "bf16")


@pytest.mark.parametrize("M,N,K", [(5, 200, 256), (64, 256, 4096), (130, 260, 384), (257, 131, 1024),
                                   (128, 128, 128), (300, 520, 640), (17, 65, 384), (33, 131, 384),
                                   (513, 230, 1152), (50, 97, 1152), (64, 1000, 640),
                                   # 17..32 rows: several groups per wave (K = 4224: 33 groups, one
                                   # wave with 5), waves with no group (K = 128, 256), ragged N
                                   (24, 1000, 4224), (20, 130, 256), (31, 97, 1152), (32, 64, 128),
                                   (32, 260, 2048), (18, 4100, 384),
                                   # 33..64 rows on the 64-row kernel (N % 4 == 0, K % 256 == 0):
                                   # one group pair, ragged last column block, many pairs
                                   (40, 68, 256), (48, 1000, 1024), (63, 4100, 512), (33, 64, 4096),
                                   # 17..32 rows on the 32-row one (N % 4 == 0, K % 512 == 0)
                                   (17, 68, 512), (25, 1000, 1024), (32, 4100, 2048)])
def test_gemm_g128_parity(M, N, K):
    say(f"gemm_g128 M={M} N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=13)
    x = workloads.activations(M, K, "bf16", seed=14)
    packed = gpu_pack(G128, W)
    y = run_matmul(w.w4a16_gemm, G128, x, packed, N, K, BF16)
    refcheck.check(bf16_f32(y), refcheck.g128(x, *oracle.quantize_g128(W)), "bf16")


@pytest.mark.parametrize("M", [65, 100, 128, 129, 200, 400, 600])
@pytest.mark.parametrize("N", [500, 499])
def test_gemm_every_tile_shape(M, N):
    """M at the edges and inside each tile-shape range of the large-M kernel (128x64, 128x128,
    128x256, 256x224),
    with a ragged N that is (500) and is not (499) a multiple of 4 -- the vector and the dword
    copy paths -- and K = 640 (five groups: an odd group count, so some splits are uneven)."""
    K = 640
    say(f"gemm tile shapes M={M} N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=17)
    x = workloads.activations(M, K, "bf16", seed=18)
    packed = gpu_pack(G128, W)
    y = run_matmul(w.w4a16_gemm, G128, x, packed, N, K, BF16)
    refcheck.check(bf16_f32(y), refcheck.g128(x, *oracle.quantize_g128(W)), "bf16")


def test_gemv_long_k_ragged_n():
    """K = 16384 (the skinny kernel makes four passes over K) with N = 999 (not a multiple of 4:
    the scalar column loads) at M = 5."""
    M, N, K = 5, 999, 16384
    say(f"gemv long K M={M} N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=19)
    x = workloads.activations(M, K, "bf16", seed=20)
    packed = gpu_pack(G128, W)
    y = run_matmul(w.w4a16_gemv, G128, x, packed, N, K, BF16)
    refcheck.check(bf16_f32(y), refcheck.g128(x, *oracle.quantize_g128(W)), "bf16")


def test_gemm_many_rows():
    """M = 2048 over few column tiles (K split over whole groups, partials in the workspace): every
    output against the oracle's product, and sampled ones against its own k-ordered sums."""
    M, N, K = 2048, 520, 1024
    say(f"gemm many rows M={M} N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=21)
    x = workloads.activations(M, K, "bf16", seed=22)
    packed = gpu_pack(G128, W)
    y = bf16_f32(run_matmul(w.w4a16_gemm, G128, x, packed, N, K, BF16))
    rc, rs, rm = oracle.quantize_g128(W)
    rng = np.random.default_rng(23)
    rows = np.concatenate([rng.integers(0, M, size=2000), [0, M - 1]])
    cols = np.concatenate([rng.integers(0, N, size=2000), [N - 1, 0]])
    assert rel_err(y[rows, cols], oracle.matmul_g128_at(x, rc, rs, rm, rows, cols)) <= TOL
    refcheck.check(y, refcheck.g128(x, rc, rs, rm), "bf16")


@pytest.mark.parametrize("act", [F16, BF16])
@pytest.mark.parametrize("M,N,K", [(1, 64, 1024), (1, 65, 96), (2, 130, 4096), (1, 257, 2080), (3, 31, 17408)])
def test_gemv_q4_parity(act, M, N, K):
    say(f"gemv_q4 act={act} M={M} N={N} K={K}")
    kind = "f16" if act == F16 else "bf16"
    W = workloads.weights(N, K, seed=15)
    x = workloads.activations(M, K, kind, seed=16)
    packed = gpu_pack(Q4, W)
    y = run_matmul(w.w4a16_gemv, Q4, x, packed, N, K, act)
    refcheck.check(workloads.bits_to_f32(y, kind), refcheck.q4b32(x, *oracle.quantize_q4b32(W), x_kind=kind), kind)


# ---------------------------------------------------------------------------------------------
# The method's degenerate groups through every matmul path.
# ---------------------------------------------------------------------------------------------

def edge_weights(N, K, group, band, seed):
    """Random weights with the groups where the factored and offset forms cancel the most:
    constant groups (max == min: scale 1), all-zero groups (Q4: zero blocks), narrow bands far
    from zero (G128: the code clamp engages; zero-point format: the zero point is clamped), a
    whole zero row, and groups ~1000x larger or smaller than their neighbours."""
    W = workloads.weights(N, K, outliers=True, seed=seed)
    rng = np.random.default_rng(seed + 7)
    G = K // group
    picks = rng.permutation(N * G)[:6 * (N * G // 40)].reshape(6, -1)
    for kind, flat in enumerate(picks):
        for f in flat:
            n, g = divmod(int(f), G)
            sl = slice(group * g, group * (g + 1))
            if kind == 0:
                W[n, sl] = np.float32(rng.choice([0.37, -1.5, 2.0 ** -9]))
            elif kind == 1:
                W[n, sl] = 0.0
            elif kind == 2:
                W[n, sl] = band + np.arange(group, dtype=np.float32) * np.float32(band * 1e-6)
            elif kind == 3:
                W[n, sl] = -band - rng.random(group, dtype=np.float32) * np.float32(band * 1e-6)
            elif kind == 4:
                W[n, sl] *= np.float32(1000.0)
            else:
                W[n, sl] *= np.float32(1e-3)
    W[N // 2] = 0.0
    return W


def edge_activations(M, K, kind, seed):
    """Rows with zeros scattered in (10%), a row spanning a wide exponent range, an all-zero row."""
    xf = workloads.bits_to_f32(workloads.activations(M, K, kind, seed=seed), kind).copy()
    rng = np.random.default_rng(seed + 3)
    xf[rng.random((M, K)) < 0.1] = 0.0
    lo, hi = (-20, 20) if kind == "bf16" else (-10, 3)
    if M >= 2:
        xf[M - 1] *= np.exp2(rng.integers(lo, hi + 1, size=K)).astype(np.float32)
    if M >= 3:
        xf[1] = 0.0
    if kind == "bf16":
        return torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return xf.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("M", [1, 4, 16, 24, 50, 65, 1024])
def test_g128_edge_groups_every_path(M):
    """G128 through the skinny kernel (1, 4, 16 rows), the 32-row and 64-row mid kernels, and the
    large-M GEMM (65 and 1024 rows), on the degenerate groups and wide-range activations."""
    N, K = 1000, 1024
    say(f"g128 edge groups M={M}")
    W = edge_weights(N, K, 128, np.float32(100.0), seed=101)
    x = edge_activations(M, K, "bf16", seed=102)
    rc, rs, rm = oracle.quantize_g128(W)
    packed = gpu_pack(G128, W)
    np.testing.assert_array_equal(host(packed[0], np.uint32), rc)
    y = bf16_f32(run_matmul(w.w4a16_matmul, G128, x, packed, N, K, BF16))
    err, worst = refcheck.check(y, refcheck.g128(x, rc, rs, rm), "bf16", f"edge M={M}")
    say(f"  rel err {err:.3e}, worst element at {worst:.2f} of its bound")
    if M >= 3:
        assert np.all(y[1] == 0)                                   # the zero row
    assert np.all(y[:, N // 2] == 0)                               # the zero weight row


@pytest.mark.parametrize("fmt,M", [(Q4, 1), (Q4, 2), (Q4, 16), (ZP, 1), (ZP, 2), (ZP, 16),
                                   (W8, 1), (W8, 2), (W8, 16)])
def test_row_major_formats_edge_groups(fmt, M):
    """Q4, the zero-point format and W8 on the same kinds of groups, fp16 activations."""
    N, K = 1000, 1024
    say(f"edge groups fmt={fmt} M={M}")
    group = {Q4: 32, ZP: 128, W8: K}[fmt]
    W = edge_weights(N, K, group, np.float32(4.0), seed=103 + fmt)
    x = edge_activations(M, K, "f16", seed=104)
    if fmt == Q4:
        rc, rs = oracle.quantize_q4b32(W)
        ref, packed = refcheck.q4b32(x, rc, rs), (dev(rc), dev(rs), None)
    elif fmt == ZP:
        rc, rs, rz = oracle.quantize_g128zp(W)
        assert np.any(rz.view(np.float16) == -2048)                # clamped zero points present
        ref, packed = refcheck.g128zp(x, rc, rs, rz), (dev(rc), dev(rs), dev(rz))
    else:
        rc, rs = oracle.quantize_w8row(W)
        ref, packed = refcheck.w8row(x, rc, rs), (torch.from_numpy(rc).cuda(), torch.from_numpy(rs).cuda(), None)
    y = workloads.bits_to_f32(run_matmul(w.w4a16_matmul, fmt, x, packed, N, K, F16), "f16")
    err, worst = refcheck.check(y, ref, "f16", f"edge fmt={fmt} M={M}")
    say(f"  rel err {err:.3e}, worst element at {worst:.2f} of its bound")
    # (an all-zero weight row gives a tiny nonzero y here, not an exact 0: the offset forms take
    # sum(x (1024 + q)) - 1032 sum(x) in fp32, and the two sums round differently; the element-wise
    # bound above holds it to 2^-20 B)


@pytest.mark.parametrize("M", [1, 3, 6, 9])
def test_gemv_wide_odd_n_two_passes(M):
    """N = 12289 takes the 64-column blocks of the small-M kernel (chosen from 12225 columns up)
    with scalar column loads (N odd); K = 8192 is two passes of 32 groups."""
    N, K = 12289, 8192
    say(f"gemv wide odd N M={M}")
    W = workloads.weights(N, K, outliers=True, seed=105)
    x = workloads.activations(M, K, "bf16", seed=106)
    rc, rs, rm = oracle.quantize_g128(W)
    packed = (dev(rc), dev(rs), dev(rm))
    y = bf16_f32(run_matmul(w.w4a16_gemv, G128, x, packed, N, K, BF16))
    err, worst = refcheck.check(y, refcheck.g128(x, rc, rs, rm), "bf16", f"wide odd N M={M}")
    say(f"  rel err {err:.3e}, worst element at {worst:.2f} of its bound")


@pytest.mark.parametrize("M,N,K", [(1, 14336, 1024), (16, 14336, 2048), (5, 12289, 2048), (1, 12289, 1536),
                                   (3, 14336, 2176), (9, 12289, 128)])
def test_gemv_wide_short_k(M, N, K):
    """Up to K = 2048 (16 groups) the small-M kernel's waves take one group each per pass; from
    17 groups two, the second pass partial (K = 2176).  64-column blocks, vector (N = 14336) and
    scalar (N odd) column loads."""
    say(f"gemv wide short K M={M} N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=107)
    x = workloads.activations(M, K, "bf16", seed=108)
    rc, rs, rm = oracle.quantize_g128(W)
    packed = (dev(rc), dev(rs), dev(rm))
    y = bf16_f32(run_matmul(w.w4a16_gemv, G128, x, packed, N, K, BF16))
    err, worst = refcheck.check(y, refcheck.g128(x, rc, rs, rm), "bf16", f"wide short K M={M} K={K}")
    say(f"  rel err {err:.3e}, worst element at {worst:.2f} of its bound")


# ---------------------------------------------------------------------------------------------
# Special cases.
# ---------------------------------------------------------------------------------------------

def _one_hot(M, K, ks):
    x = np.zeros((M, K), dtype=np.uint16)
    for m, k in enumerate(ks):
        x[m, k] = 0x3F80
    return x


def test_gemm_one_hot_returns_dequantized_column_exactly():
    """One nonzero term: the GEMM output is the bf16 dequantized weight bit for bit."""
    M, N, K = 130, 200, 512
    W = workloads.weights(N, K, outliers=True, seed=17)
    ks = [(37 * m + 5) % K for m in range(M)]
    packed = gpu_pack(G128, W)
    y = run_matmul(w.w4a16_gemm, G128, _one_hot(M, K, ks), packed, N, K, BF16)
    What = oracle.dequant_g128(*oracle.quantize_g128(W), "bf16")
    for m, k in enumerate(ks):
        np.testing.assert_array_equal(y[m], What[:, k])


def test_gemv_one_hot_within_one_bf16_ulp():
    """The factored GEMV rounds s*(128+q) + (min - 128 s) once more than fmaf(q, s, min)."""
    N, K = 200, 512
    W = workloads.weights(N, K, outliers=True, seed=18)
    packed = gpu_pack(G128, W)
    What = oracle.dequant_g128(*oracle.quantize_g128(W), "f32")
    for k in (0, 1, 127, 128, 300, 511):
        y = bf16_f32(run_matmul(w.w4a16_gemv, G128, _one_hot(1, K, [k]), packed, N, K, BF16))[0]
        ulp = np.abs(What[:, k]) * 2.0 ** -7 + 1e-30
        assert np.all(np.abs(y - What[:, k]) <= ulp)


@pytest.mark.parametrize("path", ["gemv", "gemm", "gemm48"])
def test_power_of_two_scaling_is_exact_and_runs_repeat_bitwise(path):
    M, N, K = {"gemv": (3, 300, 1024), "gemm": (70, 300, 1024), "gemm48": (48, 300, 1024)}[path]
    fn = w.w4a16_gemv if path == "gemv" else w.w4a16_gemm
    W = workloads.weights(N, K, seed=19)
    x = workloads.activations(M, K, "bf16", seed=20)
    packed = gpu_pack(G128, W)
    y1 = run_matmul(fn, G128, x, packed, N, K, BF16)
    y2 = run_matmul(fn, G128, x, packed, N, K, BF16)
    assert np.all(np.isfinite(bf16_f32(y1)))                    # every output written (NaN-filled first)
    np.testing.assert_array_equal(y1, y2)                       # run-to-run bit stability
    x4 = x.copy()
    nz = (x4 & 0x7FFF) != 0
    x4[nz] = x4[nz] + (2 << 7)                                  # bf16 exponent + 2: times 4
    y4 = run_matmul(fn, G128, x4, packed, N, K, BF16)
    np.testing.assert_array_equal(bf16_f32(y4), 4.0 * bf16_f32(y1))


def test_gemm_rows_agree_with_gemv():
    N, K = 512, 2048
    W = workloads.weights(N, K, outliers=True, seed=22)
    x = workloads.activations(64, K, "bf16", seed=23)
    packed = gpu_pack(G128, W)
    yg = bf16_f32(run_matmul(w.w4a16_gemm, G128, x, packed, N, K, BF16))
    for m in (0, 17, 63):
        yv = bf16_f32(run_matmul(w.w4a16_gemv, G128, x[m:m + 1], packed, N, K, BF16))[0]
        assert rel_err(yg[m], yv.astype(np.float64)) <= TOL


@pytest.mark.parametrize("M,N,K,splits", [(1, 4096, 14336, 4), (3, 4096, 14336, 4), (16, 4096, 14336, 4),
                                          (5, 4104, 8192, 3), (2, 4097, 8192, 3)])
def test_matmul_small_n_splits_k(M, N, K, splits):
    """With a workspace, w4a16_matmul splits K over blocks where the small-M kernel's 64-column
    blocks alone would leave CUs idle (N = 4096: 64 blocks) and sums the fp32 partials in split
    order: against the oracle, bitwise repeatable; a ragged last split (G = 64 over 3) and ragged
    column blocks, vector (N = 4104) and scalar (N = 4097) column loads."""
    say(f"small-N K split M={M} N={N} K={K}")
    assert w.w4a16_gemm_workspace_bytes(G128, M, N, K) == splits * M * N * 4
    W = workloads.weights(N, K, outliers=True, seed=109)
    x = workloads.activations(M, K, "bf16", seed=110)
    rc, rs, rm = oracle.quantize_g128(W)
    packed = (dev(rc), dev(rs), dev(rm))
    y = run_matmul(w.w4a16_matmul, G128, x, packed, N, K, BF16)
    np.testing.assert_array_equal(y, run_matmul(w.w4a16_matmul, G128, x, packed, N, K, BF16))
    err, worst = refcheck.check(bf16_f32(y), refcheck.g128(x, rc, rs, rm), "bf16", f"split M={M} N={N}")
    say(f"  rel err {err:.3e}, worst element at {worst:.2f} of its bound")
    # the unsplit GEMV (w4a16_gemv takes no workspace) meets the same bound
    yv = bf16_f32(run_matmul(w.w4a16_gemv, G128, x, packed, N, K, BF16))
    refcheck.check(yv, refcheck.g128(x, rc, rs, rm), "bf16", f"gemv M={M} N={N}")


@pytest.mark.parametrize("M,N,K,splits", [(24, 4096, 8192, 4), (48, 4096, 14336, 4), (64, 4100, 8192, 3),
                                          (17, 2048, 16384, 8),
                                          # K / 128 = 86, not a multiple of 4: 32 rows on the 64-row kernel
                                          (32, 4096, 11008, 4)])
def test_gemm_mid_rows_small_n_splits_k(M, N, K, splits):
    """17..64 rows at small N with a workspace: the R-row kernels split K over blocks (whole
    stages per split; a ragged last split at N = 4100, G = 64 over 3) and the partials are summed
    in split order: against the oracle, bitwise repeatable, and the unsplit kernel (no workspace)
    within the same bound."""
    say(f"mid-rows K split M={M} N={N} K={K}")
    assert w.w4a16_gemm_workspace_bytes(G128, M, N, K) == splits * M * N * 4
    W = workloads.weights(N, K, outliers=True, seed=111)
    x = workloads.activations(M, K, "bf16", seed=112)
    rc, rs, rm = oracle.quantize_g128(W)
    packed = (dev(rc), dev(rs), dev(rm))
    ref = refcheck.g128(x, rc, rs, rm)
    y = run_matmul(w.w4a16_gemm, G128, x, packed, N, K, BF16)
    np.testing.assert_array_equal(y, run_matmul(w.w4a16_matmul, G128, x, packed, N, K, BF16))
    err, worst = refcheck.check(bf16_f32(y), ref, "bf16", f"mid split M={M} N={N}")
    say(f"  rel err {err:.3e}, worst element at {worst:.2f} of its bound")
    codes, scales, mins = packed
    y0 = torch.full((M, N), NAN16, dtype=torch.int16, device="cuda")
    w.w4a16_gemm(G128, BF16, dev(x), M, codes, scales, mins, N, K, y0, None, 0)
    refcheck.check(bf16_f32(host(y0, np.uint16)), ref, "bf16", f"mid unsplit M={M} N={N}")


def test_matmul_dispatch_matches_both_paths():
    N, K = 384, 1024
    W = workloads.weights(N, K, seed=24)
    packed = gpu_pack(G128, W)
    cut = w.w4a16_matmul_gemv_cutoff()
    for M in (1, cut, cut + 1, 33):
        x = workloads.activations(M, K, "bf16", seed=25)
        y = run_matmul(w.w4a16_matmul, G128, x, packed, N, K, BF16)
        assert np.all(np.isfinite(bf16_f32(y)))
        direct = w.w4a16_gemv if M <= cut else w.w4a16_gemm
        np.testing.assert_array_equal(y, run_matmul(direct, G128, x, packed, N, K, BF16))


# ---------------------------------------------------------------------------------------------
# Full-size workloads.
# ---------------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def decode_weights():
    wl = workloads.DECODE
    W = workloads.weights(wl.N, wl.K, wl.outliers, wl.seed_w)
    ref_packed = oracle.quantize_g128(W)
    return W, ref_packed


def test_decode_full_pack_and_gemv(decode_weights):
    wl = workloads.DECODE
    say(f"decode full N={wl.N} K={wl.K}")
    W, (rc, rs, rm) = decode_weights
    packed = gpu_pack(G128, W)
    np.testing.assert_array_equal(host(packed[0], np.uint32), rc)
    np.testing.assert_array_equal(host(packed[1], np.uint16), rs)
    np.testing.assert_array_equal(host(packed[2], np.uint16), rm)
    x = workloads.activations(1, wl.K, "bf16", wl.seed_x)
    y = run_matmul(w.w4a16_matmul, G128, x, packed, wl.N, wl.K, BF16)
    assert rel_err(bf16_f32(y), oracle.matmul_g128(x, rc, rs, rm)) <= TOL    # the oracle's own sums
    err, worst = refcheck.check(bf16_f32(y), refcheck.g128(x, rc, rs, rm), "bf16")
    say(f"decode rel err {err:.3e}, worst element at {worst:.2f} of its bound")


@pytest.mark.parametrize("M", workloads.SWEEP_MS)
def test_sweep_full(decode_weights, M):
    """The batch sweep on the decode weights through the dispatcher, in the launch configuration
    the benchmark times: every output against the oracle's product (and sampled outputs against
    its own k-ordered sums)."""
    wl = workloads.sweep(M)
    say(f"sweep M={M}")
    W, (rc, rs, rm) = decode_weights
    packed = gpu_pack(G128, W)
    _, x = workloads.inputs(wl)
    y = bf16_f32(run_matmul(w.w4a16_matmul, G128, x, packed, wl.N, wl.K, BF16))
    rng = np.random.default_rng(M)
    rows = rng.integers(0, M, size=256)
    cols = rng.integers(0, wl.N, size=256)
    assert rel_err(y[rows, cols], oracle.matmul_g128_at(x, rc, rs, rm, rows, cols)) <= TOL
    err, worst = refcheck.check(y, refcheck.g128(x, rc, rs, rm), "bf16", f"sweep M={M}")
    say(f"  rel err {err:.3e}, worst element at {worst:.2f} of its bound")


def test_prefill_full_gemm(decode_weights):
    """Prefill (M = 1024, K = 4096, N = 14336) as the benchmark launches it: all 14.7 M outputs
    against the oracle's product, element by element, and 1,002 against its own k-ordered sums."""
    wl = workloads.PREFILL
    say(f"prefill M={wl.M} N={wl.N} K={wl.K}")
    W, (rc, rs, rm) = decode_weights
    packed = gpu_pack(G128, W)
    _, x = workloads.inputs(wl)
    y = bf16_f32(run_matmul(w.w4a16_matmul, G128, x, packed, wl.N, wl.K, BF16))
    rng = np.random.default_rng(7)
    rows = np.concatenate([rng.integers(0, wl.M, size=1000), [0, wl.M - 1]])
    cols = np.concatenate([rng.integers(0, wl.N, size=1000), [wl.N - 1, 0]])
    err = rel_err(y[rows, cols], oracle.matmul_g128_at(x, rc, rs, rm, rows, cols))
    say(f"prefill sampled rel err {err:.3e}")
    assert err <= TOL
    err, worst = refcheck.check(y, refcheck.g128(x, rc, rs, rm), "bf16", "prefill")
    say(f"prefill rel err {err:.3e} over all outputs, worst element at {worst:.2f} of its bound")


def test_q4_full_pack_and_gemv():
    wl = workloads.Q4
    say(f"q4 full N={wl.N} K={wl.K}")
    W, x = workloads.inputs(wl)
    packed = gpu_pack(Q4, W)
    rc, rs = oracle.quantize_q4b32(W)
    np.testing.assert_array_equal(host(packed[0], np.uint8), rc)
    np.testing.assert_array_equal(host(packed[1], np.uint16), rs)
    del W
    y = run_matmul(w.w4a16_matmul, Q4, x, packed, wl.N, wl.K, F16)
    assert rel_err(workloads.bits_to_f32(y, "f16"), oracle.matmul_q4b32(x, rc, rs, x_kind="f16")) <= TOL
    err, worst = refcheck.check(workloads.bits_to_f32(y, "f16"), refcheck.q4b32(x, rc, rs), "f16", "q4 full")
    say(f"q4 rel err {err:.3e}, worst element at {worst:.2f} of its bound")


# ---------------------------------------------------------------------------------------------
# The integer-zero-point format: pack and dequant bit-exact, GEMV within the tolerance.
# ---------------------------------------------------------------------------------------------

ZP_SHAPES = [(1, 128), (3, 384), (65, 1024), (130, 4096), (7, 17408), (200, 640)]


@pytest.mark.parametrize("N,K", ZP_SHAPES)
def test_pack_zp_bit_exact(N, K):
    say(f"pack_zp N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=N * 5 + K)
    W[0, :128] = 0.3                      # a degenerate group: scale 1.0, zero point -0
    if N > 1:
        W[1, -128:] = 100.0 + np.arange(128, dtype=np.float32) * 1e-4   # zero point clamped
    W[-1, :128] = np.linspace(-2.5, 12.5, 128, dtype=np.float32) * 2.0 ** -6  # zero-point tie
    c, s, z = gpu_pack(ZP, W)
    rc, rs, rz = oracle.quantize_g128zp(W)
    np.testing.assert_array_equal(host(c, np.uint32), rc)
    np.testing.assert_array_equal(host(s, np.uint16), rs)
    np.testing.assert_array_equal(host(z, np.uint16), rz)


def test_pack_zp_rounding_ties_bit_exact():
    """Codes at exact midpoints (i + 1/2) s round away from zero, on a grid of scales and zero
    points (the page's std::round; IEEE division)."""
    rng = np.random.default_rng(31)
    rows = []
    for s_exp in range(-12, 0):
        for z in (0, 3, 8, 15):
            s = 2.0 ** s_exp
            vals = [-z * s, (15 - z) * s] + [(i + 0.5) * s for i in range(-z, 15 - z)]
            vals += list((rng.integers(0, 31, size=128 - len(vals)) * 0.5 - z) * s)
            rows.append(np.array(vals, dtype=np.float32))
    W = np.stack(rows)
    c, s_, z_ = gpu_pack(ZP, W)
    rc, rs, rz = oracle.quantize_g128zp(W)
    np.testing.assert_array_equal(host(c, np.uint32), rc)
    np.testing.assert_array_equal(host(s_, np.uint16), rs)
    np.testing.assert_array_equal(host(z_, np.uint16), rz)


@pytest.mark.parametrize("dtype,kind,np_t", [(F16, "f16", np.uint16), (BF16, "bf16", np.uint16),
                                             (F32, "f32", np.float32)])
def test_dequant_zp_bit_exact(dtype, kind, np_t):
    N, K = 70, 640
    W = workloads.weights(N, K, outliers=True, seed=41)
    rc, rs, rz = oracle.quantize_g128zp(W)
    out = torch.empty((N, K), dtype=torch.float32 if dtype == F32 else torch.int16, device="cuda")
    w.w4a16_dequant(ZP, dev(rc), dev(rs), dev(rz), N, K, dtype, out)
    np.testing.assert_array_equal(host(out, np_t), oracle.dequant_g128zp(rc, rs, rz, kind))


@pytest.mark.parametrize("act", [F16, BF16])
@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (1, 65, 384), (2, 130, 4096), (3, 257, 2176), (1, 31, 17408),
                                   (16, 100, 1024), (1, 1000, 640)])
def test_gemv_zp_parity(act, M, N, K):
    say(f"gemv_zp act={act} M={M} N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=M + N + K)
    rc, rs, rz = oracle.quantize_g128zp(W)
    kind = "f16" if act == F16 else "bf16"
    x = workloads.activations(M, K, kind, seed=K)
    packed = (dev(rc), dev(rs), dev(rz))
    y = run_matmul(w.w4a16_gemv, ZP, x, packed, N, K, act)
    err, _ = refcheck.check(workloads.bits_to_f32(y, kind), refcheck.g128zp(x, rc, rs, rz, x_kind=kind), kind)
    say(f"  rel err {err:.3e}")
    np.testing.assert_array_equal(run_matmul(w.w4a16_matmul, ZP, x, packed, N, K, act), y)


def test_zp_decode_shape_full_pack_and_gemv(decode_weights):
    """The decode shape (K = 4096, N = 14336, with outliers) in the zero-point format, fp16
    activations: pack bit-exact, GEMV in full against the oracle."""
    wl = workloads.DECODE
    say(f"zp decode shape N={wl.N} K={wl.K}")
    W, _ = decode_weights
    packed = gpu_pack(ZP, W)
    rc, rs, rz = oracle.quantize_g128zp(W)
    np.testing.assert_array_equal(host(packed[0], np.uint32), rc)
    np.testing.assert_array_equal(host(packed[1], np.uint16), rs)
    np.testing.assert_array_equal(host(packed[2], np.uint16), rz)
    x = workloads.activations(1, wl.K, "f16", wl.seed_x)
    y = run_matmul(w.w4a16_matmul, ZP, x, packed, wl.N, wl.K, F16)
    assert rel_err(workloads.bits_to_f32(y, "f16"), oracle.matmul_g128zp(x, rc, rs, rz)) <= TOL
    err, _ = refcheck.check(workloads.bits_to_f32(y, "f16"), refcheck.g128zp(x, rc, rs, rz), "f16", "zp decode")
    say(f"zp decode rel err {err:.3e}")


def test_debug_checks_refuse_unstorable_weights(monkeypatch):
    """W4A16_DEBUG_CHECKS makes w4a16_quantize_pack check a host copy of the weights first: good
    weights pack exactly as without it; a NaN, or a Q4 block whose fp16 scale would overflow, is
    refused with ERR_INVALID before anything is written."""
    N, K = 64, 256
    W = workloads.weights(N, K, outliers=True, seed=501)
    plain = [host(t, np.uint32 if i == 0 else np.uint16) for i, t in enumerate(gpu_pack(G128, W))]
    monkeypatch.setenv("W4A16_DEBUG_CHECKS", "1")
    checked = [host(t, np.uint32 if i == 0 else np.uint16) for i, t in enumerate(gpu_pack(G128, W))]
    for a, b in zip(plain, checked):
        np.testing.assert_array_equal(a, b)
    for fmt, bad in ((G128, np.float32(np.nan)), (Q4, np.float32(1e6)), (ZP, np.float32(np.inf))):
        Wb = W.copy()
        Wb[3, 40] = bad
        codes, scales, mins = w.alloc_packed(fmt, N, K)
        codes.fill_(0x34)
        with pytest.raises(w.W4A16Error) as e:
            w.w4a16_quantize_pack(fmt, dev(Wb), N, K, codes, scales, mins)
        assert e.value.status == w.W4A16_ERR_INVALID
        torch.cuda.synchronize()
        assert bool((codes == 0x34).all())   # refused before any launch


# ---------------------------------------------------------------------------------------------
# The zero-point format's prepared copy: the copy decodes to the oracle's weights bit for bit,
# and its GEMV meets the same bars as the canonical one.
# ---------------------------------------------------------------------------------------------

def gpu_prepare(packed, N, K):
    nb = w.w4a16_prepared_bytes(ZP, N, K)
    prep = torch.empty(nb, dtype=torch.uint8, device="cuda")
    w.w4a16_prepare(ZP, *packed, N, K, prep, nb)
    return prep


def unpack_prepared(prep, N, K):
    """(words [K/8][N], s [K/128][N], m [K/128][N]) of a prepared copy, each part at the next
    16-byte boundary after the previous one."""
    raw = host(prep, np.uint8)
    a16 = lambda b: (b + 15) // 16 * 16
    nw, ng = K // 8 * N * 4, K // 128 * N * 4
    words = raw[:nw].view(np.uint32).reshape(K // 8, N)
    s = raw[a16(nw):a16(nw) + ng].view(np.float32).reshape(K // 128, N)
    m = raw[a16(nw) + a16(ng):a16(nw) + a16(ng) + ng].view(np.float32).reshape(K // 128, N)
    return words, s, m


@pytest.mark.parametrize("N,K", [(1, 128), (3, 384), (65, 1024), (130, 4096), (7, 17408)])
def test_prepared_copy_decodes_to_the_oracle_weights(N, K):
    """Every weight q s + m of the copy (exact in fp32, so any rounding order gives it) equals the
    oracle's fp32 (q - z) s, on weights with degenerate and clamped zero-point groups."""
    say(f"prepare zp N={N} K={K}")
    W = edge_weights(N, K, 128, np.float32(4.0), seed=N + K) if N >= 40 else \
        workloads.weights(N, K, outliers=True, seed=N + K)
    rc, rs, rz = oracle.quantize_g128zp(W)
    words, s, m = unpack_prepared(gpu_prepare((dev(rc), dev(rs), dev(rz)), N, K), N, K)
    np.testing.assert_array_equal(words, rc.T)                      # [K/8][N] column order
    q = ((words.T[:, :, None] >> (4 * np.arange(8, dtype=np.uint32))) & 15).reshape(N, K).astype(np.float32)
    sk = np.repeat(s.T, 128, axis=1)
    mk = np.repeat(m.T, 128, axis=1)
    np.testing.assert_array_equal((q * sk + mk).view(np.uint32),
                                  oracle.dequant_g128zp(rc, rs, rz, "f32").view(np.uint32))
    np.testing.assert_array_equal(s.T, rs.view(np.float16).astype(np.float32))


@pytest.mark.parametrize("act", [F16, BF16])
@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (1, 65, 384), (2, 130, 4096), (3, 257, 2176), (1, 31, 17408),
                                   (4, 1000, 640), (5, 1000, 1152), (16, 100, 1024), (16, 13001, 256),
                                   (17, 300, 1024), (40, 1000, 640), (32, 129, 384), (49, 62, 256),
                                   # one 64-row pass; 64 + 20 rows (the 32-row kernel); 64 + 64 + 8
                                   # rows (the small-M kernel last); 17..32 rows on the R = 32 kernel
                                   (64, 260, 1024), (40, 1000, 512), (84, 68, 256), (136, 260, 512),
                                   (32, 260, 512), (20, 1000, 2048)])
def test_gemv_prepared_zp_parity(act, M, N, K):
    say(f"gemv_prepared act={act} M={M} N={N} K={K}")
    W = edge_weights(N, K, 128, np.float32(4.0), seed=M + N + K)
    rc, rs, rz = oracle.quantize_g128zp(W)
    kind = "f16" if act == F16 else "bf16"
    x = edge_activations(M, K, kind, seed=K + 1)
    prep = gpu_prepare((dev(rc), dev(rs), dev(rz)), N, K)
    xd = dev(x)
    ys = []
    for _ in range(2):
        y = torch.full((M, N), NAN16, dtype=torch.int16, device="cuda")
        w.w4a16_gemv_prepared(ZP, act, xd, M, prep, N, K, y)
        ys.append(host(y, np.uint16))
    np.testing.assert_array_equal(ys[0], ys[1])                     # bitwise reproducible
    err, worst = refcheck.check(workloads.bits_to_f32(ys[0], kind), refcheck.g128zp(x, rc, rs, rz, x_kind=kind),
                                kind, f"prepared M={M} N={N} K={K}")
    say(f"  rel err {err:.3e}, worst element at {worst:.2f} of its bound")


@pytest.mark.parametrize("M", [1, 16, 32, 64])
def test_gemv_prepared_zp_decode_shape(decode_weights, M):
    """The decode shape (K = 4096, N = 14336) from the prepared copy, fp16 activations, in full."""
    wl = workloads.ZP_DECODE
    say(f"prepared zp decode M={M}")
    W, _ = decode_weights
    packed = gpu_pack(ZP, W)
    rc, rs, rz = oracle.quantize_g128zp(W)
    prep = gpu_prepare(packed, wl.N, wl.K)
    x = workloads.activations(M, wl.K, "f16", wl.seed_x)
    y = torch.full((M, wl.N), NAN16, dtype=torch.int16, device="cuda")
    w.w4a16_gemv_prepared(ZP, F16, dev(x), M, prep, wl.N, wl.K, y)
    y = workloads.bits_to_f32(host(y, np.uint16), "f16")
    err, worst = refcheck.check(y, refcheck.g128zp(x, rc, rs, rz), "f16", f"prepared zp decode M={M}")
    say(f"  rel err {err:.3e}, worst element at {worst:.2f} of its bound")


# ---------------------------------------------------------------------------------------------
# W8A16 per-row int8: pack and dequant bit-exact, GEMV within the tolerance.
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(1, 16), (3, 48), (65, 1024), (130, 4096), (5, 17408), (300, 272)])
def test_pack_w8_bit_exact(N, K):
    say(f"pack_w8 N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=N * 3 + K)
    W[0, :] = 0.0                          # an all-zero row: scale 1.0
    if N > 2:
        W[1, ::2] = np.float32(2.0 ** -7) * (np.arange(K // 2) % 64 - 32 + 0.5)  # exact ties
        W[1, 1] = np.float32(2.0 ** -7 * 127)
    c, s, _ = gpu_pack(W8, W)
    rc, rs = oracle.quantize_w8row(W)
    np.testing.assert_array_equal(host(c, np.int8), rc)
    np.testing.assert_array_equal(host(s, np.float32), rs)


@pytest.mark.parametrize("dtype,kind,np_t", [(F16, "f16", np.uint16), (BF16, "bf16", np.uint16),
                                             (F32, "f32", np.float32)])
def test_dequant_w8_bit_exact(dtype, kind, np_t):
    N, K = 70, 528
    rc, rs = oracle.quantize_w8row(workloads.weights(N, K, outliers=True, seed=61))
    out = torch.empty((N, K), dtype=torch.float32 if dtype == F32 else torch.int16, device="cuda")
    w.w4a16_dequant(W8, torch.from_numpy(rc).cuda(), torch.from_numpy(rs).cuda(), None, N, K, dtype, out)
    np.testing.assert_array_equal(host(out, np_t), oracle.dequant_w8row(rc, rs, kind))


@pytest.mark.parametrize("M,N,K", [(1, 64, 16), (1, 65, 496), (2, 130, 4096), (3, 257, 2064), (1, 31, 17408),
                                   (16, 100, 1024), (1, 1000, 640)])
def test_gemv_w8_parity(M, N, K):
    say(f"gemv_w8 M={M} N={N} K={K}")
    rc, rs = oracle.quantize_w8row(workloads.weights(N, K, outliers=True, seed=M + 2 * N + K))
    x = workloads.activations(M, K, "f16", seed=K + 1)
    packed = (torch.from_numpy(rc).cuda(), torch.from_numpy(rs).cuda(), None)
    y = run_matmul(w.w4a16_gemv, W8, x, packed, N, K, F16)
    err, _ = refcheck.check(workloads.bits_to_f32(y, "f16"), refcheck.w8row(x, rc, rs), "f16")
    say(f"  rel err {err:.3e}")
    np.testing.assert_array_equal(run_matmul(w.w4a16_matmul, W8, x, packed, N, K, F16), y)


def test_w8_decode_shape_full_pack_and_gemv(decode_weights):
    wl = workloads.DECODE
    say(f"w8 decode shape N={wl.N} K={wl.K}")
    W, _ = decode_weights
    packed = gpu_pack(W8, W)
    rc, rs = oracle.quantize_w8row(W)
    np.testing.assert_array_equal(host(packed[0], np.int8), rc)
    np.testing.assert_array_equal(host(packed[1], np.float32), rs)
    x = workloads.activations(1, wl.K, "f16", wl.seed_x)
    y = run_matmul(w.w4a16_matmul, W8, x, packed, wl.N, wl.K, F16)
    assert rel_err(workloads.bits_to_f32(y, "f16"), oracle.matmul_w8row(x, rc, rs)) <= TOL
    err, _ = refcheck.check(workloads.bits_to_f32(y, "f16"), refcheck.w8row(x, rc, rs), "f16", "w8 decode")
    say(f"w8 decode rel err {err:.3e}")


# ---------------------------------------------------------------------------------------------
# The row-major formats (Q4, zero point, W8) with several fp16 activation rows: one weight pass
# for up to 64 rows on the fp16 matrix cores, through w4a16_gemv (up to 16 rows) and w4a16_gemm.
# ---------------------------------------------------------------------------------------------

def _rowfmt_pack(fmt, W):
    if fmt == Q4:
        rc, rs = oracle.quantize_q4b32(W)
        return (dev(rc), dev(rs), None), (lambda x: refcheck.q4b32(x, rc, rs))
    if fmt == ZP:
        rc, rs, rz = oracle.quantize_g128zp(W)
        return (dev(rc), dev(rs), dev(rz)), (lambda x: refcheck.g128zp(x, rc, rs, rz))
    rc, rs = oracle.quantize_w8row(W)
    return (torch.from_numpy(rc).cuda(), torch.from_numpy(rs).cuda(), None), (lambda x: refcheck.w8row(x, rc, rs))


@pytest.mark.parametrize("fmt", [Q4, ZP, W8])
@pytest.mark.parametrize("M,N,K", [(2, 1000, 1152), (3, 65, 4224), (4, 1000, 1152), (4, 200, 16384), (3, 70, 8320),
                                   (8, 1000, 1152), (16, 130, 2048), (17, 1000, 1152),
                                   (33, 200, 640), (64, 1000, 1152), (65, 70, 1152), (130, 300, 512)])
def test_rowmajor_formats_many_rows(fmt, M, N, K):
    """Ragged N (64-row blocks), K with a partial last unit of 4 blocks for Q4 and W8 (1152 = 36
    Q4 blocks, 72 W8 blocks; 4224 = 132 and 264), the row-major GEMV's multi-row passes (two rows
    for the zero-point format, up to four for Q4 and W8, three of four real; K = 16384 and 8320
    give each wave several K-slices, the last one partial), one to three activation tiles of 16
    rows, and above 64 rows two passes over the weights.  Every output element-wise against the
    oracle."""
    say(f"rowmajor many rows fmt={fmt} M={M} N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=300 + M + fmt)
    x = workloads.activations(M, K, "f16", seed=301 + M)
    packed, ref = _rowfmt_pack(fmt, W)
    fn = w.w4a16_gemv if M <= w.w4a16_gemv_max_rows() else w.w4a16_gemm
    y = run_matmul(fn, fmt, x, packed, N, K, F16)
    err, worst = refcheck.check(workloads.bits_to_f32(y, "f16"), ref(x), "f16", f"fmt={fmt} M={M}")
    say(f"  rel err {err:.3e}, worst element at {worst:.2f} of its bound")
    np.testing.assert_array_equal(run_matmul(w.w4a16_matmul, fmt, x, packed, N, K, F16), y)   # same kernel


@pytest.mark.parametrize("fmt,M", [(Q4, 5), (W8, 5), (Q4, 40), (W8, 40)])
def test_rowmajor_ragged_last_unit(fmt, M):
    """K = 1120: 35 Q4 blocks (70 W8 blocks), so the last unit of 4 blocks is partial and its
    missing blocks meet zero activations."""
    N, K = 130, 1120
    say(f"rowmajor ragged unit fmt={fmt} M={M}")
    W = workloads.weights(N, K, outliers=True, seed=320 + fmt)
    x = workloads.activations(M, K, "f16", seed=321)
    packed, ref = _rowfmt_pack(fmt, W)
    y = run_matmul(w.w4a16_matmul, fmt, x, packed, N, K, F16)
    refcheck.check(workloads.bits_to_f32(y, "f16"), ref(x), "f16", f"ragged fmt={fmt} M={M}")


@pytest.mark.parametrize("fmt,M", [(ZP, 2), (ZP, 8), (ZP, 16), (ZP, 64), (W8, 3), (W8, 16), (Q4, 4), (Q4, 16)])
def test_rowmajor_decode_shape_many_rows(decode_weights, fmt, M):
    """The decode weights (K = 4096, N = 14336, with outliers) in the zero-point and W8 formats,
    and Q4, with 2 to 64 rows of fp16 activations, as the benchmark runs them."""
    wl = workloads.DECODE
    say(f"rowmajor decode shape fmt={fmt} M={M}")
    W, _ = decode_weights
    packed, ref = _rowfmt_pack(fmt, W)
    x = workloads.activations(M, wl.K, "f16", wl.seed_x, rows_drawn=max(workloads.SWEEP_MS))
    y = run_matmul(w.w4a16_matmul, fmt, x, packed, wl.N, wl.K, F16)
    err, worst = refcheck.check(workloads.bits_to_f32(y, "f16"), ref(x), "f16", f"decode fmt={fmt} M={M}")
    say(f"  rel err {err:.3e}, worst element at {worst:.2f} of its bound")


@pytest.mark.parametrize("fmt", [Q4, ZP])
@pytest.mark.parametrize("M", [5, 6, 7, 16])
def test_rowmajor_bf16_row_passes(fmt, M):
    """bf16 activations with the 4-bit row-major formats: passes of up to four rows (two for the
    zero-point format) over the weights, the last one with one, two or three rows; every output
    element-wise against the oracle, and the same bits as the one-row passes give each row."""
    N, K = 300, 2176
    say(f"rowmajor bf16 row passes fmt={fmt} M={M}")
    W = workloads.weights(N, K, outliers=True, seed=330 + fmt)
    x = workloads.activations(M, K, "bf16", seed=331 + M)
    if fmt == Q4:
        rc, rs = oracle.quantize_q4b32(W)
        packed, ref = (dev(rc), dev(rs), None), refcheck.q4b32(x, rc, rs, x_kind="bf16")
    else:
        rc, rs, rz = oracle.quantize_g128zp(W)
        packed, ref = (dev(rc), dev(rs), dev(rz)), refcheck.g128zp(x, rc, rs, rz, x_kind="bf16")
    y = run_matmul(w.w4a16_gemv, fmt, x, packed, N, K, BF16)
    refcheck.check(workloads.bits_to_f32(y, "bf16"), ref, "bf16", f"bf16 rows fmt={fmt} M={M}")
    for m in (0, M - 1):
        np.testing.assert_array_equal(run_matmul(w.w4a16_gemv, fmt, x[m:m + 1], packed, N, K, BF16)[0], y[m])


def test_rowmajor_bf16_rows_rejected_above_gemv():
    """bf16 activations with the row-major formats run on the row-major GEMV up to 16 rows; the
    large-M path takes fp16 activations only."""
    N, K = 64, 128
    W = workloads.weights(N, K, seed=310)
    packed, _ = _rowfmt_pack(ZP, W)
    x = workloads.activations(17, K, "bf16", seed=311)
    with pytest.raises(w.W4A16Error) as e:
        run_matmul(w.w4a16_gemm, ZP, x, packed, N, K, BF16)
    assert e.value.status == w.W4A16_ERR_UNSUPPORTED


# ---------------------------------------------------------------------------------------------
# HIP-graph capture (the benchmark replays its steps from a graph): every replay bit-identical
# to the eager call, with eager work and synchronisations between the replays.
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,act,M,N,K", [(G128, BF16, 1, 1000, 2048), (G128, BF16, 40, 520, 1024),
                                           (G128, BF16, 300, 256, 4096), (Q4, F16, 2, 300, 1024),
                                           (ZP, F16, 1, 300, 4096), (W8, F16, 3, 130, 512),
                                           (ZP, F16, 40, 300, 1024), (Q4, F16, 9, 200, 1024)])
def test_graph_replays_match_eager(fmt, act, M, N, K):
    say(f"graph replay fmt={fmt} M={M} N={N} K={K}")
    W = workloads.weights(N, K, outliers=True, seed=71)
    codes, scales, mins = gpu_pack(fmt, W)
    kind = "bf16" if act == BF16 else "f16"
    xd = dev(workloads.activations(M, K, kind, seed=72))
    ws, nb = w.alloc_workspace(fmt, M, N, K)
    y_eager = torch.empty((M, N), dtype=torch.int16, device="cuda")
    w.w4a16_matmul(fmt, act, xd, M, codes, scales, mins, N, K, y_eager, ws, nb)
    ref = host(y_eager, np.uint16).copy()
    y = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w.w4a16_matmul(fmt, act, xd, M, codes, scales, mins, N, K, y, ws, nb)  # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w.w4a16_matmul(fmt, act, xd, M, codes, scales, mins, N, K, y, ws, nb)
    junk = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for r in range(3):
        y.fill_(0)
        junk.normal_()                     # unrelated eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y, np.uint16), ref, err_msg=f"replay {r}")
