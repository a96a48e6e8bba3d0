"""Pins of the CPU oracle to facts other than itself (runs without a GPU).

Each test names what fixes the expected value: a number printed on the pages
(tests/golden/page_numbers.txt), a closed form, brute force over all candidates, an exact
special case, or an independent library conversion (torch / numpy IEEE rounding).  They are
chosen so that a plausible slip in the oracle -- a dropped term, a transposed layout, a wrong
nibble order, a wrong rounding mode, a wrong sign -- fails at least one of them.
"""
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = Path(__file__).parent / "golden" / "page_numbers.txt"


def page_numbers():
    out = {}
    for line in GOLDEN.read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        key, rest = line.split("=", 1)
        out[key.strip()] = float(rest.split("|", 1)[0])
    return out


def torch_bf16_bits(v):
    """bf16 bit patterns of fp32 values by torch's round-to-nearest-even (same shape; a scalar
    gives an int)."""
    a = np.ascontiguousarray(np.atleast_1d(np.asarray(v, dtype=np.float32)))
    out = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return int(out[0]) if np.ndim(v) == 0 else out.reshape(np.shape(v))


def bf16_value(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------------------------
# Number-format conversions, against independent IEEE implementations.
# ---------------------------------------------------------------------------------------------

def _interesting_floats(rng, n):
    bits = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ties = (rng.integers(0, 2**16, size=n // 4, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    ties = ties.view(np.float32)
    ties = ties[np.isfinite(ties)]
    small = (rng.standard_normal(n // 4) * 0.02).astype(np.float32)
    edge = np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, 3.4028235e38, 1e-45, -1e-45, 1.1754942e-38,
                     1.1754944e-38, 65504.0, 65519.996, 65520.0, -65520.0, 6.1035156e-05, 5.9604645e-08,
                     2.9802322e-08, 2.9802326e-08, 8.940697e-08], dtype=np.float32)
    return np.concatenate([f, ties, small, edge]).astype(np.float32)


def test_bf16_rounding_matches_torch():
    vals = _interesting_floats(np.random.default_rng(10), 40000)
    ours = np.array([oracle.f32_to_bf16(v) for v in vals], dtype=np.uint16)
    np.testing.assert_array_equal(ours, torch_bf16_bits(vals))


def test_bf16_widening_all_patterns_matches_torch():
    bits = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    ours = np.array([oracle.bf16_to_f32(int(b)) for b in bits], dtype=np.float32)
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(ours[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.all(np.isnan(ours[np.isnan(ref)]))


def test_f16_rounding_matches_numpy():
    vals = _interesting_floats(np.random.default_rng(11), 40000)
    # add every fp16 tie point in the normal range and a sweep of subnormal ties
    h = np.arange(0x0400, 0x7BFF, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = (np.arange(0x0400, 0x7BFF, 7, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    vals = np.concatenate([vals, ((h + nxt) / 2).astype(np.float32), np.float32(2.0**-24) * np.arange(0.5, 1100, 1, dtype=np.float32)])
    ours = np.array([oracle.f32_to_f16(v) for v in vals], dtype=np.uint16)
    with np.errstate(over="ignore"):  # values past the fp16 range round to infinity, on purpose
        ref = vals.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_f16_widening_all_patterns_matches_numpy():
    bits = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    ours = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(ours[finite], ref[finite])
    assert np.all(np.isinf(ours[np.isinf(ref)]))


def test_magic_number_identities():
    """0x4300|q read as bf16 is 128+q; 0x6400|q read as fp16 is 1024+q (vidyal.ai "Where the time
    goes at M = 1"; anrans "What production kernels do").  The kernels' unpack relies on it."""
    q = np.arange(16, dtype=np.uint16)
    bf = torch.from_numpy((0x4300 | q).view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(bf, 128.0 + q)
    hf = (0x6400 | q).view(np.float16).astype(np.float32)
    np.testing.assert_array_equal(hf, 1024.0 + q)
    for q0 in range(16):
        assert oracle.bf16_to_f32(0x4300 | q0) == 128 + q0
        assert oracle.f16_to_f64(0x6400 | q0) == 1024 + q0


# ---------------------------------------------------------------------------------------------
# Nibble packing and layouts.
# ---------------------------------------------------------------------------------------------

def test_pack_unpack_bijection():
    rng = np.random.default_rng(3)
    words = np.concatenate([rng.integers(0, 2**32, size=20000, dtype=np.uint64),
                            np.array([0, 0xFFFFFFFF, 0x76543210, 0x89ABCDEF], dtype=np.uint64)])
    for w in words:
        assert oracle.pack_word(oracle.unpack_word(int(w))) == int(w)
    for _ in range(2000):
        q = rng.integers(0, 16, size=8).astype(np.uint8)
        np.testing.assert_array_equal(oracle.unpack_word(oracle.pack_word(q)), q)


def test_nibble_j_is_bits_4j():
    """Element j of eight sits at bits 4j..4j+3, the first element lowest (vidyal.ai Step 2:
    row 8r+j of the unpacked tile is nibble j of packed row r; anrans: first element in the
    low 4 bits)."""
    for j in range(8):
        for q in (1, 9, 15):
            codes = np.zeros(8, dtype=np.uint8)
            codes[j] = q
            assert oracle.pack_word(codes) == q << (4 * j)
    np.testing.assert_array_equal(oracle.unpack_word(0x76543210), np.arange(8))


def _grid_group(rng, m_bits, s_bits, n=128):
    """A group whose values lie exactly on m + j*s (bf16-exact m, s), j = 0..15 all present."""
    m = float(bf16_value(m_bits))
    s = float(bf16_value(s_bits))
    j = np.concatenate([np.arange(16), rng.integers(0, 16, size=n - 16)])
    rng.shuffle(j)
    vals = np.array([Fraction(m) + k * Fraction(s) for k in j], dtype=object)
    w = np.array([float(v) for v in vals], dtype=np.float32)
    assert all(Fraction(float(a)) == b for a, b in zip(w, vals)), "grid values must be fp32-exact"
    return w, j


def test_g128_layout_is_k8_by_n():
    """codes are [K/8][N]: word (r, n) holds k = 8r..8r+7 of output column n (vidyal.ai Step 2: a
    K/8 by N packed matrix); scales/mins are [K/128][N]."""
    rng = np.random.default_rng(5)
    N, K = 3, 256
    W = np.zeros((N, K), dtype=np.float32)
    J = np.zeros((N, K), dtype=np.int64)
    params = {}
    for n in range(N):
        for g in range(K // 128):
            m_bits = int(torch_bf16_bits(np.float32(-(n + 1) * 0.125 - g * 0.5)))
            s_bits = torch_bf16_bits(np.float32(2.0 ** -(4 + n + g)))
            w, j = _grid_group(rng, m_bits, s_bits)
            W[n, 128 * g:128 * (g + 1)] = w
            J[n, 128 * g:128 * (g + 1)] = j
            params[(n, g)] = (m_bits, s_bits)
    codes, scales, mins = oracle.quantize_g128(W)
    assert codes.shape == (K // 8, N) and scales.shape == (K // 128, N) and mins.shape == (K // 128, N)
    for r in range(K // 8):
        for n in range(N):
            expect = sum(int(J[n, 8 * r + j]) << (4 * j) for j in range(8))
            assert int(codes[r, n]) == expect
    for (n, g), (m_bits, s_bits) in params.items():
        assert int(mins[g, n]) == m_bits and int(scales[g, n]) == s_bits


# ---------------------------------------------------------------------------------------------
# The G128 quantizer.
# ---------------------------------------------------------------------------------------------

def test_g128_grid_reconstruction_exact():
    """A group on the grid m + j*s with bf16-exact m, s gives codes j and decodes to W bit for
    bit; the group min decodes to exactly the stored minimum (code 0 gives fma(0, s, m) = m)."""
    rng = np.random.default_rng(7)
    for m_val, s_val in [(-0.125, 2.0 ** -6), (0.5, 2.0 ** -3), (-3.0, 0.375), (0.0, 2.0 ** -10),
                         (-0.0078125, 0.0078125 * 3)]:
        m_bits = torch_bf16_bits(np.float32(m_val))
        s_bits = torch_bf16_bits(np.float32(s_val))
        assert float(bf16_value(m_bits)) == m_val and float(bf16_value(s_bits)) == s_val
        w, j = _grid_group(rng, m_bits, s_bits)
        W = w.reshape(1, 128)
        codes, scales, mins = oracle.quantize_g128(W)
        got_q = np.array([oracle.unpack_word(int(codes[r, 0]))[i] for r in range(16) for i in range(8)])
        np.testing.assert_array_equal(got_q, j)
        assert int(scales[0, 0]) == s_bits and int(mins[0, 0]) == m_bits
        What = oracle.dequant_g128(codes, scales, mins, "f32")
        np.testing.assert_array_equal(What.view(np.uint32), W.view(np.uint32))
        np.testing.assert_array_equal(oracle.dequant_g128(codes, scales, mins, "f64"), W.astype(np.float64))


def _g128_check_nearest(W, codes, scales, mins):
    """Brute force: each code is a nearest of the 16 levels m + q*s (exact fp64 distances), up to
    the fp32 rounding of the quotient at near-ties; clamped codes are the nearest in-range level."""
    N, K = W.shape
    G = K // 128
    q = np.zeros((N, K), dtype=np.int64)
    for j in range(8):
        q[:, j::8] = ((codes.T.astype(np.int64) >> (4 * j)) & 0xF)
    s = np.repeat(bf16_value(scales).astype(np.float64).T, 128, axis=1)
    m = np.repeat(bf16_value(mins).astype(np.float64).T, 128, axis=1)
    levels = m[..., None] + np.arange(16)[None, None, :] * s[..., None]       # exact in fp64
    dist = np.abs(W.astype(np.float64)[..., None] - levels)
    best = dist.min(axis=-1)
    mine = np.take_along_axis(dist, q[..., None], axis=-1)[..., 0]
    assert np.all(mine <= best + s * 2.0 ** -20), "a code is not the nearest level"
    return q, s, m


def test_g128_codes_are_nearest_levels_bruteforce():
    W, _ = workloads.inputs(workloads.TINY)
    codes, scales, mins = oracle.quantize_g128(W)
    _g128_check_nearest(W, codes, scales, mins)


def test_g128_codes_clamped_where_bf16_parameters_overshoot():
    """Groups in a narrow band far from zero: bf16(min) can lie more than half a step from the
    true minimum (and bf16(s) slightly off), so (w - m_b)/s_b leaves [0, 15] at the ends.  The
    clamp of the codes (taken with the stored bf16 scale and minimum) must then give the nearest level,
    checked by brute force -- an unclamped or wrapped code would be far from every level."""
    rng = np.random.default_rng(5)
    rows = []
    for base in (1.0, -1.0, 3.0, 0.75):
        for width in (0.002, 0.01, 0.05):
            rows.append(np.float32(base) + np.float32(width) * rng.random(1024, dtype=np.float32))
    W = np.stack(rows).astype(np.float32)
    codes, scales, mins = oracle.quantize_g128(W)
    lo = W.reshape(W.shape[0], -1, 128).min(axis=2)
    s = (W.reshape(W.shape[0], -1, 128).max(axis=2) - lo) / 15
    assert np.any(np.abs(bf16_value(mins).T - lo) > 0.5 * s), "no group exercises the clamp"
    q, _, _ = _g128_check_nearest(W, codes, scales, mins)
    assert q.min() == 0 and q.max() <= 15


def test_g128_scale_and_min_definition():
    """s = bf16((max - min)/15), m = bf16(min) per group of 128 along K (vidyal.ai Step 2), with
    torch's bf16 rounding and numpy's fp32 arithmetic as the independent reference."""
    W, _ = workloads.inputs(workloads.TINY)
    codes, scales, mins = oracle.quantize_g128(W)
    Wg = W.reshape(W.shape[0], -1, 128)
    lo, hi = Wg.min(axis=2), Wg.max(axis=2)
    s = ((hi - lo) / np.float32(15.0)).astype(np.float32)
    np.testing.assert_array_equal(scales, torch_bf16_bits(s).T)
    np.testing.assert_array_equal(mins, torch_bf16_bits(lo).T)


def test_g128_error_bound_every_group():
    """|W - w_hat| <= s/2 up to the bf16 rounding of s and min (the round-to-nearest bound), on every group
    of the tiny workload and of a slice of the decode workload with its x20 outliers."""
    for W in (workloads.inputs(workloads.TINY)[0], workloads.weights(512, 4096, outliers=True)):
        codes, scales, mins = oracle.quantize_g128(W)
        q, s, m = _g128_check_nearest(W, codes, scales, mins)
        What = oracle.dequant_g128(codes, scales, mins, "f64")
        err = np.abs(W.astype(np.float64) - What)
        Wg = W.reshape(W.shape[0], -1, 128).astype(np.float64)
        lo = np.repeat(Wg.min(axis=2), 128, axis=1)
        hi = np.repeat(Wg.max(axis=2), 128, axis=1)
        s_exact = (hi - lo) / 15
        slack = np.abs(m - lo) + 15 * np.abs(s - s_exact)
        inner = (q > 0) & (q < 15)
        assert np.all(err[inner] <= s[inner] / 2 * (1 + 2.0 ** -10))
        assert np.all(err <= s / 2 * (1 + 2.0 ** -10) + slack)
        assert np.all(slack <= 0.1 * s + 1e-30)   # bf16 parameters cost a few % of a step


def test_g128_round_half_to_even_at_exact_midpoints():
    """Exact midpoints m + (j + 1/2)s go to the even neighbour (the reading of "round" as
    round-half-to-even); Python's round() is the independent reference."""
    m_val, s_val = -0.125, 2.0 ** -6
    w = [m_val, m_val + 15 * s_val] + [m_val + (j + 0.5) * s_val for j in range(15)]
    w = np.array(w + [m_val] * (128 - len(w)), dtype=np.float32)
    codes, scales, mins = oracle.quantize_g128(w.reshape(1, 128))
    assert float(bf16_value(scales[0, 0])) == s_val and float(bf16_value(mins[0, 0])) == m_val
    q = [oracle.unpack_word(int(codes[r, 0]))[i] for r in range(16) for i in range(8)]
    for j in range(15):
        assert q[2 + j] == round(j + 0.5), (j, q[2 + j])


def test_g128_degenerate_groups():
    """max == min gives scale 1.0 (anrans gemv_w4 host code), codes 0 and w_hat == min."""
    W = np.zeros((2, 256), dtype=np.float32)
    W[0, :128] = 0.0
    W[0, 128:] = -0.0
    W[1, :128] = 0.3
    W[1, 128:] = -2.5
    codes, scales, mins = oracle.quantize_g128(W)
    assert np.all(scales == 0x3F80)
    assert np.all(codes == 0)
    np.testing.assert_array_equal(mins[:, 0], [0x0000, 0x0000])      # mins are [K/128][N]
    np.testing.assert_array_equal(mins[:, 1], [torch_bf16_bits(np.float32(0.3)), torch_bf16_bits(np.float32(-2.5))])
    What = oracle.dequant_g128(codes, scales, mins, "f32")
    np.testing.assert_array_equal(What[1, :128], bf16_value(mins[0, 1]))
    assert np.all(What[0] == 0.0) and not np.any(np.signbit(What[0]))


def test_g128_dequant_bf16_is_rounded_f32():
    W, _ = workloads.inputs(workloads.TINY)
    c, s, m = oracle.quantize_g128(W)
    np.testing.assert_array_equal(oracle.dequant_g128(c, s, m, "bf16"),
                                  torch_bf16_bits(oracle.dequant_g128(c, s, m, "f32")))
    # fmaf vs the exact value: one fp32 rounding at most
    f32 = oracle.dequant_g128(c, s, m, "f32").astype(np.float64)
    f64 = oracle.dequant_g128(c, s, m, "f64")
    assert np.all(np.abs(f32 - f64) <= np.abs(f64) * 2.0 ** -24)


def test_nonfinite_input_is_rejected():
    W = np.zeros((1, 128), dtype=np.float32)
    W[0, 5] = np.inf
    with pytest.raises(ValueError):
        oracle.quantize_g128(W)
    W = np.zeros((1, 32), dtype=np.float32)
    W[0, 0] = np.nan
    with pytest.raises(ValueError):
        oracle.quantize_q4b32(W)


# ---------------------------------------------------------------------------------------------
# The Q4 block-32 quantizer.
# ---------------------------------------------------------------------------------------------

def test_q4_grid_reconstruction_and_byte_order():
    """Values j*s (fp16-exact s, j in -7..7) give codes j+8 and decode exactly; byte j of a block
    holds weight 2j in its low nibble and 2j+1 in its high nibble (thuongvuho.com: code_lo
    multiplies x[weight_idx], code_hi x[weight_idx + 1])."""
    rng = np.random.default_rng(9)
    for s_val in (2.0 ** -7, 0.01171875, 3.0):
        s_h = np.float16(s_val)
        assert float(s_h) == s_val
        j = np.concatenate([[7, -7], rng.integers(-7, 8, size=62)])
        w = (j * s_val).astype(np.float32).reshape(1, 64)
        codes, scales = oracle.quantize_q4b32(w)
        assert codes.shape == (1, 2, 16) and scales.shape == (1, 2)
        q = j + 8
        for b in range(2):
            for byte in range(16):
                lo, hi = q[32 * b + 2 * byte], q[32 * b + 2 * byte + 1]
                assert int(codes[0, b, byte]) == int(lo) | (int(hi) << 4)
        assert int(scales[0, 0]) == int(s_h.view(np.uint16))
        np.testing.assert_array_equal(oracle.dequant_q4b32(codes, scales, "f32"), w)


def test_q4_codes_are_nearest_levels_and_bound():
    W = workloads.weights(64, 1024, seed=4)
    codes, scales = oracle.quantize_q4b32(W)
    N, K = W.shape
    lo = (codes & 0xF).astype(np.int64).reshape(N, K // 2)
    hi = (codes >> 4).astype(np.int64).reshape(N, K // 2)
    q = np.empty((N, K), dtype=np.int64)
    q[:, 0::2], q[:, 1::2] = lo, hi
    s = np.repeat(scales.view(np.float16).astype(np.float64), 32, axis=1)
    levels = (np.arange(16)[None, None, :] - 8) * s[..., None]
    dist = np.abs(W.astype(np.float64)[..., None] - levels)
    mine = np.take_along_axis(dist, q[..., None], axis=-1)[..., 0]
    assert np.all(mine <= dist.min(axis=-1) + s * 2.0 ** -20)
    assert np.all(mine <= s / 2 * (1 + 2.0 ** -10))      # never clipped: |w|/s <= 7(1 + 2^-11)
    assert q.min() >= 1                                    # code 0 is unreachable with bias 8
    a = np.abs(W).reshape(N, -1, 32).max(axis=2)
    np.testing.assert_array_equal(scales, (a / np.float32(7)).astype(np.float32).astype(np.float16).view(np.uint16))


def test_q4_zero_block():
    W = np.zeros((1, 64), dtype=np.float32)
    W[0, 32:] = np.linspace(-1, 1, 32, dtype=np.float32)
    codes, scales = oracle.quantize_q4b32(W)
    assert int(scales[0, 0]) == 0x3C00
    assert np.all(codes[0, 0] == 0x88)
    assert np.all(oracle.dequant_q4b32(codes, scales, "f32")[0, :32] == 0.0)


def test_q4_dequant_f32_is_exact():
    W = workloads.weights(16, 256, seed=6)
    codes, scales = oracle.quantize_q4b32(W)
    np.testing.assert_array_equal(oracle.dequant_q4b32(codes, scales, "f32").astype(np.float64),
                                  oracle.dequant_q4b32(codes, scales, "f64"))


def _wide_range_weights(N, K, seed):
    """N(0, 0.02) rows scaled by powers of two from 2^-20 to 2^10, so that 16-bit roundings of the
    decoded weights reach fp16's subnormal range, its normal range and bf16's wider exponents."""
    W = workloads.weights(N, K, outliers=True, seed=seed)
    e = np.random.default_rng(seed + 100).integers(-20, 11, size=(N, 1))
    return (W * np.exp2(e).astype(np.float32)).astype(np.float32)


def test_q4_dequant_16bit_kinds_round_the_exact_decode():
    """The bf16 and fp16 reference dequants are the round-to-nearest-even of the exact decode
    (q - 8) * s, here formed by numpy from the packed bytes and converted by torch (bf16) and
    numpy (fp16), including fp16 subnormals and exact ties."""
    W = _wide_range_weights(64, 512, seed=7)
    codes, scales = oracle.quantize_q4b32(W)
    N, K = W.shape
    q = np.empty((N, K), dtype=np.int64)
    q[:, 0::2] = (codes & 0xF).reshape(N, K // 2)
    q[:, 1::2] = (codes >> 4).reshape(N, K // 2)
    s = np.repeat(scales.view(np.float16).astype(np.float32), 32, axis=1)
    exact = ((q - 8).astype(np.float32) * s).astype(np.float32)     # exact: 4 x 11 significant bits
    assert np.count_nonzero(np.abs(exact) < 2.0 ** -14) > 100          # fp16 subnormal results occur
    np.testing.assert_array_equal(oracle.dequant_q4b32(codes, scales, "f32"), exact)
    np.testing.assert_array_equal(oracle.dequant_q4b32(codes, scales, "f16"), exact.astype(np.float16).view(np.uint16))
    np.testing.assert_array_equal(oracle.dequant_q4b32(codes, scales, "bf16"), torch_bf16_bits(exact))
    # the two 16-bit kinds differ on most weights: neither is the other's type
    nz = exact != 0
    assert np.mean(oracle.dequant_q4b32(codes, scales, "f16")[nz] != torch_bf16_bits(exact)[nz]) > 0.9


# ---------------------------------------------------------------------------------------------
# Byte accounting against the numbers the pages print.
# ---------------------------------------------------------------------------------------------

def test_byte_accounting_matches_pages():
    P = page_numbers()
    N, K = 14336, 4096
    code_b, scale_b, min_b = (K // 8) * N * 4, (K // 128) * N * 2, (K // 128) * N * 2
    total = code_b + scale_b + min_b
    assert total == 31_195_136
    assert round(total / 1e6, 1) == P["decode_matrix_mb"]
    assert total * 8 / (N * K) == P["g128_bits_per_weight"]
    assert round(16 / P["g128_bits_per_weight"], 2) == P["g128_max_speedup_vs_bf16"]
    assert (128 // 8) * 64 * 4 == P["tile_128x64_packed_bytes"]
    assert 128 * 64 * 2 == P["tile_128x64_bf16_bytes"]
    # the oracle's own arrays have exactly these sizes
    W = np.zeros((64, 512), dtype=np.float32)
    c, s, m = oracle.quantize_g128(W)
    assert c.nbytes + s.nbytes + m.nbytes == 64 * 512 * P["g128_bits_per_weight"] / 8
    cq, sq = oracle.quantize_q4b32(W)
    assert (cq.nbytes + sq.nbytes) / (64 * 512 / 32) == P["q4_block_bytes"]
    assert round(P["q4_block_fp16_bytes"] / P["q4_block_bytes"], 2) == P["q4_size_ratio"]
    assert 16384 * 16384 // 32 * P["q4_block_bytes"] == P["q4_16384_square_mib"] * 2 ** 20


# ---------------------------------------------------------------------------------------------
# The fp64 matmul reference.
# ---------------------------------------------------------------------------------------------

def _tiny():
    W, x = workloads.inputs(workloads.TINY)
    c, s, m = oracle.quantize_g128(W)
    return W, x, c, s, m


def test_matmul_one_hot_picks_a_weight_column():
    W, x, c, s, m = _tiny()
    K = W.shape[1]
    What = oracle.dequant_g128(c, s, m, "f64")
    for k in (0, 7, 8, 127, 128, 300, K - 1):
        e = np.zeros((1, K), dtype=np.uint16)
        e[0, k] = 0x3F80                                   # bf16 1.0
        np.testing.assert_array_equal(oracle.matmul_g128(e, c, s, m)[0], What[:, k])
        e[0, k] = 0xC000                                   # bf16 -2.0
        np.testing.assert_array_equal(oracle.matmul_g128(e, c, s, m)[0], -2.0 * What[:, k])


def test_matmul_power_of_two_scaling_is_exact():
    W, x, c, s, m = _tiny()
    y = oracle.matmul_g128(x, c, s, m)
    x4 = (x.astype(np.uint32) + (2 << 7)).astype(np.uint16)    # bf16 exponent + 2: times 4
    assert np.all(x != 0)
    np.testing.assert_array_equal(oracle.matmul_g128(x4, c, s, m), 4.0 * y)


def test_matmul_matches_numpy_on_dequantized_weights():
    """A library routine on the oracle's own dequantized weights (different summation order)."""
    W, x, c, s, m = _tiny()
    xf = workloads.bits_to_f32(x, "bf16").astype(np.float64)
    ref = xf @ oracle.dequant_g128(c, s, m, "f64").T
    y = oracle.matmul_g128(x, c, s, m)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    ones = np.full((1, W.shape[1]), 0x3F80, dtype=np.uint16)
    np.testing.assert_allclose(oracle.matmul_g128(ones, c, s, m)[0],
                               oracle.dequant_g128(c, s, m, "f64").sum(axis=1), rtol=1e-13)


def test_matmul_sampled_equals_full():
    W, x, c, s, m = _tiny()
    y = oracle.matmul_g128(x, c, s, m)
    cols = np.array([0, 1, 63, 64, 255])
    np.testing.assert_array_equal(oracle.matmul_g128_at(x, c, s, m, np.zeros(5), cols), y[0, cols])


def test_quantization_error_is_about_ten_percent():
    """Relative error against the original weights: about 10% (vidyal.ai Step 2), matching the
    closed form for N(0, sigma) groups of 128: E[range] ~ 5.19 sigma, step ~ 0.346 sigma, RMS
    rounding error step/sqrt(12) ~ 0.0999 sigma.  The output error is measured over 4 x 1024
    outputs so that its sampling spread (~0.002) stays well inside the tolerance."""
    P = page_numbers()
    W = workloads.weights(1024, 4096)
    x = workloads.activations(4, 4096)
    c, s, m = oracle.quantize_g128(W)
    y_q = oracle.matmul_g128(x, c, s, m)
    y_w = oracle.matmul_original(x, W)
    rel = np.linalg.norm(y_q - y_w) / np.linalg.norm(y_w)
    assert abs(rel - P["quant_rel_error_vs_original"]) <= 0.01, rel
    What = oracle.dequant_g128(c, s, m, "f64")
    rms = np.sqrt(np.mean((What - W) ** 2)) / 0.02
    assert 0.097 <= rms <= 0.103, rms


def test_q4_matmul_special_cases():
    W = workloads.weights(32, 256, seed=8)
    codes, scales = oracle.quantize_q4b32(W)
    What = oracle.dequant_q4b32(codes, scales, "f64")
    x = workloads.activations(2, 256, "f16", seed=3)
    y = oracle.matmul_q4b32(x, codes, scales)
    ref = workloads.bits_to_f32(x, "f16").astype(np.float64) @ What.T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    e = np.zeros((1, 256), dtype=np.uint16)
    e[0, 33] = 0x3C00                                      # fp16 1.0
    np.testing.assert_array_equal(oracle.matmul_q4b32(e, codes, scales)[0], What[:, 33])
    np.testing.assert_array_equal(oracle.matmul_q4b32_at(x, codes, scales, [1, 0], [5, 31]), [y[1, 5], y[0, 31]])
    y_w = oracle.matmul_original(x, W, "f16")
    rel = np.linalg.norm(y - y_w) / np.linalg.norm(y_w)
    assert 0.05 < rel < 0.2                                # symmetric 4-bit, block 32


# ---------------------------------------------------------------------------------------------
# The integer-zero-point format (anrans.github.io "Quantization and GEMV": "The quantization
# formulas" and "W4A16: dequantizing in registers").
# ---------------------------------------------------------------------------------------------

def f16_value(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def half_away(v):
    """Round half away from zero (the page's std::round), from its definition."""
    v = np.asarray(v, dtype=np.float64)
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def _zp_grid_group(rng, s, z, n=128):
    """A group on the grid (j - z) * s, j = 0..15 all present (s fp16-exact, z an integer)."""
    j = np.concatenate([np.arange(16), rng.integers(0, 16, size=n - 16)])
    rng.shuffle(j)
    vals = [(Fraction(int(k) - z) * Fraction(s)) for k in j]
    w = np.array([float(v) for v in vals], dtype=np.float32)
    assert all(Fraction(float(a)) == b for a, b in zip(w, vals)), "grid values must be fp32-exact"
    return w, j


def _zp_codes(codes):
    """[N][K] codes from [N][K/8] words, nibble j of word r = k = 8r + j (the page's layout)."""
    N, K8 = codes.shape
    q = np.zeros((N, K8 * 8), dtype=np.int64)
    for j in range(8):
        q[:, j::8] = (codes.astype(np.int64) >> (4 * j)) & 0xF
    return q


def test_zp_layout_is_n_by_k8_and_grid_is_exact():
    """Words are [N][K/8] with k = 8r + j in nibble j; scales and zero points [N][K/128].  A group
    on the grid (j - z) s gives codes j, zero point z, scale s, and decodes to W bit for bit."""
    rng = np.random.default_rng(21)
    N, K = 3, 256
    W = np.zeros((N, K), dtype=np.float32)
    J = np.zeros((N, K), dtype=np.int64)
    params = {}
    for n in range(N):
        for g in range(K // 128):
            s = 2.0 ** -(5 + n) * (3 if g else 1)
            z = [0, 5, 15, 8, 2, 11][2 * n + g]
            w, j = _zp_grid_group(rng, s, z)
            W[n, 128 * g:128 * (g + 1)] = w
            J[n, 128 * g:128 * (g + 1)] = j
            params[(n, g)] = (s, z)
    codes, scales, zeros = oracle.quantize_g128zp(W)
    assert codes.shape == (N, K // 8) and scales.shape == (N, K // 128) and zeros.shape == (N, K // 128)
    for n in range(N):
        for r in range(K // 8):
            assert int(codes[n, r]) == sum(int(J[n, 8 * r + j]) << (4 * j) for j in range(8))
    for (n, g), (s, z) in params.items():
        assert f16_value(scales[n, g]) == s and f16_value(zeros[n, g]) == z
    np.testing.assert_array_equal(oracle.dequant_g128zp(codes, scales, zeros, "f32").view(np.uint32),
                                  W.view(np.uint32))


def test_zp_scale_and_zero_point_definition():
    """s = fp16((max - min)/15) (numpy's IEEE fp16 rounding), z = round-half-away(-min / s) in
    fp32 (the page's formulas), on random groups with and without outliers."""
    W = workloads.weights(64, 1024, outliers=True, seed=22)
    codes, scales, zeros = oracle.quantize_g128zp(W)
    g = W.reshape(64, 8, 128)
    lo, hi = g.min(axis=2), g.max(axis=2)
    s = ((hi - lo) / np.float32(15.0)).astype(np.float32).astype(np.float16)
    s = np.where(s == 0, np.float16(1.0), s)
    np.testing.assert_array_equal(scales, s.view(np.uint16))
    z = half_away((-lo / s.astype(np.float32)).astype(np.float32))
    np.testing.assert_array_equal(f16_value(zeros), np.clip(z, -2048, 2048))


def test_zp_codes_are_nearest_levels_and_bound():
    """Brute force over the 16 levels (q - z) s in exact fp64: every code is a nearest level, up
    to the fp32 rounding of w/s at near-ties.  And the error bound that follows from the formulas:
    the lowest level is within s/2 of the group minimum (z is rounded), the highest within
    s/2 + 15 |s - s_exact| of the maximum, so |w - w_hat| <= s (1/2 + 15 * 2^-11) everywhere."""
    W = workloads.weights(48, 2048, outliers=True, seed=23)
    codes, scales, zeros = oracle.quantize_g128zp(W)
    q = _zp_codes(codes)
    s = np.repeat(f16_value(scales), 128, axis=1)
    z = np.repeat(f16_value(zeros), 128, axis=1)
    levels = (np.arange(16)[None, None, :] - z[..., None]) * s[..., None]
    dist = np.abs(W.astype(np.float64)[..., None] - levels)
    mine = np.take_along_axis(dist, q[..., None], axis=-1)[..., 0]
    assert np.all(mine <= dist.min(axis=-1) + s * 2.0 ** -20), "a code is not the nearest level"
    err = np.abs(W.astype(np.float64) - oracle.dequant_g128zp(codes, scales, zeros, "f64"))
    assert np.all(err <= s * (0.5 + 15 * 2.0 ** -11) + 1e-12), float((err / s).max())


def test_zp_round_half_away_at_exact_midpoints():
    """Weights at exact midpoints (i + 1/2) s round away from zero, as the page's std::round does
    (round-half-to-even would give the even neighbour)."""
    rng = np.random.default_rng(24)
    s, z = 2.0 ** -7, 6
    w, _ = _zp_grid_group(rng, s, z)
    ties = np.array([(i + 0.5) * s for i in range(-6, 9)], dtype=np.float32)   # inside the range
    w[16:16 + len(ties)] = ties
    codes, scales, zeros = oracle.quantize_g128zp(w.reshape(1, 128))
    assert f16_value(scales[0, 0]) == s and f16_value(zeros[0, 0]) == z
    q = _zp_codes(codes)[0, 16:16 + len(ties)]
    np.testing.assert_array_equal(q, half_away(ties.astype(np.float64) / s) + z)
    assert np.any(q != np.round(ties.astype(np.float64) / s) + z)       # differs from half-to-even


def test_zp_degenerate_and_clamped_zero_point():
    """A constant group gets scale 1 (the page's zero-range rule) and decodes each value to the
    nearest integer; a group whose range is tiny against its distance from zero reaches the zero
    point's clamp at -2048, the most negative integer in [-2048, 2048] that fp16 holds exactly."""
    W = np.zeros((2, 128), dtype=np.float32)
    W[0, :] = 3.3
    W[1, :] = 100.0 + np.arange(128, dtype=np.float32) * 1e-4
    codes, scales, zeros = oracle.quantize_g128zp(W)
    assert f16_value(scales[0, 0]) == 1.0 and f16_value(zeros[0, 0]) == -3.0
    np.testing.assert_array_equal(oracle.dequant_g128zp(codes, scales, zeros, "f64")[0], 3.0)
    assert f16_value(zeros[1, 0]) == -2048.0 and int(zeros[1, 0]) == 0xE800


def test_zp_dequant_f32_is_exact():
    """(q - z) s has at most 12 + 11 significant bits, so the fp32 decode equals the fp64 one."""
    W = workloads.weights(16, 512, outliers=True, seed=25)
    codes, scales, zeros = oracle.quantize_g128zp(W)
    np.testing.assert_array_equal(oracle.dequant_g128zp(codes, scales, zeros, "f32").astype(np.float64),
                                  oracle.dequant_g128zp(codes, scales, zeros, "f64"))


def test_zp_dequant_16bit_kinds_round_the_exact_decode():
    """The bf16 and fp16 reference dequants of the zero-point format are the round-to-nearest-
    even of (q - z) * s, formed here by numpy from the packed words and converted by torch (bf16)
    and numpy (fp16), over a wide exponent range."""
    W = _wide_range_weights(64, 512, seed=27)
    codes, scales, zeros = oracle.quantize_g128zp(W)
    q = _zp_codes(codes)
    s = np.repeat(scales.view(np.float16).astype(np.float32), 128, axis=1)
    z = np.repeat(zeros.view(np.float16).astype(np.float32), 128, axis=1)
    exact = ((q.astype(np.float32) - z) * s).astype(np.float32)
    assert np.count_nonzero(np.abs(exact) < 2.0 ** -14) > 100
    np.testing.assert_array_equal(oracle.dequant_g128zp(codes, scales, zeros, "f32"), exact)
    np.testing.assert_array_equal(oracle.dequant_g128zp(codes, scales, zeros, "f16"),
                                  exact.astype(np.float16).view(np.uint16))
    np.testing.assert_array_equal(oracle.dequant_g128zp(codes, scales, zeros, "bf16"), torch_bf16_bits(exact))
    nz = exact != 0
    assert np.mean(oracle.dequant_g128zp(codes, scales, zeros, "f16")[nz] != torch_bf16_bits(exact)[nz]) > 0.9


def test_zp_matmul_special_cases():
    W = workloads.weights(64, 512, seed=26)
    codes, scales, zeros = oracle.quantize_g128zp(W)
    What = oracle.dequant_g128zp(codes, scales, zeros, "f64")
    x = workloads.activations(3, 512, "f16", seed=4)
    y = oracle.matmul_g128zp(x, codes, scales, zeros)
    ref = workloads.bits_to_f32(x, "f16").astype(np.float64) @ What.T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    e = np.zeros((1, 512), dtype=np.uint16)
    e[0, 130] = 0x3C00                                     # fp16 1.0
    np.testing.assert_array_equal(oracle.matmul_g128zp(e, codes, scales, zeros)[0], What[:, 130])
    np.testing.assert_array_equal(oracle.matmul_g128zp_at(x, codes, scales, zeros, [2, 0], [63, 7]),
                                  [y[2, 63], y[0, 7]])
    xb = workloads.activations(1, 512, "bf16", seed=4)
    np.testing.assert_array_equal(oracle.matmul_g128zp(xb, codes, scales, zeros, "bf16")[0],
                                  workloads.bits_to_f32(xb, "bf16").astype(np.float64)[0] @ What.T)
    # quantization error of the format: the same grid spacing as the min/scale form (range/15),
    # so about 10% of the output against the original weights, as for the group-128 format
    xr = workloads.activations(4, 512, "f16", seed=5)
    y_q = oracle.matmul_g128zp(xr, codes, scales, zeros)
    y_w = oracle.matmul_original(xr, W, "f16")
    rel = np.linalg.norm(y_q - y_w) / np.linalg.norm(y_w)
    assert 0.07 < rel < 0.13, rel


def test_zp_zero_point_rounds_half_away_at_a_tie():
    """-min / s exactly 2.5 (min = -2.5 s, max = 12.5 s): the zero point is 3 by the page's
    std::round; round-half-to-even would give 2."""
    s = 2.0 ** -6
    w = np.linspace(-2.5 * s, 12.5 * s, 128).astype(np.float32)
    w[0], w[-1] = -2.5 * s, 12.5 * s
    codes, scales, zeros = oracle.quantize_g128zp(w.reshape(1, 128))
    assert f16_value(scales[0, 0]) == s and f16_value(zeros[0, 0]) == 3.0


# ---------------------------------------------------------------------------------------------
# W8A16, symmetric per-channel int8 (anrans.github.io "Quantization and GEMV", "Exercises", 1).
# ---------------------------------------------------------------------------------------------

def test_w8_grid_row_is_exact():
    """A row of j * s, j = -127 .. 127, with s a power of two: max|w| / 127 = s exactly, so the
    codes are j and the decode is W bit for bit."""
    rng = np.random.default_rng(51)
    s = 2.0 ** -10
    j = np.concatenate([np.arange(-127, 128), rng.integers(-127, 128, size=1)])
    rng.shuffle(j)
    W = (j * s).astype(np.float32).reshape(1, -1)
    codes, scales = oracle.quantize_w8row(W)
    assert scales[0] == np.float32(s)
    np.testing.assert_array_equal(codes[0].astype(np.int64), j)
    np.testing.assert_array_equal(oracle.dequant_w8row(codes, scales, "f32"), W)


def test_w8_scale_definition_and_nearest_codes():
    """s = max|w| / 127 (numpy fp32 division) per row; every code is the nearest of the 255
    levels q s in exact fp64 (up to the fp32 rounding of w/s at near-ties), so |w - w_hat| <= s/2."""
    W = workloads.weights(24, 1024, outliers=True, seed=52)
    W[3, :] *= -1.0
    W[5, 7] = -1.5                                   # the largest magnitude is negative
    codes, scales = oracle.quantize_w8row(W)
    a = np.abs(W).max(axis=1)
    np.testing.assert_array_equal(scales, (a / np.float32(127.0)).astype(np.float32))
    q = codes.astype(np.int64)
    s = scales.astype(np.float64)[:, None]
    levels = np.arange(-127, 128)[None, None, :] * s[..., None]
    dist = np.abs(W.astype(np.float64)[..., None] - levels)
    mine = np.take_along_axis(dist, (q + 127)[..., None], axis=-1)[..., 0]
    assert np.all(mine <= dist.min(axis=-1) + s * 2.0 ** -20)
    assert np.all(np.abs(W - oracle.dequant_w8row(codes, scales, "f64")) <= s * (0.5 + 2.0 ** -20))


def test_w8_ties_zero_row_and_dequant_kinds():
    s = 2.0 ** -7
    ties = np.array([(i + 0.5) * s for i in range(-20, 20)], dtype=np.float32)
    W = np.zeros((2, 128), dtype=np.float32)
    W[0, :len(ties)] = ties
    W[0, -1] = 127 * s                               # fixes s exactly
    codes, scales = oracle.quantize_w8row(W)
    assert scales[0] == np.float32(s) and scales[1] == 1.0       # an all-zero row gets scale 1
    np.testing.assert_array_equal(codes[0, :len(ties)].astype(np.float64), half_away(ties.astype(np.float64) / s))
    np.testing.assert_array_equal(codes[1], 0)
    W2 = workloads.weights(4, 256, seed=53)
    c2, s2 = oracle.quantize_w8row(W2)
    exact = oracle.dequant_w8row(c2, s2, "f64")
    np.testing.assert_array_equal(exact, c2.astype(np.float64) * s2.astype(np.float64)[:, None])
    f32 = (c2.astype(np.float32) * s2[:, None]).astype(np.float32)       # numpy's IEEE fp32 product
    np.testing.assert_array_equal(oracle.dequant_w8row(c2, s2, "f32"), f32)
    np.testing.assert_array_equal(oracle.dequant_w8row(c2, s2, "f16"), f32.astype(np.float16).view(np.uint16))
    np.testing.assert_array_equal(oracle.dequant_w8row(c2, s2, "bf16"), torch_bf16_bits(f32))


def test_w8_matmul_special_cases_and_error():
    W = workloads.weights(64, 4096, seed=54)
    codes, scales = oracle.quantize_w8row(W)
    What = oracle.dequant_w8row(codes, scales, "f64")
    x = workloads.activations(2, 4096, "f16", seed=6)
    y = oracle.matmul_w8row(x, codes, scales)
    ref = workloads.bits_to_f32(x, "f16").astype(np.float64) @ What.T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    e = np.zeros((1, 4096), dtype=np.uint16)
    e[0, 4095] = 0x3C00
    np.testing.assert_array_equal(oracle.matmul_w8row(e, codes, scales)[0], What[:, 4095])
    # closed form: for N(0, sigma) rows of 4096, max|w| ~ 3.9 sigma, so s ~ 0.031 sigma and the
    # RMS rounding error s / sqrt(12) ~ 0.009 sigma
    rms = np.sqrt(np.mean((What - W) ** 2)) / 0.02
    assert 0.0075 <= rms <= 0.0105, rms


# ---------------------------------------------------------------------------------------------
# W4A8 (vidyal.ai "Low-Precision Kernels", "INT8 on a GeForce chip" and "The cost of quantizing
# activations"): per-row int8 activations, a = max|x| / 127, integer sums per group.
# ---------------------------------------------------------------------------------------------

def _bf16_bits_exact(v):
    """bf16 bits of values that bf16 holds exactly (checked)."""
    b = torch_bf16_bits(np.asarray(v, dtype=np.float32))
    assert np.array_equal(bf16_value(b), np.asarray(v, dtype=np.float32))
    return b


def test_w4a8_grid_rows_quantize_exactly():
    """Rows of j * 2^e (j = -127..127, with |j| = 127 present): a = 2^e exactly, the codes are j and
    a * xq reproduces x; the group sums are the sums of j; a zero row gets a = 1 and codes 0."""
    rng = np.random.default_rng(81)
    M, K = 4, 384
    x = np.zeros((M, K), dtype=np.float32)
    jj = np.zeros((M, K), dtype=np.int64)
    for m, e in enumerate((-6, 0, 3)):
        j = rng.integers(-127, 128, size=K)
        j[rng.integers(0, K)] = 127 if m % 2 else -127
        jj[m] = j
        x[m] = j * 2.0 ** e
    xq, a, xsum = oracle.quantize_act_i8(_bf16_bits_exact(x))
    np.testing.assert_array_equal(a, np.float32([2.0 ** -6, 1.0, 8.0, 1.0]))
    np.testing.assert_array_equal(xq.astype(np.int64), jj)
    np.testing.assert_array_equal(xsum, jj.reshape(M, K // 128, 128).sum(axis=2).T.astype(np.float32))
    np.testing.assert_array_equal(xq[3], 0)


def test_w4a8_ties_go_to_even():
    """With a = 1 (max|x| = 127), x = j + 1/2 must round to the even neighbour."""
    halves = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5, 100.5, -126.5], dtype=np.float32)
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, :len(halves)] = halves
    x[0, -1] = 127.0
    xq, a, _ = oracle.quantize_act_i8(_bf16_bits_exact(x))
    assert a[0] == 1.0
    np.testing.assert_array_equal(xq[0, :len(halves)], [0, 2, 2, 4, 0, -2, -2, -4, 100, -126])


def test_w4a8_codes_are_nearest_and_extremes_hit_127():
    """Random rows: every code is the nearest multiple of a (|x - a xq| <= a/2, up to the fp32
    rounding of x/a, at most 2^-17 for |x/a| <= 128), the largest magnitude maps to +-127 with its
    sign, and a is the fp32 quotient max|x| / 127."""
    x = workloads.activations(16, 1024, "bf16", seed=82)
    xf = bf16_value(x).astype(np.float64)
    xq, a, xsum = oracle.quantize_act_i8(x)
    amax = np.abs(xf).max(axis=1)
    np.testing.assert_array_equal(a, (amax.astype(np.float32) / np.float32(127.0)).astype(np.float32))
    err = np.abs(xf - a.astype(np.float64)[:, None] * xq.astype(np.float64))
    assert np.all(err <= a.astype(np.float64)[:, None] * (0.5 + 2.0 ** -16))
    arg = np.abs(xf).argmax(axis=1)
    top = xq[np.arange(16), arg].astype(np.int64)
    np.testing.assert_array_equal(np.abs(top), 127)
    np.testing.assert_array_equal(np.sign(top), np.sign(xf[np.arange(16), arg]))
    assert np.abs(xq.astype(np.int64)).max() == 127


def test_w4a8_matmul_equals_w4a16_on_grid_activations():
    """When every activation is on its row's int8 grid, a * xq == x exactly, so the W4A8 product
    is the W4A16 reference product bit for bit (same fp64 sums in the same order)."""
    rng = np.random.default_rng(83)
    M, N, K = 3, 40, 512
    x = (rng.integers(-127, 128, size=(M, K)) * 2.0 ** -4).astype(np.float32)
    x[:, 0] = 127 * 2.0 ** -4
    bits = _bf16_bits_exact(x)
    W = workloads.weights(N, K, outliers=True, seed=84)
    codes, scales, mins = oracle.quantize_g128(W)
    xq, a, _ = oracle.quantize_act_i8(bits)
    np.testing.assert_array_equal(oracle.matmul_w4a8(xq, a, codes, scales, mins),
                                  oracle.matmul_g128(bits, codes, scales, mins))


def test_w4a8_matmul_group_form_and_error():
    """The product equals a_m * sum_g (s * sum(xq q) + min * X_g) (integer group sums, exact), the
    sampled entry point agrees, and the activation rounding costs about a / sqrt(12) per term:
    relative error against the W4A16 product well under 2%."""
    M, N, K = 4, 24, 1024
    x = workloads.activations(M, K, "bf16", seed=85)
    W = workloads.weights(N, K, seed=86)
    codes, scales, mins = oracle.quantize_g128(W)
    xq, a, xsum = oracle.quantize_act_i8(x)
    y = oracle.matmul_w4a8(xq, a, codes, scales, mins)
    q = np.zeros((N, K), dtype=np.int64)
    for r in range(K // 8):
        for j in range(8):
            q[:, 8 * r + j] = (codes[r].astype(np.int64) >> (4 * j)) & 0xF
    s = bf16_value(scales).astype(np.float64)            # [G][N]
    mn = bf16_value(mins).astype(np.float64)
    G = K // 128
    ref = np.zeros((M, N))
    for g in range(G):
        iq = xq[:, 128 * g:128 * g + 128].astype(np.int64) @ q[:, 128 * g:128 * g + 128].T   # exact integers
        ref += iq * s[g][None, :] + xsum[g][:, None].astype(np.float64) * mn[g][None, :]
    ref *= a.astype(np.float64)[:, None]
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    rows, cols = np.array([0, 3, 1, 2]), np.array([5, 23, 0, 11])
    np.testing.assert_array_equal(oracle.matmul_w4a8_at(xq, a, codes, scales, mins, rows, cols), y[rows, cols])
    y16 = oracle.matmul_g128(x, codes, scales, mins)
    rel = np.max(np.abs(y - y16)) / np.max(np.abs(y16))
    assert 1e-4 < rel < 2e-2


def test_format_generic_calls_forward_to_each_format():
    """oracle_quantize_pack / oracle_dequant / oracle_matmul_f64 (fmt 0 G128, 1 Q4, 2 zero-point,
    3 W8) return exactly what each format's own pinned function returns, and refuse a third array
    for the formats that have none and an unknown format."""
    L = oracle.lib()
    N, K, M = 5, 256, 3
    W = workloads.weights(N, K, outliers=True, seed=77)
    x16 = workloads.activations(M, K, "f16", seed=78)
    xbf = workloads.activations(M, K, "bf16", seed=79)
    cases = {0: (oracle.quantize_g128(W), xbf, 0), 1: (oracle.quantize_q4b32(W), x16, 1),
             2: (oracle.quantize_g128zp(W), x16, 1), 3: (oracle.quantize_w8row(W), x16, 1)}
    ptr = lambda a: None if a is None else a.ctypes.data
    for fmt, (packed, x, xk) in cases.items():
        packed = tuple(np.ascontiguousarray(a) for a in packed)
        mine = tuple(np.zeros_like(a) for a in packed)
        mins_out = ptr(mine[2]) if len(mine) > 2 else None
        assert L.oracle_quantize_pack(fmt, W.ctypes.data, N, K, ptr(mine[0]), ptr(mine[1]), mins_out) == 0
        for a, b in zip(packed, mine):
            np.testing.assert_array_equal(a, b)
        mins_in = ptr(packed[2]) if len(packed) > 2 else None
        for kind, dt in ((0, np.float32), (2, np.float64)):
            out = np.zeros((N, K), dtype=dt)
            assert L.oracle_dequant(fmt, ptr(packed[0]), ptr(packed[1]), mins_in, N, K, kind, out.ctypes.data) == 0
            ref = {0: oracle.dequant_g128, 1: oracle.dequant_q4b32, 2: oracle.dequant_g128zp,
                   3: oracle.dequant_w8row}[fmt](*packed, "f32" if kind == 0 else "f64")
            np.testing.assert_array_equal(out, ref)
        y = np.zeros((M, N))
        assert L.oracle_matmul_f64(fmt, x.ctypes.data, xk, M, ptr(packed[0]), ptr(packed[1]), mins_in, N, K,
                                   y.ctypes.data) == 0
        xkind = "bf16" if xk == 0 else "f16"
        ref = {0: oracle.matmul_g128, 1: oracle.matmul_q4b32, 2: oracle.matmul_g128zp,
               3: oracle.matmul_w8row}[fmt](x, *packed, x_kind=xkind)
        np.testing.assert_array_equal(y, ref)
        if fmt in (1, 3):   # no third array
            assert L.oracle_quantize_pack(fmt, W.ctypes.data, N, K, ptr(mine[0]), ptr(mine[1]), ptr(mine[0])) != 0
    assert L.oracle_quantize_pack(7, W.ctypes.data, N, K, None, None, None) != 0
