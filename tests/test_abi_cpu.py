"""The C ABI without a GPU: the library loads, exports every symbol the header declares, and
rejects bad arguments on the host before anything touches a device (no compute calls here)."""
import ctypes
import re
from pathlib import Path

import pytest

import gemm_w4a16_amd as w

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "w4a16.h"

G128, Q4 = w.W4A16_FMT_G128_ASYM_BF16, w.W4A16_FMT_Q4_B32_SYM_FP16
BF16, F16, F32 = w.W4A16_BF16, w.W4A16_FP16, w.W4A16_FP32
FAKE = 0x10000   # a 16-byte-aligned address that is never dereferenced: every call below fails validation


def declared_functions():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:const char\*|w4a16_status_t|int64_t|size_t)\s+(w4a16_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(w.EXPORTED)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(w.library_path)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    assert w.status_string(0) == "ok"
    for s in (1, 2, 3):
        assert w.status_string(s) and w.status_string(s) != "ok"
    assert w.status_string(99) == "unknown status"


def test_packed_sizes_match_the_formats():
    # G128: 4 bits per weight + bf16 scale and minimum per 128 (the decode matrix is 31,195,136 B)
    assert w.w4a16_packed_sizes(G128, 14336, 4096) == (29_360_128, 917_504, 917_504)
    # Q4: 16 B of codes + 2 B scale per 32 weights (16384^2: 144 MiB in all)
    c, s, m = w.w4a16_packed_sizes(Q4, 16384, 16384)
    assert (c, s, m) == (134_217_728, 16_777_216, 0) and c + s == 144 * 2 ** 20
    # an odd scale count is padded to whole 4-byte words (the GEMM reads scales as aligned words)
    assert w.w4a16_packed_sizes(G128, 1, 128) == (64, 4, 4)
    assert w.w4a16_packed_sizes(G128, 3, 384) == (576, 20, 20)
    assert w.w4a16_packed_sizes(G128, 2, 128) == (128, 4, 4)
    assert w.w4a16_packed_sizes(Q4, 1, 32) == (16, 2, 0)


@pytest.mark.parametrize("fmt,N,K", [(G128, 0, 128), (G128, 5, 0), (G128, 5, 64), (G128, 5, 200), (Q4, 5, 48),
                                     (Q4, -1, 32), (7, 5, 128), (G128, 1 << 31, 128)])
def test_packed_sizes_rejects_bad_shapes(fmt, N, K):
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_packed_sizes(fmt, N, K)
    assert e.value.status == w.W4A16_ERR_INVALID


def test_extents_past_the_32_bit_offsets_are_unsupported():
    """N above 2^26 or K above 2^22 would overflow the kernels' 32-bit per-lane byte offsets: every
    entry point refuses them before any launch (the limits themselves are accepted)."""
    big_n, big_k = (1 << 26) + 64, (1 << 22) + 128
    assert w.w4a16_packed_sizes(G128, 1 << 26, 128)[0] == (1 << 26) * 64
    assert w.w4a16_packed_sizes(G128, 64, 1 << 22)[0] == 64 * (1 << 21)
    for fmt, n, k in [(G128, big_n, 128), (G128, 64, big_k), (Q4, big_n, 32), (Q4, 64, big_k)]:
        assert _status(w.w4a16_packed_sizes, fmt, n, k) == w.W4A16_ERR_UNSUPPORTED
    mins = lambda fmt: FAKE if fmt == G128 else None
    act = lambda fmt: BF16 if fmt == G128 else F16
    for fmt, n, k in [(G128, big_n, 128), (G128, 64, big_k), (Q4, 64, big_k)]:
        assert _status(w.w4a16_gemv, fmt, act(fmt), FAKE, 1, FAKE, FAKE, mins(fmt), n, k, FAKE, 0) \
            == w.W4A16_ERR_UNSUPPORTED
        assert _status(w.w4a16_quantize_pack, fmt, FAKE, n, k, FAKE, FAKE, mins(fmt), 0) == w.W4A16_ERR_UNSUPPORTED
        assert _status(w.w4a16_dequant, fmt, FAKE, FAKE, mins(fmt), n, k, BF16, FAKE, 0) == w.W4A16_ERR_UNSUPPORTED
    for n, k in [(big_n, 128), (64, big_k)]:
        assert _status(w.w4a16_gemm, G128, BF16, FAKE, 300, FAKE, FAKE, FAKE, n, k, FAKE, FAKE, 1 << 40, 0) \
            == w.W4A16_ERR_UNSUPPORTED


def test_matmul_w4a8_validation():
    f = w.w4a16_matmul_w4a8
    assert _status(f, G128, FAKE, 0, FAKE, FAKE, FAKE, 256, 128, FAKE, 0) == w.W4A16_ERR_INVALID       # M
    assert _status(f, G128, FAKE + 2, 1, FAKE, FAKE, FAKE, 256, 128, FAKE, 0) == w.W4A16_ERR_INVALID   # x
    assert _status(f, G128, FAKE, 1, FAKE, FAKE, None, 256, 128, FAKE, 0) == w.W4A16_ERR_INVALID       # mins
    assert _status(f, G128, FAKE, 1, FAKE, FAKE, FAKE, 256, 100, FAKE, 0) == w.W4A16_ERR_INVALID       # K % 128
    assert _status(f, G128, FAKE, 2, FAKE, FAKE, FAKE, 256, 128, FAKE, 0) == w.W4A16_ERR_UNSUPPORTED   # one row
    assert _status(f, G128, FAKE, 1, FAKE, FAKE, FAKE, 258, 128, FAKE, 0) == w.W4A16_ERR_UNSUPPORTED   # N % 4
    assert _status(f, Q4, FAKE, 1, FAKE, FAKE, None, 256, 128, FAKE, 0) == w.W4A16_ERR_UNSUPPORTED     # G128 only


def _status(fn, *args):
    try:
        fn(*args)
    except w.W4A16Error as e:
        return e.status
    return w.W4A16_OK


def test_quantize_pack_validation():
    q = w.w4a16_quantize_pack
    assert _status(q, G128, FAKE, 4, 100, FAKE, FAKE, FAKE, 0) == w.W4A16_ERR_INVALID     # K % 128
    assert _status(q, G128, FAKE + 4, 4, 128, FAKE, FAKE, FAKE, 0) == w.W4A16_ERR_INVALID  # misaligned W
    assert _status(q, G128, None, 4, 128, FAKE, FAKE, FAKE, 0) == w.W4A16_ERR_INVALID      # null W
    assert _status(q, G128, FAKE, 4, 128, FAKE, FAKE, None, 0) == w.W4A16_ERR_INVALID      # G128 needs mins
    assert _status(q, Q4, FAKE, 4, 32, FAKE, FAKE, FAKE, 0) == w.W4A16_ERR_INVALID         # Q4 takes no mins
    assert _status(q, Q4, FAKE, 0, 32, FAKE, FAKE, None, 0) == w.W4A16_ERR_INVALID


def test_dequant_validation():
    d = w.w4a16_dequant
    assert _status(d, G128, FAKE, FAKE, FAKE, 4, 128, 7, FAKE, 0) == w.W4A16_ERR_INVALID   # dtype
    assert _status(d, G128, FAKE, FAKE, FAKE, 4, 128, BF16, FAKE + 2, 0) == w.W4A16_ERR_INVALID
    assert _status(d, Q4, FAKE, FAKE, None, 4, 40, BF16, FAKE, 0) == w.W4A16_ERR_INVALID    # K % 32


def test_gemv_validation():
    g = w.w4a16_gemv
    mx = w.w4a16_gemv_max_rows()
    assert mx >= 1
    assert _status(g, G128, BF16, FAKE, mx + 1, FAKE, FAKE, FAKE, 8, 128, FAKE, 0) == w.W4A16_ERR_UNSUPPORTED
    assert _status(g, G128, BF16, FAKE, 0, FAKE, FAKE, FAKE, 8, 128, FAKE, 0) == w.W4A16_ERR_INVALID
    assert _status(g, G128, F16, FAKE, 1, FAKE, FAKE, FAKE, 8, 128, FAKE, 0) == w.W4A16_ERR_UNSUPPORTED
    assert _status(g, Q4, F32, FAKE, 1, FAKE, FAKE, None, 8, 128, FAKE, 0) == w.W4A16_ERR_UNSUPPORTED
    assert _status(g, G128, BF16, FAKE + 8, 1, FAKE, FAKE, FAKE, 8, 128, FAKE, 0) == w.W4A16_ERR_INVALID
    assert _status(g, G128, BF16, FAKE, 1, FAKE, FAKE, FAKE, 8, 128, None, 0) == w.W4A16_ERR_INVALID
    assert _status(g, G128, 9, FAKE, 1, FAKE, FAKE, FAKE, 8, 128, FAKE, 0) == w.W4A16_ERR_INVALID


def test_gemm_validation_and_workspace():
    # a large-M shape whose tile grid is small needs a K-split workspace; too little is refused
    # on the host.  Up to 64 rows the GEMM streams the weights per row slice and needs none.
    need = w.w4a16_gemm_workspace_bytes(G128, 300, 256, 4096)
    assert need > 0 and need % (300 * 256 * 4) == 0
    assert w.w4a16_gemm_workspace_bytes(G128, 64, 256, 4096) == 0
    assert w.w4a16_gemm_workspace_bytes(Q4, 300, 256, 4096) == 0
    assert w.w4a16_gemm_workspace_bytes(G128, 0, 256, 4096) == 0
    # up to 16 rows, w4a16_matmul splits K over blocks where the 64-column blocks would leave CUs
    # idle and the codes are at least 16 MiB: 256 / 64 = 4 splits at N = 4096, fp32 partials
    assert w.w4a16_gemm_workspace_bytes(G128, 16, 4096, 14336) == 4 * 16 * 4096 * 4
    assert w.w4a16_gemm_workspace_bytes(G128, 1, 2048, 16384) == 8 * 1 * 2048 * 4
    assert w.w4a16_gemm_workspace_bytes(G128, 1, 8192, 4096) == 0       # 256 blocks of 32 columns
    assert w.w4a16_gemm_workspace_bytes(G128, 1, 4096, 4096) == 0       # 8 MiB of codes
    assert w.w4a16_gemm_workspace_bytes(G128, 16, 14336, 4096) == 0     # 224 column blocks
    # 17..64 rows: the R-row kernels' K split at small N (64-column blocks, codes >= 8 MiB)
    assert w.w4a16_gemm_workspace_bytes(G128, 17, 4096, 14336) == 4 * 17 * 4096 * 4
    assert w.w4a16_gemm_workspace_bytes(G128, 64, 4100, 8192) == 3 * 64 * 4100 * 4
    assert w.w4a16_gemm_workspace_bytes(G128, 64, 4097, 8192) == 0      # N % 4: no R-row kernel
    assert w.w4a16_gemm_workspace_bytes(G128, 48, 14336, 4096) == 0     # 224 column blocks
    assert w.w4a16_gemm_workspace_bytes(G128, 32, 11008, 4096) == 0     # 172: two splits need two waves
    assert w.w4a16_gemm_workspace_bytes(G128, 32, 8192, 4096) == 2 * 32 * 8192 * 4
    assert w.w4a16_gemm_workspace_bytes(G128, 32, 4096, 11008) == 4 * 32 * 4096 * 4  # on the 64-row kernel
    assert w.w4a16_gemm_workspace_bytes(ZP, 16, 4096, 14336) == 0
    g = w.w4a16_gemm
    assert _status(g, G128, BF16, FAKE, 300, FAKE, FAKE, FAKE, 256, 4096, FAKE, FAKE, need - 4, 0) == w.W4A16_ERR_INVALID
    assert _status(g, G128, BF16, FAKE, 300, FAKE, FAKE, FAKE, 256, 4096, FAKE, None, 0, 0) == w.W4A16_ERR_INVALID
    # the row-major formats reach the large-M path with fp16 activations only
    assert _status(g, Q4, BF16, FAKE, 64, FAKE, FAKE, None, 256, 4096, FAKE, None, 0, 0) == w.W4A16_ERR_UNSUPPORTED
    m = w.w4a16_matmul
    assert _status(m, Q4, BF16, FAKE, w.w4a16_gemv_max_rows() + 1, FAKE, FAKE, None, 64, 64, FAKE, None, 0, 0) \
        == w.W4A16_ERR_UNSUPPORTED
    assert 1 <= w.w4a16_matmul_gemv_cutoff() <= w.w4a16_gemv_max_rows()


ZP = w.W4A16_FMT_G128_ZP_FP16


def test_zero_point_format_sizes_and_validation():
    # words [N][K/8] plus an fp16 scale and an fp16 zero point per group of 128
    assert w.w4a16_packed_sizes(ZP, 14336, 4096) == (29_360_128, 917_504, 917_504)
    assert w.w4a16_packed_sizes(ZP, 1, 128) == (64, 2, 2)
    for N, K in ((5, 64), (5, 200), (0, 128)):
        with pytest.raises(w.W4A16Error):
            w.w4a16_packed_sizes(ZP, N, K)
    q = w.w4a16_quantize_pack
    assert _status(q, ZP, FAKE, 4, 128, FAKE, FAKE, None, 0) == w.W4A16_ERR_INVALID        # needs zero points
    assert _status(q, ZP, FAKE, 4, 96, FAKE, FAKE, FAKE, 0) == w.W4A16_ERR_INVALID         # K % 128
    g = w.w4a16_gemv
    assert _status(g, ZP, F32, FAKE, 1, FAKE, FAKE, FAKE, 8, 128, FAKE, 0) == w.W4A16_ERR_UNSUPPORTED
    assert _status(g, ZP, F16, FAKE, 1, FAKE, FAKE, None, 8, 128, FAKE, 0) == w.W4A16_ERR_INVALID
    assert _status(g, ZP, F16, FAKE, w.w4a16_gemv_max_rows() + 1, FAKE, FAKE, FAKE, 8, 128, FAKE, 0) \
        == w.W4A16_ERR_UNSUPPORTED
    # the large-M path: fp16 activations only, and no workspace
    assert _status(w.w4a16_gemm, ZP, BF16, FAKE, 64, FAKE, FAKE, FAKE, 256, 4096, FAKE, None, 0, 0) \
        == w.W4A16_ERR_UNSUPPORTED
    assert _status(w.w4a16_gemm, ZP, F16, FAKE, 64, FAKE, FAKE, None, 256, 4096, FAKE, None, 0, 0) \
        == w.W4A16_ERR_INVALID
    assert w.w4a16_gemm_workspace_bytes(ZP, 300, 256, 4096) == 0


W8 = w.W4A16_FMT_W8_ROW_FP32


def test_w8_format_sizes_and_validation():
    # one byte per weight and an fp32 scale per row
    assert w.w4a16_packed_sizes(W8, 14336, 4096) == (58_720_256, 57_344, 0)
    assert w.w4a16_packed_sizes(W8, 3, 16) == (48, 12, 0)
    for N, K in ((5, 8), (5, 40), (0, 16)):
        with pytest.raises(w.W4A16Error):
            w.w4a16_packed_sizes(W8, N, K)
    q = w.w4a16_quantize_pack
    assert _status(q, W8, FAKE, 4, 32, FAKE, FAKE, FAKE, 0) == w.W4A16_ERR_INVALID         # takes no mins
    g = w.w4a16_gemv
    assert _status(g, W8, BF16, FAKE, 1, FAKE, FAKE, None, 8, 128, FAKE, 0) == w.W4A16_ERR_UNSUPPORTED
    assert _status(g, W8, F32, FAKE, 1, FAKE, FAKE, None, 8, 128, FAKE, 0) == w.W4A16_ERR_UNSUPPORTED
    assert _status(w.w4a16_gemm, W8, BF16, FAKE, 64, FAKE, FAKE, None, 256, 4096, FAKE, None, 0, 0) \
        == w.W4A16_ERR_UNSUPPORTED
    assert _status(w.w4a16_gemm, W8, F16, FAKE, 64, FAKE, FAKE, FAKE, 256, 4096, FAKE, None, 0, 0) \
        == w.W4A16_ERR_INVALID                                                             # takes no mins


def test_w4a8_validation():
    qa = w.w4a16_quantize_act_i8
    assert _status(qa, FAKE, 0, 128, FAKE, FAKE, FAKE, 0) == w.W4A16_ERR_INVALID            # M = 0
    assert _status(qa, FAKE, 4, 100, FAKE, FAKE, FAKE, 0) == w.W4A16_ERR_INVALID            # K % 128
    assert _status(qa, FAKE + 8, 4, 128, FAKE, FAKE, FAKE, 0) == w.W4A16_ERR_INVALID        # misaligned x
    assert _status(qa, FAKE, 4, 128, FAKE, None, FAKE, 0) == w.W4A16_ERR_INVALID            # null ascale
    assert _status(qa, FAKE, 1 << 20, 1 << 12, FAKE, FAKE, FAKE, 0) == w.W4A16_ERR_INVALID  # M*K >= 2^31
    g = w.w4a16_gemm_w4a8
    assert _status(g, Q4, FAKE, FAKE, FAKE, 64, FAKE, FAKE, None, 256, 1024, FAKE, 0) \
        == w.W4A16_ERR_UNSUPPORTED                                                           # G128 only
    assert _status(g, G128, FAKE, FAKE, FAKE, 64, FAKE, FAKE, FAKE, 258, 1024, FAKE, 0) \
        == w.W4A16_ERR_UNSUPPORTED                                                           # N % 4
    assert _status(g, G128, FAKE, FAKE, FAKE, 64, FAKE, FAKE, None, 256, 1024, FAKE, 0) \
        == w.W4A16_ERR_INVALID                                                               # no mins
    assert _status(g, G128, FAKE, FAKE, FAKE + 4, 64, FAKE, FAKE, FAKE, 256, 1024, FAKE, 0) \
        == w.W4A16_ERR_INVALID                                                               # misaligned xsum
    assert _status(g, G128, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, 256, 1024, FAKE, 0) == w.W4A16_ERR_INVALID
    assert _status(g, G128, FAKE, FAKE, FAKE, 64, FAKE, FAKE, FAKE, 256, 1000, FAKE, 0) == w.W4A16_ERR_INVALID


def test_check_weights_rejects_what_the_formats_cannot_store():
    """The debug weight check (host memory, no GPU): every weight finite, and each group's stored
    parameter representable -- the Q4 fp16 scale max|w|/7 and the zero-point format's fp16 scale
    (max - min)/15 below 65520 (the rounding midpoint past fp16's largest value, 65504), the G128
    bf16 scale and minimum below bf16's overflow midpoint."""
    import numpy as np
    ZP, W8 = w.W4A16_FMT_G128_ZP_FP16, w.W4A16_FMT_W8_ROW_FP32
    ok = (np.random.default_rng(0).standard_normal((4, 256)) * 0.02).astype(np.float32)
    for fmt in (G128, Q4, ZP, W8):
        w.w4a16_check_weights(fmt, ok, 4, 256)
    for fmt in (G128, Q4, ZP, W8):
        bad = ok.copy()
        bad[2, 200] = np.nan
        assert _status(w.w4a16_check_weights, fmt, bad, 4, 256) == w.W4A16_ERR_INVALID
        bad[2, 200] = np.inf
        assert _status(w.w4a16_check_weights, fmt, bad, 4, 256) == w.W4A16_ERR_INVALID
    # Q4: max|w| / 7 just below and at the fp16 overflow midpoint, in the last block of a row
    edge = np.float32(65520.0 * 7)
    q4 = ok.copy()
    q4[3, 255] = np.nextafter(edge, np.float32(0))
    assert np.float32(q4[3, 255]) / np.float32(7) < 65520
    w.w4a16_check_weights(Q4, q4, 4, 256)
    q4[3, 255] = -edge
    assert _status(w.w4a16_check_weights, Q4, q4, 4, 256) == w.W4A16_ERR_INVALID
    w.w4a16_check_weights(G128, q4, 4, 256)          # bf16 holds that scale; W8's fp32 too
    w.w4a16_check_weights(W8, q4, 4, 256)
    # zero-point format: the range sets the scale (a group from -a to +a has scale 2a / 15)
    zp = ok.copy()
    zp[1, 0], zp[1, 1] = -4.0e5, 4.0e5             # 8e5 / 15 = 53333: fits
    w.w4a16_check_weights(ZP, zp, 4, 256)
    zp[1, 1] = 6.0e5                                # 1e6 / 15 = 66667: overflows fp16
    assert _status(w.w4a16_check_weights, ZP, zp, 4, 256) == w.W4A16_ERR_INVALID
    assert _status(w.w4a16_check_weights, Q4, zp, 4, 256) == w.W4A16_ERR_INVALID   # 6e5 / 7
    w.w4a16_check_weights(G128, zp, 4, 256)
    # G128: a range that overflows fp32 (and so the bf16 scale), and a minimum past bf16's range
    g = ok.copy()
    g[0, 5], g[0, 6] = -3.0e38, 3.0e38
    assert _status(w.w4a16_check_weights, G128, g, 4, 256) == w.W4A16_ERR_INVALID
    g = ok.copy()
    g[0, :128] = np.float32(-3.4e38)                # a constant group: scale 0 (fine), min overflows bf16
    assert _status(w.w4a16_check_weights, G128, g, 4, 256) == w.W4A16_ERR_INVALID
    g[0, :128] = np.float32(-3.38e38)              # rounds to bf16's largest finite value
    w.w4a16_check_weights(G128, g, 4, 256)
    # shape errors as w4a16_packed_sizes
    assert _status(w.w4a16_check_weights, G128, ok, 4, 100) == w.W4A16_ERR_INVALID
    assert _status(w.w4a16_check_weights, G128, None, 4, 256) == w.W4A16_ERR_INVALID


def test_matmul_noalloc_validation():
    """The no-allocation entry point checks like w4a16_matmul, and refuses on the host a shape
    whose split-K partials exceed its scratch array (no device is touched by any of these)."""
    f = w.w4a16_matmul_noalloc
    assert w.w4a16_matmul_noalloc_max_scratch_bytes() == 16 << 20
    assert _status(f, G128, BF16, FAKE, 0, FAKE, FAKE, FAKE, 256, 128, FAKE, 0) == w.W4A16_ERR_INVALID
    assert _status(f, G128, BF16, FAKE + 2, 1, FAKE, FAKE, FAKE, 256, 128, FAKE, 0) == w.W4A16_ERR_INVALID
    assert _status(f, G128, BF16, FAKE, 1, FAKE, FAKE, None, 256, 128, FAKE, 0) == w.W4A16_ERR_INVALID
    assert _status(f, G128, F16, FAKE, 1, FAKE, FAKE, FAKE, 256, 128, FAKE, 0) == w.W4A16_ERR_UNSUPPORTED
    assert w.w4a16_gemm_workspace_bytes(G128, 2048, 520, 1024) > 16 << 20
    assert _status(f, G128, BF16, FAKE, 2048, FAKE, FAKE, FAKE, 520, 1024, FAKE, 0) == w.W4A16_ERR_UNSUPPORTED


def test_prepared_copy_sizes_and_validation():
    """The zero-point format's prepared copy: words [K/8][N] plus fp32 s and m [K/128][N], each part
    16-byte aligned; no other format has one.  Every call below fails on the host."""
    assert w.w4a16_prepared_bytes(ZP, 14336, 4096) == 29_360_128 + 2 * 1_835_008
    assert w.w4a16_prepared_bytes(ZP, 3, 128) == 192 + 16 + 16     # 12-byte fp32 parts padded to 16
    assert w.w4a16_prepared_bytes(ZP, 3, 100) == 0                  # no such shape
    for fmt in (G128, Q4, W8):
        assert w.w4a16_prepared_bytes(fmt, 256, 4096) == 0
    need = w.w4a16_prepared_bytes(ZP, 256, 4096)
    p = w.w4a16_prepare
    assert _status(p, ZP, FAKE, FAKE, FAKE, 256, 4096, FAKE, need - 1, 0) == w.W4A16_ERR_INVALID   # too small
    assert _status(p, ZP, FAKE, FAKE, FAKE, 256, 4096, FAKE + 8, need, 0) == w.W4A16_ERR_INVALID   # alignment
    assert _status(p, ZP, FAKE, FAKE, None, 256, 4096, FAKE, need, 0) == w.W4A16_ERR_INVALID       # zero points
    assert _status(p, ZP, FAKE, FAKE, FAKE, 256, 100, FAKE, need, 0) == w.W4A16_ERR_INVALID        # K % 128
    assert _status(p, G128, FAKE, FAKE, FAKE, 256, 4096, FAKE, need, 0) == w.W4A16_ERR_UNSUPPORTED
    g = w.w4a16_gemv_prepared
    assert _status(g, ZP, F16, FAKE, 0, FAKE, 256, 4096, FAKE, 0) == w.W4A16_ERR_INVALID           # M = 0
    assert _status(g, ZP, F16, FAKE + 4, 1, FAKE, 256, 4096, FAKE, 0) == w.W4A16_ERR_INVALID       # alignment
    assert _status(g, ZP, F16, FAKE, 1, None, 256, 4096, FAKE, 0) == w.W4A16_ERR_INVALID           # no copy
    assert _status(g, ZP, 7, FAKE, 1, FAKE, 256, 4096, FAKE, 0) == w.W4A16_ERR_INVALID             # no such type
    assert _status(g, ZP, F32, FAKE, 1, FAKE, 256, 4096, FAKE, 0) == w.W4A16_ERR_UNSUPPORTED
    assert _status(g, Q4, F16, FAKE, 1, FAKE, 256, 4096, FAKE, 0) == w.W4A16_ERR_UNSUPPORTED
