"""CPU oracle for the W4A16 format and matmul -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The product (``gemm_w4a16_amd``) never imports it, and it imports nothing from
the product: the two share no code.

The arithmetic lives in ``w4a16_oracle.c`` (plain C, fp64 sums, compiled with gcc, no fast-math,
no FMA contraction); this module only marshals numpy arrays into it.  Each function names the
passage of the pages it follows:

* ``quantize_g128`` / ``dequant_g128`` / ``matmul_g128`` -- vidyal.ai "Low-Precision Kernels",
  section "Step 2: a W4A16 kernel in Triton" (group 128, scale (max-min)/15, code
  round((w-min)/scale), eight codes per int32 along K, K/8 x N packed, K/128 x N bf16 scale and
  minimum, dequant q*s+min, FP64 reference with the same 4-bit weights).
* ``quantize_g128zp`` / ``dequant_g128zp`` / ``matmul_g128zp`` -- anrans.github.io "Quantization
  and GEMV", sections "The quantization formulas" (s = (max-min)/15, z = round(-min/s),
  q = clamp(round(w/s) + z, 0, 15), w_hat = (q - z) s) and "W4A16: dequantizing in registers"
  (eight codes per word along K, first in the low bits; words [N][K/8]; a scale and a zero point
  per group of 128, the zero point kept as fp16).
* ``quantize_w8row`` / ``dequant_w8row`` / ``matmul_w8row`` -- the same page, "Exercises", 1:
  symmetric per-channel int8, s = max|w|/127 per row, q = clamp(round(w/s), -127, 127), int8
  [N][K], the row scale applied after the row's sum.
* ``quantize_q4b32`` / ``dequant_q4b32`` / ``matmul_q4b32`` -- thuongvuho.com "Why My 4-Bit
  CUDA Kernel Wasn't Faster", sections "Why fewer bytes should have helped" and "Loading the
  same bytes differently" (blocks of 32: 16 code bytes + fp16 scale, decode (code-bias)*scale,
  low nibble of byte j pairs with x[2j]).

Every function here is pinned by ``tests/test_oracle_pins.py`` against facts fixed by the
pages and by mathematics (closed forms, brute force, special cases, library conversions).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "w4a16_oracle.c"
_LIB_PATH = _HERE / "liboracle.so"

# Readings of the pages that the C file implements, kept here for the tests to report.
ORACLE_OK, ORACLE_BAD_ARG, ORACLE_NONFINITE = 0, 1, 2


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc: IEEE arithmetic, no fast-math, no FMA contraction."""
    if force or not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB_PATH.with_suffix(f".so.tmp{os.getpid()}")
        compile_to(_SRC, tmp)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def compile_to(src: Path, out: Path) -> Path:
    """Compile an oracle C source to a shared library with the oracle's flags (the tests use
    this to build deliberately broken copies and check that the pins catch them)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-frounding-math", "-o", str(out), str(src), "-lm"]
    subprocess.run(cmd, check=True)
    return out


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build(force=False)
        _lib = bind(_LIB_PATH)
    return _lib


def bind(path) -> ctypes.CDLL:
    """Load an oracle library and declare its signatures."""
    L = ctypes.CDLL(str(path))
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.oracle_f32_to_bf16.argtypes, L.oracle_f32_to_bf16.restype = [ctypes.c_float], ctypes.c_uint16
    L.oracle_bf16_to_f32.argtypes, L.oracle_bf16_to_f32.restype = [ctypes.c_uint16], ctypes.c_float
    L.oracle_f32_to_f16.argtypes, L.oracle_f32_to_f16.restype = [ctypes.c_float], ctypes.c_uint16
    L.oracle_f16_to_f64.argtypes, L.oracle_f16_to_f64.restype = [ctypes.c_uint16], ctypes.c_double
    L.oracle_pack_word.argtypes, L.oracle_pack_word.restype = [P], ctypes.c_uint32
    L.oracle_unpack_word.argtypes, L.oracle_unpack_word.restype = [ctypes.c_uint32, P], None
    L.oracle_quantize_g128.argtypes = [P, I64, I64, P, P, P]
    L.oracle_dequant_g128.argtypes = [P, P, P, I64, I64, I, P]
    L.oracle_quantize_q4b32.argtypes = [P, I64, I64, P, P]
    L.oracle_dequant_q4b32.argtypes = [P, P, I64, I64, I, P]
    L.oracle_matmul_g128_f64.argtypes = [P, I, I64, P, P, P, I64, I64, P]
    L.oracle_matmul_g128_f64_at.argtypes = [P, I, I64, P, P, P, I64, I64, P, P, I64, P]
    L.oracle_matmul_q4b32_f64.argtypes = [P, I, I64, P, P, I64, I64, P]
    L.oracle_matmul_q4b32_f64_at.argtypes = [P, I, I64, P, P, I64, I64, P, P, I64, P]
    L.oracle_matmul_f32w_f64.argtypes = [P, I, I64, P, I64, I64, P]
    L.oracle_quantize_g128zp.argtypes = [P, I64, I64, P, P, P]
    L.oracle_dequant_g128zp.argtypes = [P, P, P, I64, I64, I, P]
    L.oracle_matmul_g128zp_f64.argtypes = [P, I, I64, P, P, P, I64, I64, P]
    L.oracle_matmul_g128zp_f64_at.argtypes = [P, I, I64, P, P, P, I64, I64, P, P, I64, P]
    L.oracle_quantize_w8row.argtypes = [P, I64, I64, P, P]
    L.oracle_dequant_w8row.argtypes = [P, P, I64, I64, I, P]
    L.oracle_matmul_w8row_f64.argtypes = [P, I, I64, P, P, I64, I64, P]
    L.oracle_quantize_pack.argtypes = [I, P, I64, I64, P, P, P]
    L.oracle_dequant.argtypes = [I, P, P, P, I64, I64, I, P]
    L.oracle_matmul_f64.argtypes = [I, P, I, I64, P, P, P, I64, I64, P]
    L.oracle_quantize_act_i8.argtypes = [P, I64, I64, P, P, P]
    L.oracle_matmul_w4a8_f64.argtypes = [P, P, I64, P, P, P, I64, I64, P]
    L.oracle_matmul_w4a8_f64_at.argtypes = [P, P, I64, P, P, P, I64, I64, P, P, I64, P]
    for name in ("oracle_quantize_pack", "oracle_dequant", "oracle_matmul_f64", "oracle_quantize_act_i8", "oracle_matmul_w4a8_f64", "oracle_matmul_w4a8_f64_at",
                 "oracle_quantize_w8row", "oracle_dequant_w8row", "oracle_matmul_w8row_f64",
                 "oracle_quantize_g128zp", "oracle_dequant_g128zp", "oracle_matmul_g128zp_f64",
                 "oracle_matmul_g128zp_f64_at",
                 "oracle_quantize_g128", "oracle_dequant_g128", "oracle_quantize_q4b32",
                 "oracle_dequant_q4b32", "oracle_matmul_g128_f64", "oracle_matmul_g128_f64_at",
                 "oracle_matmul_q4b32_f64", "oracle_matmul_q4b32_f64_at", "oracle_matmul_f32w_f64"):
        getattr(L, name).restype = I
    return L


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != ORACLE_OK:
        raise ValueError(f"oracle {what} failed with code {rc} "
                         f"({'bad argument' if rc == ORACLE_BAD_ARG else 'non-finite input'})")


# ---- scalar conversions ------------------------------------------------------------------

def f32_to_bf16(v: float) -> int:
    return int(lib().oracle_f32_to_bf16(float(v)))


def bf16_to_f32(b: int) -> float:
    return float(lib().oracle_bf16_to_f32(int(b)))


def f32_to_f16(v: float) -> int:
    return int(lib().oracle_f32_to_f16(float(v)))


def f16_to_f64(h: int) -> float:
    return float(lib().oracle_f16_to_f64(int(h)))


def pack_word(q) -> int:
    a = np.ascontiguousarray(np.asarray(q, dtype=np.uint8))
    assert a.shape == (8,)
    return int(lib().oracle_pack_word(_ptr(a)))


def unpack_word(w: int) -> np.ndarray:
    out = np.zeros(8, dtype=np.uint8)
    lib().oracle_unpack_word(ctypes.c_uint32(int(w) & 0xFFFFFFFF), _ptr(out))
    return out


# ---- format G128: asymmetric, group 128, bf16 scale + minimum ----------------------------

def quantize_g128(W: np.ndarray):
    """W fp32 [N][K] -> (codes uint32 [K/8][N], scales bf16-bits uint16 [K/128][N], mins same)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    codes = np.zeros((K // 8, N), dtype=np.uint32)
    scales = np.zeros((K // 128, N), dtype=np.uint16)
    mins = np.zeros((K // 128, N), dtype=np.uint16)
    _check(lib().oracle_quantize_g128(_ptr(W), N, K, _ptr(codes), _ptr(scales), _ptr(mins)),
           "quantize_g128")
    return codes, scales, mins


def dequant_g128(codes, scales, mins, kind: str = "f32") -> np.ndarray:
    """kind 'f32': fmaf(q, s, m); 'bf16': bf16 bits of that (uint16); 'f64': exact q*s+m."""
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    mins = np.ascontiguousarray(mins, dtype=np.uint16)
    K8, N = codes.shape
    K = K8 * 8
    k_id, dt = {"f32": (0, np.float32), "bf16": (1, np.uint16), "f64": (2, np.float64)}[kind]
    out = np.zeros((N, K), dtype=dt)
    _check(lib().oracle_dequant_g128(_ptr(codes), _ptr(scales), _ptr(mins), N, K, k_id, _ptr(out)),
           "dequant_g128")
    return out


def matmul_g128(x_bits: np.ndarray, codes, scales, mins, x_kind: str = "bf16") -> np.ndarray:
    """x_bits uint16 [M][K] (bf16 or fp16 bits) -> y float64 [M][N] with exact dequant weights."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    mins = np.ascontiguousarray(mins, dtype=np.uint16)
    M, K = x_bits.shape
    N = codes.shape[1]
    y = np.zeros((M, N), dtype=np.float64)
    _check(lib().oracle_matmul_g128_f64(_ptr(x_bits), 0 if x_kind == "bf16" else 1, M, _ptr(codes),
                                        _ptr(scales), _ptr(mins), N, K, _ptr(y)), "matmul_g128")
    return y


def matmul_g128_at(x_bits, codes, scales, mins, rows, cols, x_kind: str = "bf16") -> np.ndarray:
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    mins = np.ascontiguousarray(mins, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    M, K = x_bits.shape
    N = codes.shape[1]
    y = np.zeros(len(rows), dtype=np.float64)
    _check(lib().oracle_matmul_g128_f64_at(_ptr(x_bits), 0 if x_kind == "bf16" else 1, M,
                                           _ptr(codes), _ptr(scales), _ptr(mins), N, K, _ptr(rows),
                                           _ptr(cols), len(rows), _ptr(y)), "matmul_g128_at")
    return y


# ---- W4A8: per-row int8 activations with the G128 weights ----------------------------------

def quantize_act_i8(x_bits: np.ndarray):
    """x_bits uint16 [M][K] bf16 -> (xq int8 [M][K], ascale float32 [M], xsum float32 [K/128][M]).

    Per row a = max|x| / 127 (1.0 for a zero row), xq = clamp(rint(x / a), -127, 127); xsum holds
    each group's exact integer sum of xq (vidyal.ai "Low-Precision Kernels", "The cost of
    quantizing activations")."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    xq = np.zeros((M, K), dtype=np.int8)
    ascale = np.zeros(M, dtype=np.float32)
    xsum = np.zeros((K // 128, M), dtype=np.float32)
    _check(lib().oracle_quantize_act_i8(_ptr(x_bits), M, K, _ptr(xq), _ptr(ascale), _ptr(xsum)), "quantize_act_i8")
    return xq, ascale, xsum


def matmul_w4a8(xq, ascale, codes, scales, mins) -> np.ndarray:
    """y float64 [M][N] = (a_m * xq) . (q * s + min)^T in fp64, G128 weights."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    ascale = np.ascontiguousarray(ascale, dtype=np.float32)
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    mins = np.ascontiguousarray(mins, dtype=np.uint16)
    M, K = xq.shape
    N = codes.shape[1]
    y = np.zeros((M, N), dtype=np.float64)
    _check(lib().oracle_matmul_w4a8_f64(_ptr(xq), _ptr(ascale), M, _ptr(codes), _ptr(scales), _ptr(mins), N, K,
                                        _ptr(y)), "matmul_w4a8")
    return y


def matmul_w4a8_at(xq, ascale, codes, scales, mins, rows, cols) -> np.ndarray:
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    ascale = np.ascontiguousarray(ascale, dtype=np.float32)
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    mins = np.ascontiguousarray(mins, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    M, K = xq.shape
    N = codes.shape[1]
    y = np.zeros(len(rows), dtype=np.float64)
    _check(lib().oracle_matmul_w4a8_f64_at(_ptr(xq), _ptr(ascale), M, _ptr(codes), _ptr(scales), _ptr(mins), N, K,
                                           _ptr(rows), _ptr(cols), len(rows), _ptr(y)), "matmul_w4a8_at")
    return y


# ---- format G128-ZP: asymmetric, group 128, fp16 scale + fp16 integer zero point ------------

def quantize_g128zp(W: np.ndarray):
    """W fp32 [N][K] -> (codes uint32 [N][K/8], scales fp16-bits uint16 [N][K/128], zeros same)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    codes = np.zeros((N, K // 8), dtype=np.uint32)
    scales = np.zeros((N, K // 128), dtype=np.uint16)
    zeros = np.zeros((N, K // 128), dtype=np.uint16)
    _check(lib().oracle_quantize_g128zp(_ptr(W), N, K, _ptr(codes), _ptr(scales), _ptr(zeros)),
           "quantize_g128zp")
    return codes, scales, zeros


def dequant_g128zp(codes, scales, zeros, kind: str = "f32") -> np.ndarray:
    """kind 'f32' (exact (q - z) s), 'bf16' bits, 'f64', 'f16' bits."""
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint16)
    N, K8 = codes.shape
    K = K8 * 8
    k_id, dt = {"f32": (0, np.float32), "bf16": (1, np.uint16), "f64": (2, np.float64),
                "f16": (3, np.uint16)}[kind]
    out = np.zeros((N, K), dtype=dt)
    _check(lib().oracle_dequant_g128zp(_ptr(codes), _ptr(scales), _ptr(zeros), N, K, k_id, _ptr(out)),
           "dequant_g128zp")
    return out


def matmul_g128zp(x_bits: np.ndarray, codes, scales, zeros, x_kind: str = "f16") -> np.ndarray:
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint16)
    M, K = x_bits.shape
    N = codes.shape[0]
    y = np.zeros((M, N), dtype=np.float64)
    _check(lib().oracle_matmul_g128zp_f64(_ptr(x_bits), 0 if x_kind == "bf16" else 1, M, _ptr(codes),
                                          _ptr(scales), _ptr(zeros), N, K, _ptr(y)), "matmul_g128zp")
    return y


def matmul_g128zp_at(x_bits, codes, scales, zeros, rows, cols, x_kind: str = "f16") -> np.ndarray:
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    M, K = x_bits.shape
    N = codes.shape[0]
    y = np.zeros(len(rows), dtype=np.float64)
    _check(lib().oracle_matmul_g128zp_f64_at(_ptr(x_bits), 0 if x_kind == "bf16" else 1, M,
                                             _ptr(codes), _ptr(scales), _ptr(zeros), N, K, _ptr(rows),
                                             _ptr(cols), len(rows), _ptr(y)), "matmul_g128zp_at")
    return y


# ---- format W8: symmetric per-row int8, fp32 row scale -----------------------------------

def quantize_w8row(W: np.ndarray):
    """W fp32 [N][K] -> (codes int8 [N][K], scales fp32 [N])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    codes = np.zeros((N, K), dtype=np.int8)
    scales = np.zeros(N, dtype=np.float32)
    _check(lib().oracle_quantize_w8row(_ptr(W), N, K, _ptr(codes), _ptr(scales)), "quantize_w8row")
    return codes, scales


def dequant_w8row(codes, scales, kind: str = "f32") -> np.ndarray:
    """kind 'f32' (q*s rounded once), 'bf16' / 'f16' bits of that fp32 value, 'f64' (exact)."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    N, K = codes.shape
    k_id, dt = {"f32": (0, np.float32), "bf16": (1, np.uint16), "f64": (2, np.float64),
                "f16": (3, np.uint16)}[kind]
    out = np.zeros((N, K), dtype=dt)
    _check(lib().oracle_dequant_w8row(_ptr(codes), _ptr(scales), N, K, k_id, _ptr(out)), "dequant_w8row")
    return out


def matmul_w8row(x_bits: np.ndarray, codes, scales, x_kind: str = "f16") -> np.ndarray:
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    M, K = x_bits.shape
    N = codes.shape[0]
    y = np.zeros((M, N), dtype=np.float64)
    _check(lib().oracle_matmul_w8row_f64(_ptr(x_bits), 0 if x_kind == "bf16" else 1, M, _ptr(codes),
                                         _ptr(scales), N, K, _ptr(y)), "matmul_w8row")
    return y


# ---- format Q4B32: symmetric blocks of 32, fp16 scale, bias 8 -----------------------------

def quantize_q4b32(W: np.ndarray):
    """W fp32 [N][K] -> (codes uint8 [N][K/32][16], scales fp16-bits uint16 [N][K/32])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    codes = np.zeros((N, K // 32, 16), dtype=np.uint8)
    scales = np.zeros((N, K // 32), dtype=np.uint16)
    _check(lib().oracle_quantize_q4b32(_ptr(W), N, K, _ptr(codes), _ptr(scales)), "quantize_q4b32")
    return codes, scales


def dequant_q4b32(codes, scales, kind: str = "f32") -> np.ndarray:
    """kind 'f32' (exact), 'bf16' bits, 'f64', 'f16' bits."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    N, B = scales.shape
    K = B * 32
    k_id, dt = {"f32": (0, np.float32), "bf16": (1, np.uint16), "f64": (2, np.float64),
                "f16": (3, np.uint16)}[kind]
    out = np.zeros((N, K), dtype=dt)
    _check(lib().oracle_dequant_q4b32(_ptr(codes), _ptr(scales), N, K, k_id, _ptr(out)),
           "dequant_q4b32")
    return out


def matmul_q4b32(x_bits: np.ndarray, codes, scales, x_kind: str = "f16") -> np.ndarray:
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    M, K = x_bits.shape
    N = scales.shape[0]
    y = np.zeros((M, N), dtype=np.float64)
    _check(lib().oracle_matmul_q4b32_f64(_ptr(x_bits), 0 if x_kind == "bf16" else 1, M, _ptr(codes),
                                         _ptr(scales), N, K, _ptr(y)), "matmul_q4b32")
    return y


def matmul_q4b32_at(x_bits, codes, scales, rows, cols, x_kind: str = "f16") -> np.ndarray:
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    M, K = x_bits.shape
    N = scales.shape[0]
    y = np.zeros(len(rows), dtype=np.float64)
    _check(lib().oracle_matmul_q4b32_f64_at(_ptr(x_bits), 0 if x_kind == "bf16" else 1, M,
                                            _ptr(codes), _ptr(scales), N, K, _ptr(rows), _ptr(cols),
                                            len(rows), _ptr(y)), "matmul_q4b32_at")
    return y


def matmul_original(x_bits: np.ndarray, W: np.ndarray, x_kind: str = "bf16") -> np.ndarray:
    """fp64 product with the original fp32 weights: the format's quantization-error reference."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    W = np.ascontiguousarray(W, dtype=np.float32)
    M, K = x_bits.shape
    N = W.shape[0]
    y = np.zeros((M, N), dtype=np.float64)
    _check(lib().oracle_matmul_f32w_f64(_ptr(x_bits), 0 if x_kind == "bf16" else 1, M, _ptr(W), N, K,
                                        _ptr(y)), "matmul_original")
    return y
