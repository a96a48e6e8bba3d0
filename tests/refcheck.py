"""Reference products and the element-wise bound every matmul output is checked against.

Test infrastructure (CPU, numpy).  The reference for every output is the oracle's fp64 product:
the weights come from the oracle's exact fp64 dequant and the product is numpy's fp64 matmul,
which tests/test_oracle_pins.py pins equal to the oracle's own k-ordered sums (vidyal.ai
"Low-Precision Kernels", Step 2: the FP64 product with the same 4-bit weights).  A library
matmul may serve as that step; it lets the tests compare all 14.7 M outputs of the prefill shape.

Each output is held to two bars:

* the relative L2 error over all outputs, <= 5e-3 (the bar for the whole product);
* an element-wise bound, in the manner of the page's check_close (anrans.github.io "Quantization
  and GEMV", "W4A16: dequantizing in registers", which compares every element with a relative
  and an absolute tolerance), but derived from the arithmetic of the paths under test:

      |y - y_ref| <= u_out |y_ref| + 2^-5 R + 2^-20 B,

  - u_out |y_ref|: the output's rounding to the activation type (u_out = 2^-8 for bf16, 2^-11
    for fp16; the accumulator's own error is carried by the other two terms);
  - 2^-5 R, with R = sqrt(sum_k x_k^2 w_k^2): the large-M path rounds each dequantized weight to
    bf16, an error of at most 2^-8 |w_k| per term.  Taking the roundings as independent, Hoeffding's
    inequality puts the sum of the K errors past 8 * 2^-8 R = 2^-5 R with probability below
    2 exp(-32) ~ 3e-14 per output;
  - 2^-20 B: the factored and offset forms (s * sum(x (128 + q)) + (min - 128 s) * sum(x), and the
    1024 + q fp16 offsets of the row-major GEMVs) sum terms far larger than the weights and cancel
    them in fp32.  B sums, per group, the largest magnitude those fp32 terms reach per unit of
    sum|x|, times sum|x| over the group; 2^-20 allows sixteen fp32 roundings (2^-24 each) on them.

An output the kernel never writes (the tests fill y with NaN first), a wrong tile or a dropped
group breaks the element-wise bound even where the L2 norm over millions of outputs would not
notice it.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads

TOL = 5e-3
U_OUT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
C_ROUND = 2.0 ** -5     # Hoeffding allowance for bf16-rounded weights (8 half-ulps of R)
C_CANCEL = 2.0 ** -20   # sixteen fp32 roundings of the factored / offset terms


def _x64(x_bits, x_kind):
    return workloads.bits_to_f32(x_bits, x_kind).astype(np.float64)


def _group_abs_sums(x, size):
    M, K = x.shape
    return np.abs(x).reshape(M, K // size, size).sum(axis=2)      # [M][K/size]


CHUNK = 2048  # output columns dequantized at a time (the fp64 weights of 16384^2 are 2 GiB)


def _ref_and_r(x, N, dequant_cols):
    """y_ref = x . W_hat^T and R over column chunks; dequant_cols(n0, n1) gives fp64 W_hat rows
    n0..n1-1 ([n1 - n0][K]) from the oracle."""
    M = x.shape[0]
    y, R = np.empty((M, N)), np.empty((M, N))
    x2 = x * x
    for n0 in range(0, N, CHUNK):
        n1 = min(N, n0 + CHUNK)
        Wc = dequant_cols(n0, n1)
        y[:, n0:n1] = x @ Wc.T
        R[:, n0:n1] = np.sqrt(x2 @ (Wc * Wc).T)
    return y, R


def g128(x_bits, codes, scales, mins, x_kind="bf16"):
    """(y_ref, R, B) for the G128 format.  B per group: s (128 + 15) + |min - 128 s| <= 271 s + |min|
    (the factored form's two fp32 sums), times sum|x| over the group."""
    x = _x64(x_bits, x_kind)
    N = codes.shape[1]
    y, R = _ref_and_r(x, N, lambda a, b: oracle.dequant_g128(np.ascontiguousarray(codes[:, a:b]),
                                                             np.ascontiguousarray(scales[:, a:b]),
                                                             np.ascontiguousarray(mins[:, a:b]), "f64"))
    s = workloads.bits_to_f32(scales, "bf16").astype(np.float64)         # [G][N]
    m = workloads.bits_to_f32(mins, "bf16").astype(np.float64)
    B = _group_abs_sums(x, 128) @ (271.0 * s + np.abs(m))
    return y, R, B


def q4b32(x_bits, codes, scales, x_kind="f16"):
    """Q4: per block the offset sums reach (1024 + 15) + (1024 + 240) + 1032 + 1152 < 4500 per unit
    of x, times the block scale."""
    x = _x64(x_bits, x_kind)
    N = scales.shape[0]
    y, R = _ref_and_r(x, N, lambda a, b: oracle.dequant_q4b32(codes[a:b], scales[a:b], "f64"))
    s = scales.view(np.float16).astype(np.float64)                       # [N][K/32]
    B = _group_abs_sums(x, 32) @ (4500.0 * s).T
    return y, R, B


def g128zp(x_bits, codes, scales, zeros, x_kind="f16"):
    """Zero-point format: the Q4 offsets plus z sum(x): s (4500 + |z|) per unit of x."""
    x = _x64(x_bits, x_kind)
    N = codes.shape[0]
    y, R = _ref_and_r(x, N, lambda a, b: oracle.dequant_g128zp(codes[a:b], scales[a:b], zeros[a:b], "f64"))
    s = scales.view(np.float16).astype(np.float64)                       # [N][K/128]
    z = zeros.view(np.float16).astype(np.float64)
    B = _group_abs_sums(x, 128) @ (s * (4500.0 + np.abs(z))).T
    return y, R, B


def w8row(x_bits, codes, scales, x_kind="f16"):
    """W8: 1024 + (q + 128) <= 1279 against a 1152 offset per 16-byte block: 2431 s per unit of x."""
    x = _x64(x_bits, x_kind)
    N = codes.shape[0]
    y, R = _ref_and_r(x, N, lambda a, b: oracle.dequant_w8row(codes[a:b], scales[a:b], "f64"))
    B = np.abs(x).sum(axis=1, keepdims=True) * (2431.0 * scales.astype(np.float64))[None, :]
    return y, R, B


def w4a8(xq, ascale, codes, scales, mins):
    """W4A8 with G128 weights: the activations are a_m * xq (exact in fp64); the integer sums are
    exact and the per-group epilogue s * sum(xq q) + min * X_g runs in fp32, whose terms reach
    (15 s + |min|) per unit of |a xq|."""
    x = ascale.astype(np.float64)[:, None] * xq.astype(np.float64)
    N = codes.shape[1]
    y, R = _ref_and_r(x, N, lambda a, b: oracle.dequant_g128(np.ascontiguousarray(codes[:, a:b]),
                                                             np.ascontiguousarray(scales[:, a:b]),
                                                             np.ascontiguousarray(mins[:, a:b]), "f64"))
    s = workloads.bits_to_f32(scales, "bf16").astype(np.float64)
    m = workloads.bits_to_f32(mins, "bf16").astype(np.float64)
    B = _group_abs_sums(x, 128) @ (15.0 * s + np.abs(m))
    return y, R, B


def bound(y_ref, R, B, out_kind):
    return U_OUT[out_kind] * np.abs(y_ref) + C_ROUND * R + C_CANCEL * B


def check(y, ref, out_kind, what=""):
    """Assert both bars on a product y (fp32 or fp64 values of the 16-bit output) against
    ref = (y_ref, R, B); return (relative L2 error, worst ratio of error to the bound)."""
    y_ref, R, B = ref
    y = np.asarray(y, dtype=np.float64)
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    bad = ~np.isfinite(y)
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs not finite (never written?), first at " \
                          f"{np.argwhere(bad)[0].tolist()}"
    lim = bound(y_ref, R, B, out_kind)
    err = np.abs(y - y_ref)
    ratio = err / np.maximum(lim, 1e-300)
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert ratio[worst] <= 1.0, (f"{what}: element {list(worst)} off by {err[worst]:.4g}, bound {lim[worst]:.4g}; "
                                 f"{int((ratio > 1).sum())} elements over the bound")
    nrm = float(np.linalg.norm(y_ref))
    rel = float(np.linalg.norm(y - y_ref) / nrm) if nrm > 0 else float(np.linalg.norm(y))
    assert rel <= TOL, f"{what}: relative L2 error {rel:.3e} > {TOL}"
    return rel, float(ratio[worst])
