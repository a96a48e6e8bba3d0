"""The element-wise check of tests/refcheck.py, pinned on the CPU.

Numpy emulations of the two arithmetics the GPU paths use must pass it: the large-M path (weights
dequantized as fmaf(q, s, min), rounded to bf16, summed in fp32, output rounded to bf16; vidyal.ai
"Low-Precision Kernels", Step 2) and the factored small-M path (per group, in fp32,
s * sum(x (128 + q)) + (min - 128 s) * sum(x)).  Outputs a faulty kernel would produce must fail
it: an output never written, a zeroed 16-column segment, a group dropped from one column, a tile
whose columns are shifted by one, and a group whose minimum has the wrong sign.
"""
import numpy as np
import pytest
import torch

import oracle
import refcheck
import workloads

M, N, K = 70, 300, 1024


def _bf16_round(v):
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.float().numpy()


@pytest.fixture(scope="module")
def problem():
    W = workloads.weights(N, K, outliers=True, seed=81)
    W[3, :128] = 0.7                                                   # max == min: scale 1
    W[5, 128:256] = 100.0 + np.arange(128, dtype=np.float32) * 1e-4    # narrow band far from zero
    x = workloads.activations(M, K, "bf16", seed=82)
    x[4] = 0                                                           # a zero row
    xf = workloads.bits_to_f32(x, "bf16")
    xf[6] *= np.float32(2.0 ** 12)                                     # rows of different scale
    xf[7] *= np.float32(2.0 ** -12)
    x = _bf16_bits(xf)
    packed = oracle.quantize_g128(W)
    return x, packed, refcheck.g128(x, *packed)


def _bf16_bits(v):
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _gemm_emulation(x, packed):
    Wb = workloads.bits_to_f32(oracle.dequant_g128(*packed, "bf16"), "bf16")   # bf16(fmaf(q, s, m))
    y32 = workloads.bits_to_f32(x, "bf16") @ Wb.T                                # fp32 sums
    return _bf16_round(y32)


def _factored_emulation(x, packed):
    codes, scales, mins = packed
    xf = workloads.bits_to_f32(x, "bf16")
    q = np.empty((N, K), dtype=np.float32)
    for j in range(8):
        q[:, j::8] = ((codes >> (4 * j)) & 0xF).T.astype(np.float32)
    s = workloads.bits_to_f32(scales, "bf16")
    m = workloads.bits_to_f32(mins, "bf16")
    y = np.zeros((M, N), dtype=np.float32)
    for g in range(K // 128):
        sl = slice(128 * g, 128 * g + 128)
        acc = xf[:, sl] @ (128.0 + q[:, sl]).T.astype(np.float32)       # fp32 sums
        accs = xf[:, sl].sum(axis=1, dtype=np.float32)[:, None]
        c = (m[g] - np.float32(128.0) * s[g]).astype(np.float32)
        y = (y + s[g] * acc).astype(np.float32)
        y = (y + c * accs).astype(np.float32)
    return _bf16_round(y)


def test_both_arithmetics_pass(problem):
    x, packed, ref = problem
    rel_g, worst_g = refcheck.check(_gemm_emulation(x, packed), ref, "bf16", "gemm emulation")
    rel_f, worst_f = refcheck.check(_factored_emulation(x, packed), ref, "bf16", "factored emulation")
    assert rel_g < 3e-3 and rel_f < 3e-3
    assert worst_g < 0.5 and worst_f < 0.5          # the bound has room, but not orders of magnitude
    assert worst_g > 1e-3


def _fails(y, ref):
    with pytest.raises(AssertionError):
        refcheck.check(y, ref, "bf16")


def test_planted_faults_fail(problem):
    x, packed, ref = problem
    good = _gemm_emulation(x, packed)
    y = good.copy()
    y[10, 200] = np.nan                               # an output never written (NaN sentinel)
    _fails(y, ref)
    y = good.copy()
    y[33, 64:80] = 0.0                                # one 16-column segment of one row
    _fails(y, ref)
    y = good.copy()
    y[:, 120:184] = good[:, 121:185]                  # a 64-column tile read one column off
    _fails(y, ref)
    codes, scales, mins = packed
    # one group (g = 5) dropped from column 17, in every row
    xf = workloads.bits_to_f32(x, "bf16").astype(np.float64)
    What = oracle.dequant_g128(codes, scales, mins, "f64")
    y = good.copy()
    y[:, 17] -= (xf[:, 640:768] @ What[17, 640:768]).astype(np.float32)
    _fails(y, ref)
    # the minimum of group 2 of column 40 with the wrong sign
    m = workloads.bits_to_f32(mins, "bf16").astype(np.float64)
    y = good.copy()
    y[:, 40] -= (2 * m[2, 40] * xf[:, 256:384].sum(axis=1)).astype(np.float32)
    _fails(y, ref)


def test_zero_row_must_be_exactly_zero(problem):
    x, packed, ref = problem
    y = _gemm_emulation(x, packed)
    assert np.all(y[4] == 0)
    y[4, 9] = 1e-30
    _fails(y, ref)
