"""Seeded synthetic inputs for the W4A16 matmul: the only module shared by the oracle side and
the HIP side.  It holds random draws and shapes, none of the method's arithmetic.

Shapes follow the pages' workloads: the Llama-3-8B MLP up projection, K=4096 -> N=14336, that
vidyal.ai "Low-Precision Kernels" times from 1 to 4,096 rows (sections "Step 1" and "Step 3"),
and the 16384 x 16384 Q4 GEMV of thuongvuho.com "Why My 4-Bit CUDA Kernel Wasn't Faster"
(section "Where the time went").  Both pages time random weights, as here.

Recipe (the same arrays reach the oracle and the GPU; nothing is read from disk):
* weights: numpy ``default_rng(seed_w).standard_normal((N, K), float32) * 0.02``;
* outliers (decode shape): ``default_rng(seed_w + 1)`` picks ``round(0.001*N*K)`` distinct flat
  positions, multiplied by 20;
* activations: ``default_rng(seed_x).standard_normal((M, K), float32)``, rounded to bf16 (torch,
  round-to-nearest-even) or to fp16 (numpy, round-to-nearest-even), returned as raw 16-bit
  patterns; a batch sweep takes the first M rows of one draw of the largest M.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    fmt: str          # "g128" (asymmetric group 128, bf16 scale+min), "q4b32" (symmetric block 32) or
                      # "g128zp" (group 128, fp16 scale + integer zero point) or "w8row" (int8, row scale)
    M: int
    N: int
    K: int
    act: str          # "bf16" or "f16"
    outliers: bool = False
    seed_w: int = 0
    seed_x: int = 2


# The five workloads: a tiny GEMV, the decode GEMV, its batch sweep, the Q4 GEMV and prefill.
TINY = Workload("tiny_gemv_m1_n256_k512", "g128", 1, 256, 512, "bf16")
DECODE = Workload("decode_gemv_m1_k4096_n14336", "g128", 1, 14336, 4096, "bf16", outliers=True)
SWEEP_MS = (1, 2, 4, 8, 16, 32, 64, 128, 256)
Q4 = Workload("q4b32_gemv_m1_k16384_n16384", "q4b32", 1, 16384, 16384, "f16")
PREFILL = Workload("prefill_gemm_m1024_k4096_n14336", "g128", 1024, 14336, 4096, "bf16", outliers=True)
# The decode shape in the integer-zero-point format of anrans.github.io "Quantization and GEMV"
# (its GEMV example uses fp32 activations and notes that real kernels use FP16/BF16).
ZP_DECODE = Workload("zp_gemv_m1_k4096_n14336", "g128zp", 1, 14336, 4096, "f16", outliers=True)
# ... and in the per-row int8 format of that page's first exercise (W8A16).
W8_DECODE = Workload("w8_gemv_m1_k4096_n14336", "w8row", 1, 14336, 4096, "f16", outliers=True)


def sweep(M: int) -> Workload:
    assert M in SWEEP_MS
    return Workload(f"sweep_m{M}_k4096_n14336", "g128", M, 14336, 4096, "bf16", outliers=True)


def weights(N: int, K: int, outliers: bool = False, seed: int = 0) -> np.ndarray:
    """fp32 [N][K] ~ N(0, 0.02); with ``outliers`` 0.1% of the entries are scaled by 20."""
    W = np.random.default_rng(seed).standard_normal((N, K), dtype=np.float32)
    W *= np.float32(0.02)
    if outliers:
        count = int(round(0.001 * N * K))
        idx = np.random.default_rng(seed + 1).choice(N * K, size=count, replace=False)
        W.reshape(-1)[idx] *= np.float32(20.0)
    return W


def activations(M: int, K: int, dtype: str = "bf16", seed: int = 2, rows_drawn: int | None = None) -> np.ndarray:
    """[M][K] 16-bit patterns (uint16) of x ~ N(0, 1) rounded to ``dtype`` ("bf16" or "f16").

    ``rows_drawn`` > M draws that many rows and keeps the first M (the batch sweep)."""
    R = max(M, rows_drawn or M)
    x = np.random.default_rng(seed).standard_normal((R, K), dtype=np.float32)[:M]
    x = np.ascontiguousarray(x)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    raise ValueError(f"unknown activation dtype {dtype!r}")


def inputs(w: Workload):
    """(W fp32 [N][K], x bits uint16 [M][K]) for a workload."""
    rows = max(SWEEP_MS) if w.name.startswith("sweep_") else None
    return (weights(w.N, w.K, w.outliers, w.seed_w),
            activations(w.M, w.K, w.act, w.seed_x, rows_drawn=rows))


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen 16-bit patterns to fp32 (exact) -- a view change for test plumbing, not the method."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    return bits.view(np.float16).astype(np.float32)
