"""Build libw4a16.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python gemm_w4a16_amd/build.py         # or __graft_entry__.build()

Flags that matter for the numerics:
  -fhip-fp32-correctly-rounded-divide-sqrt  the quantizers use IEEE fp32 division
  -fno-gpu-flush-denormals-to-zero          fp32 denormals are kept
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                            no packed-fp32 (v_pk_*_f32) instructions are emitted
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libw4a16.so"
BUILD_DIR = PKG / "_build"
ARCH = "gfx950"

SOURCES = ["api.hip", "pack.hip", "gemv.hip", "rowmma.hip", "skinny.hip", "mid.hip", "gemm.hip", "w4a8.hip"]
# The benchmark's measured roofs (a streaming read, an empty launch): a library of their own, so
# that nothing in libw4a16 exists only to be timed.
ROOF_SOURCE, ROOF_LIB = "roof.hip", PKG / "libw4a16_roof.so"
# Per-file extra flags.  In the weight-streaming kernels the first kernel arguments arrive in SGPRs
# at wave launch, so a wave's first loads wait for no scalar fetch of the argument block (a code
# object still runs where the dispatcher does not preload: it then starts at a short block that
# loads the same SGPRs).  Measured: 0.4-1.7% faster for 1..16 rows and the row-major GEMVs, 0.5-2.6%
# for the row-major matrix-core kernel, 2% for W4A8's quantize-and-product step; the 17..64-row
# kernels ran 1-4% slower with it and the GEMM alike, so they do without.
PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=16"]
FILE_FLAGS: dict = {"skinny.hip": PRELOAD, "gemv.hip": PRELOAD, "rowmma.hip": PRELOAD, "w4a8.hip": PRELOAD}

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the W4A16 HIP library cannot be built")
    return path


def _compile(src: str) -> Path:
    obj = BUILD_DIR / (Path(src).stem + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), "-c", str(CSRC / src), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(noise))
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def _link(objs, out: Path) -> None:
    tmp = out.with_suffix(f".so.tmp{os.getpid()}")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + res.stderr)
    os.replace(tmp, out)


def build() -> Path:
    """Compile every source (in parallel) and link libw4a16.so and libw4a16_roof.so; always
    rebuilds."""
    BUILD_DIR.mkdir(exist_ok=True)
    srcs = SOURCES + [ROOF_SOURCE]
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:-1], LIB)
    _link(objs[-1:], ROOF_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
