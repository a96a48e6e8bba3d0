"""Python binding of libw4a16 (MI355X / gfx950 W4A16 matmul).

Argument marshalling only: every function below forwards to the C entry point of the same
name in ``libw4a16.so`` (declared in ``include/w4a16.h``) and does no arithmetic of its own.
PyTorch supplies device memory and the current HIP stream; nothing here falls back to torch or
to the CPU.  If the library has not been built, importing this package fails with an error
that says how to build it.

Array arguments may be torch tensors (their ``data_ptr()`` is passed), plain integers (raw
device pointers) or ``None`` (a NULL pointer).
"""
from __future__ import annotations

import ctypes
from pathlib import Path

_LIB_PATH = Path(__file__).resolve().parent / "libw4a16.so"

W4A16_OK, W4A16_ERR_INVALID, W4A16_ERR_UNSUPPORTED, W4A16_ERR_DEVICE = 0, 1, 2, 3
W4A16_FMT_G128_ASYM_BF16, W4A16_FMT_Q4_B32_SYM_FP16, W4A16_FMT_G128_ZP_FP16, W4A16_FMT_W8_ROW_FP32 = 0, 1, 2, 3
W4A16_BF16, W4A16_FP16, W4A16_FP32 = 0, 1, 2

# Every symbol include/w4a16.h declares.
EXPORTED = (
    "w4a16_status_string", "w4a16_packed_sizes", "w4a16_quantize_pack", "w4a16_dequant",
    "w4a16_gemv", "w4a16_gemv_max_rows", "w4a16_gemm_workspace_bytes", "w4a16_gemm",
    "w4a16_matmul", "w4a16_matmul_gemv_cutoff", "w4a16_quantize_act_i8", "w4a16_gemm_w4a8",
    "w4a16_matmul_w4a8", "w4a16_check_weights", "w4a16_matmul_noalloc", "w4a16_matmul_noalloc_max_scratch_bytes",
    "w4a16_prepared_bytes", "w4a16_prepare", "w4a16_gemv_prepared",
)


class W4A16Error(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {status_string(status)} (status {status})")


def _load() -> ctypes.CDLL:
    if not _LIB_PATH.exists():
        raise ImportError(f"{_LIB_PATH} is not built; run `python gemm_w4a16_amd/build.py` "
                          "(hipcc for gfx950). There is no fallback path.")
    # PyTorch ships its own HIP runtime (libamdhip64.so.7).  It must be the one in the process
    # before libw4a16.so is loaded, so that the library's dependency on libamdhip64.so.7 binds to
    # it: loaded first, libw4a16.so would pull in the system runtime and torch would then load a
    # second one, whose streams and allocations the library's runtime does not know (every
    # launch on a torch stream would then fail).
    import torch  # noqa: F401
    L = ctypes.CDLL(str(_LIB_PATH))
    P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.w4a16_status_string.argtypes, L.w4a16_status_string.restype = [I], ctypes.c_char_p
    L.w4a16_packed_sizes.argtypes = [I, I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ), ctypes.POINTER(SZ)]
    L.w4a16_quantize_pack.argtypes = [I, P, I64, I64, P, P, P, P]
    L.w4a16_dequant.argtypes = [I, P, P, P, I64, I64, I, P, P]
    L.w4a16_check_weights.argtypes = [I, P, I64, I64]
    L.w4a16_gemv.argtypes = [I, I, P, I64, P, P, P, I64, I64, P, P]
    L.w4a16_gemv_max_rows.argtypes, L.w4a16_gemv_max_rows.restype = [], I64
    L.w4a16_gemm_workspace_bytes.argtypes, L.w4a16_gemm_workspace_bytes.restype = [I, I64, I64, I64], SZ
    L.w4a16_gemm.argtypes = [I, I, P, I64, P, P, P, I64, I64, P, P, SZ, P]
    L.w4a16_matmul.argtypes = [I, I, P, I64, P, P, P, I64, I64, P, P, SZ, P]
    L.w4a16_matmul_gemv_cutoff.argtypes, L.w4a16_matmul_gemv_cutoff.restype = [], I64
    L.w4a16_matmul_noalloc.argtypes = [I, I, P, I64, P, P, P, I64, I64, P, P]
    L.w4a16_matmul_noalloc_max_scratch_bytes.argtypes = []
    L.w4a16_matmul_noalloc_max_scratch_bytes.restype = SZ
    L.w4a16_prepared_bytes.argtypes, L.w4a16_prepared_bytes.restype = [I, I64, I64], SZ
    L.w4a16_prepare.argtypes = [I, P, P, P, I64, I64, P, SZ, P]
    L.w4a16_gemv_prepared.argtypes = [I, I, P, I64, P, I64, I64, P, P]
    L.w4a16_quantize_act_i8.argtypes = [P, I64, I64, P, P, P, P]
    L.w4a16_gemm_w4a8.argtypes = [I, P, P, P, I64, P, P, P, I64, I64, P, P]
    L.w4a16_matmul_w4a8.argtypes = [I, P, I64, P, P, P, I64, I64, P, P]
    for name in ("w4a16_packed_sizes", "w4a16_quantize_pack", "w4a16_check_weights", "w4a16_dequant", "w4a16_gemv",
                 "w4a16_gemm", "w4a16_matmul", "w4a16_matmul_noalloc", "w4a16_quantize_act_i8", "w4a16_gemm_w4a8",
                 "w4a16_matmul_w4a8", "w4a16_prepare", "w4a16_gemv_prepared"):
        getattr(L, name).restype = I
    return L


lib = _load()
library_path = str(_LIB_PATH)


def _p(a):
    """Device pointer of a torch tensor / raw int / None."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ok(status: int, call: str) -> None:
    if status != W4A16_OK:
        raise W4A16Error(status, call)


def status_string(status: int) -> str:
    return lib.w4a16_status_string(int(status)).decode()


w4a16_status_string = status_string


def w4a16_packed_sizes(fmt: int, N: int, K: int):
    c, s, m = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _ok(lib.w4a16_packed_sizes(fmt, N, K, ctypes.byref(c), ctypes.byref(s), ctypes.byref(m)),
        "w4a16_packed_sizes")
    return c.value, s.value, m.value


def w4a16_quantize_pack(fmt: int, W, N: int, K: int, codes, scales, mins, stream=None) -> None:
    _ok(lib.w4a16_quantize_pack(fmt, _p(W), N, K, _p(codes), _p(scales), _p(mins), _stream(stream)),
        "w4a16_quantize_pack")


def w4a16_check_weights(fmt: int, W, N: int, K: int) -> None:
    """Host-side weight check (W: a C-contiguous float32 numpy array or a host address)."""
    addr = W if isinstance(W, int) or W is None else W.ctypes.data
    _ok(lib.w4a16_check_weights(fmt, addr, N, K), "w4a16_check_weights")


def w4a16_dequant(fmt: int, codes, scales, mins, N: int, K: int, out_dtype: int, W_hat, stream=None) -> None:
    _ok(lib.w4a16_dequant(fmt, _p(codes), _p(scales), _p(mins), N, K, out_dtype, _p(W_hat), _stream(stream)),
        "w4a16_dequant")


def w4a16_gemv(fmt: int, act: int, x, M: int, codes, scales, mins, N: int, K: int, y, stream=None) -> None:
    _ok(lib.w4a16_gemv(fmt, act, _p(x), M, _p(codes), _p(scales), _p(mins), N, K, _p(y), _stream(stream)),
        "w4a16_gemv")


def w4a16_gemv_max_rows() -> int:
    return int(lib.w4a16_gemv_max_rows())


def w4a16_gemm_workspace_bytes(fmt: int, M: int, N: int, K: int) -> int:
    return int(lib.w4a16_gemm_workspace_bytes(fmt, M, N, K))


def w4a16_gemm(fmt: int, act: int, x, M: int, codes, scales, mins, N: int, K: int, y, workspace=None,
               workspace_bytes: int = 0, stream=None) -> None:
    _ok(lib.w4a16_gemm(fmt, act, _p(x), M, _p(codes), _p(scales), _p(mins), N, K, _p(y), _p(workspace),
                       workspace_bytes, _stream(stream)), "w4a16_gemm")


def w4a16_matmul(fmt: int, act: int, x, M: int, codes, scales, mins, N: int, K: int, y, workspace=None,
                 workspace_bytes: int = 0, stream=None) -> None:
    _ok(lib.w4a16_matmul(fmt, act, _p(x), M, _p(codes), _p(scales), _p(mins), N, K, _p(y), _p(workspace),
                         workspace_bytes, _stream(stream)), "w4a16_matmul")


def w4a16_matmul_noalloc(fmt: int, act: int, x, M: int, codes, scales, mins, N: int, K: int, y, stream=None) -> None:
    _ok(lib.w4a16_matmul_noalloc(fmt, act, _p(x), M, _p(codes), _p(scales), _p(mins), N, K, _p(y), _stream(stream)),
        "w4a16_matmul_noalloc")


def w4a16_matmul_noalloc_max_scratch_bytes() -> int:
    return int(lib.w4a16_matmul_noalloc_max_scratch_bytes())


def w4a16_prepared_bytes(fmt: int, N: int, K: int) -> int:
    return int(lib.w4a16_prepared_bytes(fmt, N, K))


def w4a16_prepare(fmt: int, codes, scales, mins, N: int, K: int, prepared, prepared_bytes: int, stream=None) -> None:
    _ok(lib.w4a16_prepare(fmt, _p(codes), _p(scales), _p(mins), N, K, _p(prepared), prepared_bytes,
                             _stream(stream)), "w4a16_prepare")


def w4a16_gemv_prepared(fmt: int, act: int, x, M: int, prepared, N: int, K: int, y, stream=None) -> None:
    _ok(lib.w4a16_gemv_prepared(fmt, act, _p(x), M, _p(prepared), N, K, _p(y), _stream(stream)),
        "w4a16_gemv_prepared")


def w4a16_matmul_gemv_cutoff() -> int:
    return int(lib.w4a16_matmul_gemv_cutoff())


def w4a16_quantize_act_i8(x, M: int, K: int, xq, ascale, xsum, stream=None) -> None:
    _ok(lib.w4a16_quantize_act_i8(_p(x), M, K, _p(xq), _p(ascale), _p(xsum), _stream(stream)),
        "w4a16_quantize_act_i8")


def w4a16_gemm_w4a8(fmt: int, xq, ascale, xsum, M: int, codes, scales, mins, N: int, K: int, y,
                    stream=None) -> None:
    _ok(lib.w4a16_gemm_w4a8(fmt, _p(xq), _p(ascale), _p(xsum), M, _p(codes), _p(scales), _p(mins), N, K,
                            _p(y), _stream(stream)), "w4a16_gemm_w4a8")


def w4a16_matmul_w4a8(fmt: int, x, M: int, codes, scales, mins, N: int, K: int, y, stream=None) -> None:
    _ok(lib.w4a16_matmul_w4a8(fmt, _p(x), M, _p(codes), _p(scales), _p(mins), N, K, _p(y), _stream(stream)),
        "w4a16_matmul_w4a8")


# ---- memory plumbing (torch allocations with the ABI's shapes and dtypes) ------------------------

def alloc_packed(fmt: int, N: int, K: int, device="cuda"):
    """Empty (codes, scales, mins) device tensors for an N x K weight (mins is None for Q4 and W8;
    the zero points for the zero-point format)."""
    import torch
    w4a16_packed_sizes(fmt, N, K)  # validates the shape
    if fmt == W4A16_FMT_G128_ASYM_BF16:
        # scales/mins: [K/128][N] views of buffers padded to the size w4a16_packed_sizes asks for
        n = K // 128 * N
        padded = n + (n & 1)
        return (torch.empty((K // 8, N), dtype=torch.int32, device=device),
                torch.empty(padded, dtype=torch.int16, device=device)[:n].view(K // 128, N),
                torch.empty(padded, dtype=torch.int16, device=device)[:n].view(K // 128, N))
    if fmt == W4A16_FMT_W8_ROW_FP32:
        return (torch.empty((N, K), dtype=torch.int8, device=device),
                torch.empty(N, dtype=torch.float32, device=device),
                None)
    if fmt == W4A16_FMT_G128_ZP_FP16:
        return (torch.empty((N, K // 8), dtype=torch.int32, device=device),
                torch.empty((N, K // 128), dtype=torch.int16, device=device),
                torch.empty((N, K // 128), dtype=torch.int16, device=device))
    return (torch.empty((N, K // 32, 16), dtype=torch.uint8, device=device),
            torch.empty((N, K // 32), dtype=torch.int16, device=device),
            None)


def alloc_act_i8(M: int, K: int, device="cuda"):
    """Empty (xq int8 [M][K], ascale fp32 [M], xsum fp32 [K/128][M]) for w4a16_quantize_act_i8."""
    import torch
    return (torch.empty((M, K), dtype=torch.int8, device=device),
            torch.empty(M, dtype=torch.float32, device=device),
            torch.empty((K // 128, M), dtype=torch.float32, device=device))


def alloc_workspace(fmt: int, M: int, N: int, K: int, device="cuda"):
    """(tensor or None, bytes) sized for w4a16_gemm / w4a16_matmul on this shape."""
    import torch
    nbytes = w4a16_gemm_workspace_bytes(fmt, M, N, K)
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes
