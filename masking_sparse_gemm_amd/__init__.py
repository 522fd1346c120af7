"""Python binding of libnm, the MI355X (gfx950) N:M masking / compression / sparse-GEMM library.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
of ``include/nm.h``.  PyTorch supplies device memory and the current stream.
There is no CPU fallback: if ``libnm.so`` has not been built, importing the
library functions raises.

    values, meta = compress(W, 2, 4)          # W: (R, K) bf16/fp16/fp32 on a gfx950 GPU
    Y = spmm(values, meta, X, 2, 4)           # X: (K, T), Y: (R, T)
    keep = mask(W, 2, 4)                      # bool (R, K)
    Wd = decompress(values, meta, 2, 4, K)    # dense (R, K), +0 where pruned
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnm.so")

NM_F32, NM_F16, NM_BF16 = 0, 1, 2
_DT = {torch.float32: NM_F32, torch.float16: NM_F16, torch.bfloat16: NM_BF16}
_TORCH_DT = {v: k for k, v in _DT.items()}
STATUS = ["ok", "null", "shape", "pattern", "dtype", "align", "unsupported", "device"]

# every function the C header declares
EXPORTS = ("nm_abi_version", "nm_status_str", "nm_values_bytes", "nm_meta_words_per_row",
           "nm_mask", "nm_compress", "nm_decompress", "nm_spmm")


class NMError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {text} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libnm.so with argument types declared (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m masking_sparse_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.nm_abi_version.restype = i32
        L.nm_status_str.argtypes = [i32]
        L.nm_status_str.restype = ctypes.c_char_p
        L.nm_values_bytes.argtypes = [i64, i64, i32, i32, i32]
        L.nm_values_bytes.restype = ctypes.c_size_t
        L.nm_meta_words_per_row.argtypes = [i64, i32, i32]
        L.nm_meta_words_per_row.restype = i64
        L.nm_mask.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp]
        L.nm_compress.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp]
        L.nm_decompress.argtypes = [vp, vp, i32, i64, i64, i32, i32, vp, vp]
        L.nm_spmm.argtypes = [vp, vp, i64, i64, i32, i32, vp, i64, i32, vp, i32, vp]
        for f in ("nm_mask", "nm_compress", "nm_decompress", "nm_spmm"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def status_str(code: int) -> str:
    return lib().nm_status_str(code).decode()


def _check(fn: str, code: int) -> None:
    if code != 0:
        raise NMError(fn, code, status_str(code))


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _dense_input(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    if t.dtype not in _DT:
        raise ValueError(f"{name} must be float32, float16 or bfloat16")
    return _DT[t.dtype]


def meta_words_per_row(K: int, n: int, m: int) -> int:
    return int(lib().nm_meta_words_per_row(K, n, m))


def mask(W: torch.Tensor, n: int = 2, m: int = 4) -> torch.Tensor:
    """Bool (R, K): True where the weight is kept by the magnitude-best N:M pattern."""
    dt = _dense_input(W, "W")
    R, K = W.shape
    out = torch.empty((R, K), dtype=torch.bool, device=W.device)
    _check("nm_mask", lib().nm_mask(_ptr(W), dt, R, K, n, m, _ptr(out), _stream(W)))
    return out


def compress(W: torch.Tensor, n: int = 2, m: int = 4):
    """(values (R, K*n/m) in W's dtype, meta (R, words) int32 holding the uint32 bit fields)."""
    dt = _dense_input(W, "W")
    R, K = W.shape
    if K % m:
        raise ValueError("K must be a multiple of m")
    words = meta_words_per_row(K, n, m)
    if words < 0:
        _check("nm_compress", 3)
    values = torch.empty((R, K // m * n), dtype=W.dtype, device=W.device)
    meta = torch.empty((R, words), dtype=torch.int32, device=W.device)
    _check("nm_compress", lib().nm_compress(_ptr(W), dt, R, K, n, m, _ptr(values), _ptr(meta),
                                            _stream(W)))
    return values, meta


def _check_compressed(values: torch.Tensor, meta: torch.Tensor, n: int, m: int, K: int) -> int:
    dt = _dense_input(values, "values")
    R = values.shape[0]
    words = meta_words_per_row(K, n, m)
    if words < 0:
        _check("nm_decompress", 3)
    if values.shape != (R, K // m * n):
        raise ValueError(f"values must be ({R}, {K // m * n}) for K={K}, {n}:{m}")
    if meta.dtype != torch.int32 or meta.shape != (R, words) or not meta.is_contiguous():
        raise ValueError(f"meta must be a contiguous int32 ({R}, {words}) tensor")
    if meta.device != values.device:
        raise ValueError("values and meta must be on the same device")
    return dt


def decompress(values: torch.Tensor, meta: torch.Tensor, n: int, m: int, K: int) -> torch.Tensor:
    """Dense (R, K): stored values at their positions, +0 elsewhere."""
    dt = _check_compressed(values, meta, n, m, K)
    R = values.shape[0]
    out = torch.empty((R, K), dtype=values.dtype, device=values.device)
    _check("nm_decompress", lib().nm_decompress(_ptr(values), _ptr(meta), dt, R, K, n, m,
                                                _ptr(out), _stream(values)))
    return out


def spmm(values: torch.Tensor, meta: torch.Tensor, X: torch.Tensor, n: int = 2, m: int = 4,
         out_dtype: torch.dtype | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Y (R, T) = W_sparse @ X with fp32 accumulation; out_dtype is X's dtype or float32."""
    xdt = _dense_input(X, "X")
    K, T = X.shape
    dt = _check_compressed(values, meta, n, m, K)
    if dt != xdt:
        raise ValueError("values and X must have the same dtype")
    R = values.shape[0]
    y_dtype = out_dtype or X.dtype
    if out is None:
        out = torch.empty((R, T), dtype=y_dtype, device=X.device)
    elif out.shape != (R, T) or out.dtype != y_dtype or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    if y_dtype not in _DT:
        raise ValueError("out_dtype must be float32, float16 or bfloat16")
    _check("nm_spmm", lib().nm_spmm(_ptr(values), _ptr(meta), R, K, n, m, _ptr(X), T, dt,
                                    _ptr(out), _DT[y_dtype], _stream(X)))
    return out
