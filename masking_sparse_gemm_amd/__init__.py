"""Python binding of libnm, the MI355X (gfx950) N:M masking / compression / sparse-GEMM library.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
of ``include/nm.h``.  PyTorch supplies device memory and the current stream.
There is no CPU fallback: if ``libnm.so`` has not been built, importing the
library functions raises.

    values, meta = compress(W, 2, 4)          # W: (R, K) bf16/fp16/fp32 on a gfx950 GPU
    Y = spmm(values, meta, X, 2, 4)           # X: (K, T), Y: (R, T)
    keep = mask(W, 2, 4)                      # bool (R, K)
    Wd = decompress(values, meta, 2, 4, K)    # dense (R, K), +0 where pruned
    Wp = prune(W, 2, 4)                       # SR-STE forward weight: W where kept, +0 else
    srste_grad(W, G, 2, 4, out=G)             # SR-STE backward, in place on G
    Wt = tprune(W, 2, 4)                      # transposable 2:4 mask applied (4x4 blocks)
    vt, mt = compress_t(Wt, 2, 4)             # compressed W^T: spmm(vt, mt, dY) = W^T dY

The compressed pair comes in two layouts (defined in include/nm.h): "rows"
(values (R, K*n/m), meta (R, words)) and "blocked" (blocks of 16 rows x 64
columns, the order the sparse product streams; values (G, S, 16, 64*n/m), meta
(G, S, words per block) with G = ceil(R/16), S = K/64).  A blocked pair does not
record R, so decompress and spmm take it as ``rows=``.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# NM_LIB_PATH names another build of the same library (the sanitizer test's host-instrumented one)
LIB_PATH = os.environ.get("NM_LIB_PATH") or os.path.join(HERE, "libnm.so")

NM_F32, NM_F16, NM_BF16, NM_I8, NM_I32, NM_FP8 = 0, 1, 2, 3, 4, 5
_DT = {torch.float32: NM_F32, torch.float16: NM_F16, torch.bfloat16: NM_BF16, torch.int8: NM_I8,
       torch.int32: NM_I32, torch.float8_e4m3fn: NM_FP8}
_BYTE = (torch.int8, torch.float8_e4m3fn)  # 1-byte element types (no training-side calls)
_FLOAT = (torch.float32, torch.float16, torch.bfloat16)
_TORCH_DT = {v: k for k, v in _DT.items()}
STATUS = ["ok", "null", "shape", "pattern", "dtype", "align", "unsupported", "device", "layout",
          "alias", "scratch"]
LAYOUTS = {"rows": 0, "blocked": 1}
ABI_VERSION = 10

# every function the C header declares
EXPORTS = ("nm_abi_version", "nm_status_str", "nm_values_bytes", "nm_meta_bytes",
           "nm_meta_words_per_row", "nm_mask", "nm_compress", "nm_decompress", "nm_spmm",
           "nm_prune", "nm_srste_grad", "nm_tmask", "nm_tprune", "nm_compress_t",
           "nm_perm_workspace_bytes", "nm_perm_gains", "nm_perm_search", "nm_check_meta",
           "nm_mask_compress", "nm_perm_gains_static")
STATIC_SCRATCH_BYTES = 64 << 20  # NM_STATIC_SCRATCH_BYTES
SRSTE_DECAY = 0.0002  # the SR-STE page's default decay


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
        L.nm_values_bytes.argtypes = [i64, i64, i32, i32, i32, i32]
        L.nm_values_bytes.restype = ctypes.c_size_t
        L.nm_meta_bytes.argtypes = [i64, i64, i32, i32, i32]
        L.nm_meta_bytes.restype = ctypes.c_size_t
        L.nm_meta_words_per_row.argtypes = [i64, i32, i32]
        L.nm_meta_words_per_row.restype = i64
        L.nm_check_meta.argtypes = [vp, i64, i64, i32, i32, i32]
        L.nm_check_meta.restype = i64
        L.nm_mask.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp]
        L.nm_compress.argtypes = [vp, i32, i64, i64, i32, i32, i32, vp, vp, vp]
        L.nm_mask_compress.argtypes = [vp, i32, i64, i64, i32, i32, i32, vp, vp, vp, vp]
        L.nm_decompress.argtypes = [vp, vp, i32, i64, i64, i32, i32, i32, vp, vp]
        L.nm_spmm.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, i64, i32, vp, i32, vp]
        L.nm_prune.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp]
        L.nm_srste_grad.argtypes = [vp, vp, i32, i64, i64, i32, i32, ctypes.c_float, vp, vp]
        L.nm_tmask.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp]
        L.nm_tprune.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp]
        L.nm_compress_t.argtypes = [vp, i32, i64, i64, i32, i32, i32, vp, vp, vp]
        L.nm_perm_workspace_bytes.argtypes = [i64, i64, i32, i32]
        L.nm_perm_workspace_bytes.restype = ctypes.c_size_t
        L.nm_perm_gains.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.nm_perm_search.argtypes = [vp, i32, i64, i64, i32, i32, i32, vp, vp, vp,
                                     ctypes.c_size_t, vp]
        L.nm_perm_gains_static.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp, vp]
        for f in ("nm_mask", "nm_compress", "nm_decompress", "nm_spmm", "nm_prune",
                  "nm_srste_grad", "nm_tmask", "nm_tprune", "nm_compress_t", "nm_perm_gains",
                  "nm_perm_search", "nm_perm_gains_static"):
            getattr(L, f).restype = i32
        if L.nm_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} has ABI {L.nm_abi_version()}, expected {ABI_VERSION}: "
                              "rebuild it")
        _lib = L
    return _lib


PROBE_LIB_PATH = os.path.join(HERE, "libnm_probe.so")
_probe = None


def probe_lib() -> ctypes.CDLL:
    """The loaded libnm_probe.so (include/nm_probe.h): the benchmark's matrix-core, VALU,
    copy and load-path probes (raises if it is not built)."""
    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError(f"{PROBE_LIB_PATH} is missing: build it with "
                              "`python -m masking_sparse_gemm_amd.build`")
        P = ctypes.CDLL(PROBE_LIB_PATH)
        vp = ctypes.c_void_p
        P.nm_probe_operand_bytes.restype = ctypes.c_int64
        P.nm_probe_operand_bytes.argtypes = []
        P.nm_probe_matrix_core.argtypes = [ctypes.c_int, vp, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, vp, vp, vp]
        P.nm_probe_matrix_core.restype = ctypes.c_int
        P.nm_probe_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                    vp, vp]
        P.nm_probe_valu.restype = ctypes.c_int
        P.nm_probe_copy.argtypes = [vp, vp, ctypes.c_int64, vp]
        P.nm_probe_copy.restype = ctypes.c_int
        P.nm_probe_load_path.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int64, vp]
        P.nm_probe_load_path.restype = ctypes.c_int
        _probe = P
    return _probe


def status_str(code: int) -> str:
    return lib().nm_status_str(code).decode()


def _check(fn: str, code: int) -> None:
    if code != 0:
        raise NMError(fn, code, status_str(code))


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _dense_input(t: torch.Tensor, name: str, int8: bool = True) -> int:
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    if t.dtype not in _FLOAT and not (int8 and t.dtype in _BYTE):
        raise ValueError(f"{name} must be float32, float16 or bfloat16" +
                         (", int8 or float8_e4m3fn" if int8 else ""))
    return _DT[t.dtype]


def meta_words_per_row(K: int, n: int, m: int) -> int:
    return int(lib().nm_meta_words_per_row(K, n, m))


def check_meta(meta: torch.Tensor, R: int, K: int, n: int = 2, m: int = 4,
               layout: str = "rows") -> int:
    """Host-side check of metadata (copied to host memory first): -1 if every group's
    positions are strictly ascending and row padding bits are zero, else the row-major
    index of the first malformed group."""
    host = meta.detach().to("cpu").contiguous()
    if host.dtype != torch.int32:
        raise ValueError("meta must be int32 (holding the uint32 words)")
    need = int(lib().nm_meta_bytes(R, K, n, m, _layout(layout)))
    if R * K and host.numel() * 4 < need:
        raise ValueError(f"meta holds {host.numel() * 4} bytes, {need} needed")
    res = int(lib().nm_check_meta(ctypes.c_void_p(host.data_ptr()), R, K, n, m, _layout(layout)))
    if res == -2:
        raise ValueError("invalid arguments (pattern, shape or layout)")
    return res


def _layout(layout: str) -> int:
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    return LAYOUTS[layout]


def compressed_shapes(R: int, K: int, n: int, m: int, layout: str = "rows"):
    """Shapes of (values, meta) for an R x K matrix: meta is int32 holding uint32 words."""
    lay = _layout(layout)
    words = meta_words_per_row(K, n, m)  # -1 for a bad pattern or K % m != 0
    if words < 0:
        _check("nm_compress", 2 if (m in (2, 4, 8) and 1 <= n <= m) else 3)
    if lay == 0:
        return (R, K // m * n), (R, words)
    if K % 64:
        _check("nm_compress", 8)
    V = 64 // m * n                      # values per row and 64-wide step
    B = V * {2: 1, 4: 2, 8: 3}[m] // 8   # metadata bytes per row and step
    return ((R + 15) // 16, K // 64, 16, V), ((R + 15) // 16, K // 64, 4 * B)


def mask(W: torch.Tensor, n: int = 2, m: int = 4) -> torch.Tensor:
    """Bool (R, K): True where the weight is kept by the magnitude-best N:M pattern."""
    dt = _dense_input(W, "W")
    R, K = W.shape
    out = torch.empty((R, K), dtype=torch.bool, device=W.device)
    _check("nm_mask", lib().nm_mask(_ptr(W), dt, R, K, n, m, _ptr(out), _stream(W)))
    return out


def compress(W: torch.Tensor, n: int = 2, m: int = 4, layout: str = "rows"):
    """(values in W's dtype, meta int32 holding the uint32 bit fields) in `layout`."""
    dt = _dense_input(W, "W")
    R, K = W.shape
    lay = _layout(layout)
    vshape, mshape = compressed_shapes(R, K, n, m, layout)
    values = torch.empty(vshape, dtype=W.dtype, device=W.device)
    meta = torch.empty(mshape, dtype=torch.int32, device=W.device)
    _check("nm_compress", lib().nm_compress(_ptr(W), dt, R, K, n, m, lay, _ptr(values),
                                            _ptr(meta), _stream(W)))
    return values, meta


def mask_compress(W: torch.Tensor, n: int = 2, m: int = 4, layout: str = "rows"):
    """(mask, values, meta) from one pass over W: mask as mask(), the pair as compress()."""
    dt = _dense_input(W, "W")
    R, K = W.shape
    lay = _layout(layout)
    vshape, mshape = compressed_shapes(R, K, n, m, layout)
    mask_out = torch.empty((R, K), dtype=torch.bool, device=W.device)
    values = torch.empty(vshape, dtype=W.dtype, device=W.device)
    meta = torch.empty(mshape, dtype=torch.int32, device=W.device)
    _check("nm_mask_compress", lib().nm_mask_compress(_ptr(W), dt, R, K, n, m, lay, _ptr(mask_out),
                                                      _ptr(values), _ptr(meta), _stream(W)))
    return mask_out, values, meta


def _check_compressed(values: torch.Tensor, meta: torch.Tensor, n: int, m: int, K: int,
                      layout: str, rows: int | None) -> tuple[int, int]:
    """(dtype code, R) of a compressed pair, after checking its shapes against K and n:m."""
    ok = values.dtype in _FLOAT or values.dtype in _BYTE
    if not ok or not values.is_cuda or not values.is_contiguous():
        raise ValueError("values must be a contiguous float32/float16/bfloat16/int8/float8 GPU "
                         "tensor")
    if _layout(layout) == 0:
        R = values.shape[0] if values.dim() == 2 else -1
        if rows is not None and rows != R:
            raise ValueError(f"rows={rows} does not match values ({R} rows)")
    else:
        if rows is None:
            raise ValueError("the blocked layout needs rows= (the matrix's row count)")
        R = rows
        if values.dim() != 4 or values.shape[0] != (R + 15) // 16:
            raise ValueError(f"blocked values must be ({(R + 15) // 16}, S, 16, V) for R={R}")
    vshape, mshape = compressed_shapes(R, K, n, m, layout)
    if tuple(values.shape) != tuple(vshape):
        raise ValueError(f"values must be {tuple(vshape)} for K={K}, {n}:{m}, {layout}")
    if meta.dtype != torch.int32 or tuple(meta.shape) != tuple(mshape) or not meta.is_contiguous():
        raise ValueError(f"meta must be a contiguous int32 {tuple(mshape)} tensor")
    if meta.device != values.device:
        raise ValueError("values and meta must be on the same device")
    return _DT[values.dtype], R


def decompress(values: torch.Tensor, meta: torch.Tensor, n: int, m: int, K: int,
               layout: str = "rows", rows: int | None = None) -> torch.Tensor:
    """Dense (R, K): stored values at their positions, +0 elsewhere."""
    dt, R = _check_compressed(values, meta, n, m, K, layout, rows)
    out = torch.empty((R, K), dtype=values.dtype, device=values.device)
    _check("nm_decompress", lib().nm_decompress(_ptr(values), _ptr(meta), dt, R, K, n, m,
                                                _layout(layout), _ptr(out), _stream(values)))
    return out


def spmm(values: torch.Tensor, meta: torch.Tensor, X: torch.Tensor, n: int = 2, m: int = 4,
         out_dtype: torch.dtype | None = None, out: torch.Tensor | None = None,
         layout: str = "rows", rows: int | None = None) -> torch.Tensor:
    """Y (R, T) = W_sparse @ X with fp32 accumulation; out_dtype is X's dtype or float32.
    int8 values and X give the exact int32 product (out_dtype torch.int32).  fp8 2:4 and
    1:2 products run on the fp8 structured-sparse instruction, which sums each run of 16 K
    in fixed point before the fp32 accumulator (include/nm.h states the bound)."""
    xdt = _dense_input(X, "X")
    K, T = X.shape
    dt, R = _check_compressed(values, meta, n, m, K, layout, rows)
    if dt != xdt:
        raise ValueError("values and X must have the same dtype")
    y_dtype = out_dtype or {torch.int8: torch.int32, torch.float8_e4m3fn: torch.float32}.get(
        X.dtype, X.dtype)
    if out is None:
        out = torch.empty((R, T), dtype=y_dtype, device=X.device)
    elif out.shape != (R, T) or out.dtype != y_dtype or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    if y_dtype not in _DT:
        raise ValueError("out_dtype must be float32, float16 or bfloat16")
    _check("nm_spmm", lib().nm_spmm(_ptr(values), _ptr(meta), R, K, n, m, _layout(layout),
                                    _ptr(X), T, dt, _ptr(out), _DT[y_dtype], _stream(X)))
    return out


def _same_dense(t: torch.Tensor, like: torch.Tensor, name: str) -> None:
    if t.shape != like.shape or t.dtype != like.dtype or t.device != like.device:
        raise ValueError(f"{name} must match W's shape, dtype and device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")


def prune(W: torch.Tensor, n: int = 2, m: int = 4, out: torch.Tensor | None = None) -> torch.Tensor:
    """SR-STE forward weight: W where the N:M mask keeps it, +0 elsewhere (out may be W)."""
    dt = _dense_input(W, "W", int8=False)
    R, K = W.shape
    if out is None:
        out = torch.empty_like(W)
    else:
        _same_dense(out, W, "out")
    _check("nm_prune", lib().nm_prune(_ptr(W), dt, R, K, n, m, _ptr(out), _stream(W)))
    return out


def srste_grad(W: torch.Tensor, G: torch.Tensor, n: int = 2, m: int = 4,
               decay: float = SRSTE_DECAY, out: torch.Tensor | None = None) -> torch.Tensor:
    """SR-STE backward: G where W is kept, G + decay*W where pruned (out may be G)."""
    dt = _dense_input(W, "W", int8=False)
    _same_dense(G, W, "G")
    R, K = W.shape
    if out is None:
        out = torch.empty_like(G)
    else:
        _same_dense(out, W, "out")
    _check("nm_srste_grad", lib().nm_srste_grad(_ptr(W), _ptr(G), dt, R, K, n, m, float(decay),
                                                _ptr(out), _stream(W)))
    return out


def tmask(W: torch.Tensor, n: int = 2, m: int = 4) -> torch.Tensor:
    """Bool (R, K): the transposable N:M mask (greedy, per m x m block)."""
    dt = _dense_input(W, "W", int8=False)
    R, K = W.shape
    out = torch.empty((R, K), dtype=torch.bool, device=W.device)
    _check("nm_tmask", lib().nm_tmask(_ptr(W), dt, R, K, n, m, _ptr(out), _stream(W)))
    return out


def tprune(W: torch.Tensor, n: int = 2, m: int = 4, out: torch.Tensor | None = None) -> torch.Tensor:
    """W where the transposable mask keeps it, +0 elsewhere (out may be W)."""
    dt = _dense_input(W, "W", int8=False)
    R, K = W.shape
    if out is None:
        out = torch.empty_like(W)
    else:
        _same_dense(out, W, "out")
    _check("nm_tprune", lib().nm_tprune(_ptr(W), dt, R, K, n, m, _ptr(out), _stream(W)))
    return out


def compress_t(W: torch.Tensor, n: int = 2, m: int = 4, layout: str = "rows"):
    """compress() of W's transpose (a K x R matrix, groups along R) without forming it."""
    dt = _dense_input(W, "W", int8=False)
    R, K = W.shape
    lay = _layout(layout)
    if R % m:
        _check("nm_compress_t", 2)
    vshape, mshape = compressed_shapes(K, R, n, m, layout)
    values = torch.empty(vshape, dtype=W.dtype, device=W.device)
    meta = torch.empty(mshape, dtype=torch.int32, device=W.device)
    _check("nm_compress_t", lib().nm_compress_t(_ptr(W), dt, R, K, n, m, lay, _ptr(values),
                                                _ptr(meta), _stream(W)))
    return values, meta


def _perm_workspace(W: torch.Tensor, n: int, m: int) -> torch.Tensor:
    R, K = W.shape
    nbytes = int(lib().nm_perm_workspace_bytes(R, K, n, m))
    if nbytes == 0 and R * K > 0:
        _check("nm_perm_workspace_bytes", 2)
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=W.device)


def perm_gains(W: torch.Tensor, perm: torch.Tensor, n: int = 2, m: int = 4):
    """(gain float32 (G, G), pick int32 (G, G)) of the best swap for every pair of column
    groups g1 < g2 under the permutation perm (int32 (K,) on W's device); other entries 0."""
    dt = _dense_input(W, "W")
    R, K = W.shape
    G = K // m
    if perm.dtype != torch.int32 or perm.shape != (K,) or perm.device != W.device:
        raise ValueError("perm must be an int32 (K,) tensor on W's device")
    gain = torch.zeros((G, G), dtype=torch.float32, device=W.device)
    pick = torch.zeros((G, G), dtype=torch.int32, device=W.device)
    ws = _perm_workspace(W, n, m)
    _check("nm_perm_gains", lib().nm_perm_gains(_ptr(W), dt, R, K, n, m, _ptr(perm.contiguous()),
                                                _ptr(gain), _ptr(pick), _ptr(ws), ws.numel(),
                                                _stream(W)))
    return gain, pick


def perm_gains_static(W: torch.Tensor, perm: torch.Tensor, n: int = 2, m: int = 4):
    """perm_gains through nm_perm_gains_static: the library's fixed device scratch buffer
    stands in for the workspace (R*K <= 16,777,216), so the C call allocates nothing; the
    result tensors are allocated here, before the call."""
    dt = _dense_input(W, "W")
    R, K = W.shape
    G = K // m
    if perm.dtype != torch.int32 or perm.shape != (K,) or perm.device != W.device:
        raise ValueError("perm must be an int32 (K,) tensor on W's device")
    gain = torch.zeros((G, G), dtype=torch.float32, device=W.device)
    pick = torch.zeros((G, G), dtype=torch.int32, device=W.device)
    _check("nm_perm_gains_static", lib().nm_perm_gains_static(
        _ptr(W), dt, R, K, n, m, _ptr(perm.contiguous()), _ptr(gain), _ptr(pick), _stream(W)))
    return gain, pick


def perm_search(W: torch.Tensor, n: int = 2, m: int = 4, max_rounds: int = 1000, perm=None):
    """(perm, rounds): a column permutation (CPU int32 (K,)) whose N:M mask keeps at least
    the kept magnitude of the start (identity by default), by rounds of group swaps."""
    import numpy as np

    dt = _dense_input(W, "W")
    R, K = W.shape
    p = np.arange(K, dtype=np.int32) if perm is None else np.array(perm, dtype=np.int32)
    if p.shape != (K,):
        raise ValueError("perm must have K entries")
    rounds = ctypes.c_int(0)
    ws = _perm_workspace(W, n, m)
    _check("nm_perm_search", lib().nm_perm_search(
        _ptr(W), dt, R, K, n, m, int(max_rounds), p.ctypes.data_as(ctypes.c_void_p),
        ctypes.byref(rounds), _ptr(ws), ws.numel(), _stream(W)))
    return torch.from_numpy(p), rounds.value
