"""CPU oracle for N:M masking, compression and sparse x dense products.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The GPU
library never loads it and shares no code with it.

The arithmetic lives in ``nm_oracle.c`` (plain C99, compiled with gcc); this
module only builds that file and marshals numpy arrays into it.  Functions
follow the definitions cited in ``nm_oracle.h``:

* ``mask`` / ``compress``: ASP's exhaustive best-pattern search
  ("量化友好的SR-STE稀疏化训练", section "NVIDA Apex内的静态掩码稀疏"), exact
  scores, first (lexicographically smallest) best pattern on ties.
* ``compress`` / ``decompress``: value array plus b-bit position fields
  ("[리뷰] Accelerating Sparse Deep Neural Networks", section
  "2:4 Sparsity의 benefits").
* ``spmm``: dense product of the decompressed operand with X in double
  (same review, section "Tensor Scores 상에서 구조적인 sparse GEMM").
* ``prune`` / ``srste_grad``: SR-STE's masked forward weight and its backward
  gradient ("量化友好的SR-STE稀疏化训练", section
  "基于直通估计的动态掩码精炼化稀疏(SR-STE)"), the gradient in the printed
  backward's fp32 order; ``round_from_f32`` is its final rounding to the
  element type, exposed for the pins.
* ``tmask_greedy`` / ``tmask_optimal`` / ``tprune``: transposable N:M masks per
  M x M block ("[论文解读] Accelerated Sparse Neural Training: ... N:M
  Transposable Masks", ABSTRACT and "提出的方法"): the greedy 2-approximation
  the GPU runs, the minimum-cost-flow optimum as a reference, and the forward
  weight under the greedy mask.  ``compress_t`` is compress of the transpose.
* ``kept_l1`` / ``perm_gains`` / ``perm_search``: channel permutation before
  masking ("[리뷰] Accelerating Sparse Deep Neural Networks", "Step-2: Weight
  Pruning", Fig. 6), the kept magnitude of a column permutation and a
  pairwise-swap search for a better one.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nm_oracle.c")
_LIB = os.path.join(_HERE, "libnm_oracle.so")

F32, F16, BF16, I8, FP8 = 0, 1, 2, 3, 4
_DT_CODE = {"f32": F32, "f16": F16, "bf16": BF16, "i8": I8, "fp8": FP8}
_ELEM = {F32: np.uint32, F16: np.uint16, BF16: np.uint16, I8: np.uint8, FP8: np.uint8}


def build(force: bool = True) -> str:
    """Compile nm_oracle.c into libnm_oracle.so with gcc."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-Wall", "-Wextra", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """The loaded oracle library: libnm_oracle.so, built here when stale, or the build named
    by NM_ORACLE_LIB (the sanitizer test's instrumented build of the same source)."""
    global _lib
    if _lib is None:
        path = os.environ.get("NM_ORACLE_LIB")
        if not path:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            path = _LIB
        L = ctypes.CDLL(path)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.nmo_meta_bits.argtypes = [i32]
        L.nmo_meta_bits.restype = i32
        L.nmo_meta_words_per_row.argtypes = [i64, i32, i32]
        L.nmo_meta_words_per_row.restype = i64
        L.nmo_mask.argtypes = [vp, i32, i64, i64, i32, i32, vp]
        L.nmo_compress.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp]
        L.nmo_decompress.argtypes = [vp, vp, i32, i64, i64, i32, i32, vp]
        L.nmo_spmm.argtypes = [vp, vp, i64, i64, i32, i32, vp, i64, i32, vp]
        L.nmo_spmm_rows.argtypes = [vp, vp, i64, i64, i32, i32, vp, i64, i32, i64, i64, vp]
        L.nmo_spmm_sample.argtypes = [vp, vp, i64, i64, i32, i32, vp, i64, i32, vp, vp, i64, vp]
        L.nmo_prune.argtypes = [vp, i32, i64, i64, i32, i32, vp]
        L.nmo_srste_grad.argtypes = [vp, vp, i32, i64, i64, i32, i32, ctypes.c_float, vp]
        L.nmo_round_from_f32.argtypes = [vp, i32, i64, vp]
        L.nmo_tmask_greedy.argtypes = [vp, i32, i64, i64, i32, i32, vp]
        L.nmo_tmask_optimal.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp]
        L.nmo_tprune.argtypes = [vp, i32, i64, i64, i32, i32, vp]
        L.nmo_kept_l1.argtypes = [vp, i32, i64, i64, i32, i32, vp]
        L.nmo_kept_l1.restype = ctypes.c_double
        L.nmo_perm_gains.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp]
        L.nmo_perm_search.argtypes = [vp, i32, i64, i64, i32, i32, i32, vp, vp]
        L.nmo_to_double.argtypes = [vp, i32, i64]
        L.nmo_to_double.restype = ctypes.c_double
        for f in ("nmo_mask", "nmo_compress", "nmo_decompress", "nmo_spmm", "nmo_spmm_rows",
                  "nmo_spmm_sample", "nmo_prune", "nmo_srste_grad", "nmo_round_from_f32",
                  "nmo_tmask_greedy", "nmo_tmask_optimal", "nmo_tprune", "nmo_perm_gains",
                  "nmo_perm_search"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def _code(dt) -> int:
    return _DT_CODE[dt] if isinstance(dt, str) else int(dt)


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def meta_bits(m: int) -> int:
    return lib().nmo_meta_bits(m)


def meta_words_per_row(K: int, n: int, m: int) -> int:
    return lib().nmo_meta_words_per_row(K, n, m)


def _as_bits(W: np.ndarray, dt: int) -> np.ndarray:
    want = _ELEM[dt]
    if W.dtype != want:
        W = W.view(want)
    return np.ascontiguousarray(W)


def mask(W: np.ndarray, dt, n: int, m: int) -> np.ndarray:
    """uint8 R x K: 1 where the weight is kept."""
    dt = _code(dt)
    W = _as_bits(W, dt)
    R, K = W.shape
    out = np.empty((R, K), dtype=np.uint8)
    _check(lib().nmo_mask(_ptr(W), dt, R, K, n, m, _ptr(out)), "mask")
    return out


def compress(W: np.ndarray, dt, n: int, m: int):
    """(values R x K*n/m as raw bits, meta R x words_per_row uint32)."""
    dt = _code(dt)
    W = _as_bits(W, dt)
    R, K = W.shape
    if K % m:
        raise ValueError("K must be a multiple of m")
    vals = np.empty((R, K // m * n), dtype=_ELEM[dt])
    wpr = meta_words_per_row(K, n, m)
    meta = np.empty((R, max(wpr, 0)), dtype=np.uint32)
    _check(lib().nmo_compress(_ptr(W), dt, R, K, n, m, _ptr(vals), _ptr(meta)), "compress")
    return vals, meta


def decompress(values: np.ndarray, meta: np.ndarray, dt, R: int, K: int, n: int, m: int) -> np.ndarray:
    dt = _code(dt)
    values = _as_bits(values, dt)
    meta = np.ascontiguousarray(meta, dtype=np.uint32)
    out = np.empty((R, K), dtype=_ELEM[dt])
    _check(lib().nmo_decompress(_ptr(values), _ptr(meta), dt, R, K, n, m, _ptr(out)), "decompress")
    return out


def spmm(values, meta, R: int, K: int, n: int, m: int, X: np.ndarray, dt) -> np.ndarray:
    """Y (R x T, float64) = decompress(values, meta) @ X."""
    dt = _code(dt)
    values = _as_bits(values, dt)
    meta = np.ascontiguousarray(meta, dtype=np.uint32)
    X = _as_bits(X, dt)
    T = X.shape[1]
    Y = np.empty((R, T), dtype=np.float64)
    _check(lib().nmo_spmm(_ptr(values), _ptr(meta), R, K, n, m, _ptr(X), T, dt, _ptr(Y)), "spmm")
    return Y


def spmm_rows(values, meta, R, K, n, m, X, dt, r0: int, r1: int, Y: np.ndarray) -> None:
    """Fill rows [r0, r1) of the R x T float64 array Y (other rows untouched)."""
    dt = _code(dt)
    assert Y.dtype == np.float64 and Y.flags["C_CONTIGUOUS"]
    rc = lib().nmo_spmm_rows(_ptr(values), _ptr(meta), R, K, n, m, _ptr(X), X.shape[1], dt, r0, r1,
                             _ptr(Y))
    _check(rc, "spmm_rows")


def spmm_sample(values, meta, R, K, n, m, X, dt, rs, ts) -> np.ndarray:
    """Y[rs[i], ts[i]] of the product, one exact dot product per sample."""
    dt = _code(dt)
    values = _as_bits(values, dt)
    meta = np.ascontiguousarray(meta, dtype=np.uint32)
    X = _as_bits(X, dt)
    rs = np.ascontiguousarray(rs, dtype=np.int64)
    ts = np.ascontiguousarray(ts, dtype=np.int64)
    out = np.empty(len(rs), dtype=np.float64)
    rc = lib().nmo_spmm_sample(_ptr(values), _ptr(meta), R, K, n, m, _ptr(X), X.shape[1], dt,
                               _ptr(rs), _ptr(ts), len(rs), _ptr(out))
    _check(rc, "spmm_sample")
    return out


def prune(W: np.ndarray, dt, n: int, m: int) -> np.ndarray:
    """SR-STE forward weight (raw bits): W where kept, +0 where pruned."""
    dt = _code(dt)
    W = _as_bits(W, dt)
    R, K = W.shape
    out = np.empty((R, K), dtype=_ELEM[dt])
    _check(lib().nmo_prune(_ptr(W), dt, R, K, n, m, _ptr(out)), "prune")
    return out


def srste_grad(W: np.ndarray, G: np.ndarray, dt, n: int, m: int, decay: float) -> np.ndarray:
    """SR-STE backward gradient (raw bits): G where W is kept, else G + decay * W
    in fp32 (product, then sum), rounded to the element type."""
    dt = _code(dt)
    W = _as_bits(W, dt)
    G = _as_bits(G, dt)
    if W.shape != G.shape:
        raise ValueError("W and G must have the same shape")
    R, K = W.shape
    out = np.empty((R, K), dtype=_ELEM[dt])
    _check(lib().nmo_srste_grad(_ptr(W), _ptr(G), dt, R, K, n, m, float(decay), _ptr(out)),
           "srste_grad")
    return out


def round_from_f32(x: np.ndarray, dt) -> np.ndarray:
    """Raw bits of every float32 of x rounded to dt (nearest, ties to even)."""
    dt = _code(dt)
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape[0], dtype=_ELEM[dt])
    _check(lib().nmo_round_from_f32(_ptr(flat), dt, flat.shape[0], _ptr(out)), "round_from_f32")
    return out.reshape(x.shape)


def tmask_greedy(W: np.ndarray, dt, n: int, m: int) -> np.ndarray:
    """uint8 R x K transposable mask by the greedy (1 = kept)."""
    dt = _code(dt)
    W = _as_bits(W, dt)
    R, K = W.shape
    out = np.empty((R, K), dtype=np.uint8)
    _check(lib().nmo_tmask_greedy(_ptr(W), dt, R, K, n, m, _ptr(out)), "tmask_greedy")
    return out


def tmask_optimal(W: np.ndarray, dt, n: int, m: int):
    """(uint8 R x K optimal transposable mask, its kept L1 norm)."""
    dt = _code(dt)
    W = _as_bits(W, dt)
    R, K = W.shape
    out = np.empty((R, K), dtype=np.uint8)
    l1 = ctypes.c_double(0.0)
    _check(lib().nmo_tmask_optimal(_ptr(W), dt, R, K, n, m, _ptr(out), ctypes.byref(l1)),
           "tmask_optimal")
    return out, l1.value


def tprune(W: np.ndarray, dt, n: int, m: int) -> np.ndarray:
    """Raw bits: W where the greedy transposable mask keeps it, +0 elsewhere."""
    dt = _code(dt)
    W = _as_bits(W, dt)
    R, K = W.shape
    out = np.empty((R, K), dtype=_ELEM[dt])
    _check(lib().nmo_tprune(_ptr(W), dt, R, K, n, m, _ptr(out)), "tprune")
    return out


def compress_t(W: np.ndarray, dt, n: int, m: int):
    """compress of the transpose: (values K x R*n/m, meta K x words) of W.T."""
    dt = _code(dt)
    return compress(np.ascontiguousarray(_as_bits(W, dt).T), dt, n, m)


def _perm(perm, K):
    p = np.arange(K, dtype=np.int32) if perm is None else np.ascontiguousarray(perm, dtype=np.int32)
    if p.shape != (K,):
        raise ValueError("perm must have K entries")
    return p


def kept_l1(W: np.ndarray, dt, n: int, m: int, perm=None) -> float:
    """Kept L1 of the N:M mask of W[:, perm] (perm None = identity)."""
    dt = _code(dt)
    W = _as_bits(W, dt)
    R, K = W.shape
    p = _perm(perm, K)
    v = lib().nmo_kept_l1(_ptr(W), dt, R, K, n, m, _ptr(p))
    if v < 0:
        raise ValueError("oracle kept_l1 rejected its arguments")
    return v


def perm_gains(W: np.ndarray, dt, n: int, m: int, perm=None):
    """(gain, pick) tables (G x G, upper triangle filled) of the best swap per group pair."""
    dt = _code(dt)
    W = _as_bits(W, dt)
    R, K = W.shape
    G = K // m
    p = _perm(perm, K)
    gain = np.zeros((G, G), dtype=np.float64)
    pick = np.zeros((G, G), dtype=np.int32)
    _check(lib().nmo_perm_gains(_ptr(W), dt, R, K, n, m, _ptr(p), _ptr(gain), _ptr(pick)),
           "perm_gains")
    return gain, pick


def perm_search(W: np.ndarray, dt, n: int, m: int, max_rounds: int = 1000, perm=None):
    """(perm, rounds applied) after the swap search, starting from perm (None = identity)."""
    dt = _code(dt)
    W = _as_bits(W, dt)
    R, K = W.shape
    p = _perm(perm, K).copy()
    done = ctypes.c_int(0)
    _check(lib().nmo_perm_search(_ptr(W), dt, R, K, n, m, max_rounds, _ptr(p), ctypes.byref(done)),
           "perm_search")
    return p, done.value


def to_double(a: np.ndarray, dt) -> np.ndarray:
    """Exact float64 value of every element (raw bits in, doubles out)."""
    dt = _code(dt)
    a = _as_bits(a, dt)
    flat = a.reshape(-1)
    L = lib()
    out = np.empty(flat.shape[0], dtype=np.float64)
    p = _ptr(flat)
    for i in range(flat.shape[0]):
        out[i] = L.nmo_to_double(p, dt, i)
    return out.reshape(a.shape)
