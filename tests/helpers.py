"""Small helpers shared by the tests (no method arithmetic lives here)."""
from __future__ import annotations

import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def encode(values, dtype: str) -> np.ndarray:
    """Python floats -> the raw storage the libraries take (float32 or uint16 bits)."""
    v = np.asarray(values, dtype=np.float64)
    if dtype == "f32":
        return v.astype(np.float32)
    return synth.round_to(v, dtype)


def as_bits(a: np.ndarray) -> np.ndarray:
    """Raw bit patterns of a float32 / uint16 array."""
    if a.dtype in (np.uint16, np.uint32):
        return a
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def read_hand_groups():
    rows = []
    with open(os.path.join(GOLDEN, "hand_groups.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, vals, kept, meta, why = [p.strip() for p in line.split("|")]
            dt, n, m = head.split()
            values = [float(x) for x in vals.split()]
            # keep the sign of "-0"
            values = [(-0.0 if tok == "-0" else v) for tok, v in zip(vals.split(), values)]
            rows.append(dict(dtype=dt, n=int(n), m=int(m), values=values,
                             kept=[int(x) for x in kept.split()], meta=int(meta, 16), why=why))
    return rows


def read_kv(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                out[k] = float(v)
    return out


def normwise_rel_err(y: np.ndarray, y_ref: np.ndarray) -> float:
    """max |y - y_ref| / max |y_ref| (infinity-norm relative error)."""
    den = float(np.max(np.abs(y_ref))) if y_ref.size else 0.0
    num = float(np.max(np.abs(y.astype(np.float64) - y_ref))) if y_ref.size else 0.0
    return num / den if den > 0 else num


# ---------------------------------------------------------------------------
# NM_LAYOUT_BLOCKED (include/nm.h): the ROWS arrays regrouped into blocks of
# 16 rows x one 64-wide K step.  A storage permutation, no arithmetic.
# ---------------------------------------------------------------------------
META_BITS = {2: 1, 4: 2, 8: 3}


def blocked_dims(R: int, K: int, n: int, m: int):
    """(G, S, V, B): row groups, K steps, values and metadata bytes per row and step."""
    V = 64 // m * n
    return -(-R // 16), K // 64, V, V * META_BITS[m] // 8


def meta_row_bytes(meta_words: np.ndarray) -> np.ndarray:
    """(R, words) uint32 -> (R, 4 * words) uint8; byte i of a row holds bits 8i .. 8i+7."""
    w = np.ascontiguousarray(meta_words).astype("<u4")
    return w.view(np.uint8).reshape(w.shape[0], -1)


def blocked_from_rows(values: np.ndarray, meta_words: np.ndarray, R: int, K: int, n: int, m: int):
    """ROWS (values (R, K*n/m), meta (R, words) uint32) -> BLOCKED (values (G, S, 16, V),
    meta (G, S, 4*B) uint32); padding rows are zeros."""
    G, S, V, B = blocked_dims(R, K, n, m)
    vpad = np.zeros((G * 16, S * V), dtype=values.dtype)
    vpad[:R] = values.reshape(R, S * V)
    vb = vpad.reshape(G, 16, S, V).transpose(0, 2, 1, 3)
    mpad = np.zeros((G * 16, S * B), dtype=np.uint8)
    mpad[:R] = meta_row_bytes(meta_words)[:, :S * B]
    mb = mpad.reshape(G, 16, S, B).transpose(0, 2, 1, 3).reshape(G, S, 16 * B)
    return (np.ascontiguousarray(vb),
            np.ascontiguousarray(mb).view("<u4").astype(np.uint32).reshape(G, S, 4 * B))


def rows_from_blocked(vb: np.ndarray, mb: np.ndarray, R: int, K: int, n: int, m: int):
    """Inverse of blocked_from_rows (ROWS metadata rows padded with zero bits)."""
    G, S, V, B = blocked_dims(R, K, n, m)
    values = vb.reshape(G, S, 16, V).transpose(0, 2, 1, 3).reshape(G * 16, S * V)[:R]
    mbytes = np.ascontiguousarray(mb.astype("<u4")).view(np.uint8).reshape(G, S, 16, B)
    mbytes = mbytes.transpose(0, 2, 1, 3).reshape(G * 16, S * B)[:R]
    words = -(-(S * B) // 4)
    out = np.zeros((R, 4 * words), dtype=np.uint8)
    out[:, :S * B] = mbytes
    return np.ascontiguousarray(values), out.view("<u4").astype(np.uint32).reshape(R, words)
