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
