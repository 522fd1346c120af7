"""Host-side metadata check (nm_check_meta): metadata the oracle writes is well formed in
both layouts, and planted faults are found at the right group.

A group is well formed when its n positions are strictly ascending; a row of the row
layout must also leave its padding bits zero.  Faults are planted by rewriting single
b-bit fields of the oracle's metadata (field f = g*n + j of a row at bit f*b of the row's
bitstream, least significant bit first), then regrouped for the blocked layout with the
same regrouping the layout tests pin.
"""
import os

import numpy as np
import pytest
import torch

import masking_sparse_gemm_amd as nm
import oracle
from tests.helpers import blocked_from_rows

needs_lib = pytest.mark.skipif(not os.path.exists(nm.LIB_PATH), reason="libnm.so not built")

PATTERNS = [(1, 2), (2, 2), (1, 4), (2, 4), (3, 4), (4, 4), (1, 8), (2, 8), (3, 8), (4, 8),
            (6, 8), (8, 8)]


def bits_of(m):
    return {2: 1, 4: 2, 8: 3}[m]


def valid_meta(R, K, n, m, seed):
    rng = np.random.default_rng(seed)
    W = np.round(rng.standard_normal((R, K)) * 3).astype(np.float32)  # many ties
    _, meta = oracle.compress(W, "f32", n, m)
    return meta.copy()


def set_field(meta, r, f, b, v):
    """Write value v into field f (b bits) of row r of row-layout metadata."""
    row = meta[r]
    for k in range(b):
        bit = f * b + k
        w, s = divmod(bit, 32)
        if (v >> k) & 1:
            row[w] |= np.uint32(1 << s)
        else:
            row[w] &= np.uint32(~(1 << s) & 0xFFFFFFFF)


def get_field(meta, r, f, b):
    v = 0
    for k in range(b):
        w, s = divmod(f * b + k, 32)
        v |= ((int(meta[r][w]) >> s) & 1) << k
    return v


def check(meta, R, K, n, m, layout="rows"):
    return nm.check_meta(torch.from_numpy(np.ascontiguousarray(meta).view(np.int32)), R, K, n, m,
                         layout)


def check_both_layouts(meta, R, K, n, m):
    got = check(meta, R, K, n, m)
    if K % 64 == 0:
        vals = np.zeros((R, K // m * n), dtype=np.uint32)
        _, mb = blocked_from_rows(vals, meta, R, K, n, m)
        assert check(mb, R, K, n, m, "blocked") == got
    return got


@needs_lib
@pytest.mark.parametrize("n,m", PATTERNS)
def test_oracle_metadata_is_well_formed(n, m):
    for R, K in [(5, 96), (20, 128), (1, 8 * m), (17, 64)]:
        if K % m:
            continue
        assert check_both_layouts(valid_meta(R, K, n, m, R + K), R, K, n, m) == -1


@needs_lib
@pytest.mark.parametrize("n,m", [p for p in PATTERNS if p[0] >= 2])
def test_a_repeated_or_descending_position_is_found(n, m):
    R, K = 20, 128
    G, b = K // m, bits_of(m)
    rng = np.random.default_rng(n * 10 + m)
    for _ in range(6):
        meta = valid_meta(R, K, n, m, 7)
        r, g, j = int(rng.integers(R)), int(rng.integers(G)), int(rng.integers(n - 1))
        f = g * n + j
        a, c = get_field(meta, r, f, b), get_field(meta, r, f + 1, b)
        if rng.random() < 0.5:
            set_field(meta, r, f, b, c)  # repeat
        else:
            set_field(meta, r, f, b, c)  # swap: descending
            set_field(meta, r, f + 1, b, a)
        assert check_both_layouts(meta, R, K, n, m) == r * G + g


@needs_lib
def test_the_first_fault_in_row_major_order_is_reported():
    R, K, n, m = 8, 64, 2, 4
    G = K // m
    meta = valid_meta(R, K, n, m, 3)
    for r, g in [(6, 1), (3, 9), (3, 2)]:
        set_field(meta, r, g * n, 2, get_field(meta, r, g * n + 1, 2))
    assert check_both_layouts(meta, R, K, n, m) == 3 * G + 2


@needs_lib
def test_padding_bits_of_a_row_must_be_zero():
    R, K, n, m = 4, 24, 3, 8  # 3 groups x 3 fields x 3 bits = 27 bits: 5 padding bits
    G = K // m
    meta = valid_meta(R, K, n, m, 5)
    assert check(meta, R, K, n, m) == -1
    meta[2, 0] |= np.uint32(1 << 30)
    assert check(meta, R, K, n, m) == 2 * G + G - 1


@needs_lib
def test_single_position_groups_and_edge_arguments():
    R, K = 6, 64
    meta = valid_meta(R, K, 1, 4, 9)
    # any single position is well formed
    set_field(meta, 4, 5, 2, 3)
    assert check(meta, R, K, 1, 4) == -1
    assert nm.check_meta(torch.zeros(0, dtype=torch.int32), 0, 64, 2, 4) == -1
    with pytest.raises(ValueError):
        nm.check_meta(torch.zeros(16, dtype=torch.int32), 4, 66, 2, 4)  # K % m != 0
    with pytest.raises(ValueError):
        nm.check_meta(torch.zeros(64, dtype=torch.int32), 4, 96, 2, 4, "blocked")  # K % 64
    with pytest.raises(ValueError):
        nm.check_meta(torch.zeros(1, dtype=torch.int32), 4, 64, 2, 4)  # too short
