"""The test-side reference of NM_LAYOUT_BLOCKED (tests/helpers.py) against the
definition in include/nm.h, element by element, before GPU tests rely on it."""
import numpy as np
import pytest

import oracle
from tests.helpers import blocked_dims, blocked_from_rows, meta_row_bytes, rows_from_blocked

CASES = [(17, 128, 2, 4), (16, 64, 1, 2), (33, 192, 4, 8), (5, 256, 3, 8), (40, 64, 1, 8),
         (1, 128, 7, 8), (31, 64, 3, 4), (48, 128, 2, 2)]


def random_rows(rng, R, K, n, m):
    V = K // m * n
    words = -(-(K // m * n * {2: 1, 4: 2, 8: 3}[m]) // 32)
    values = rng.integers(0, 1 << 16, (R, V), dtype=np.uint16)
    meta = rng.integers(0, 1 << 32, (R, words), dtype=np.uint64).astype(np.uint32)
    used = K // m * n * {2: 1, 4: 2, 8: 3}[m]
    if used % 32:  # unused high bits of a row's last word are zero
        meta[:, -1] &= np.uint32((1 << (used % 32)) - 1)
    return values, meta


@pytest.mark.parametrize("R,K,n,m", CASES)
def test_blocked_matches_the_definition_elementwise(R, K, n, m):
    """Every value and metadata byte sits where the header's formulas put it."""
    rng = np.random.default_rng(R * 1000 + K + n * 10 + m)
    values, meta = random_rows(rng, R, K, n, m)
    vb, mb = blocked_from_rows(values, meta, R, K, n, m)
    G, S, V, B = blocked_dims(R, K, n, m)
    flat_v = vb.reshape(-1)
    flat_m = np.ascontiguousarray(mb.astype("<u4")).view(np.uint8).reshape(-1)
    row_bytes = meta_row_bytes(meta)
    assert flat_v.size == G * 16 * (K // m * n) and flat_m.size == G * 16 * S * B
    for g in range(G):
        for s in range(S):
            for r in range(16):
                row = 16 * g + r
                for j in range(V):
                    want = values[row, s * V + j] if row < R else 0
                    assert flat_v[((g * S + s) * 16 + r) * V + j] == want
                for i in range(B):
                    want = row_bytes[row, s * B + i] if row < R else 0
                    assert flat_m[((g * S + s) * 16 + r) * B + i] == want


@pytest.mark.parametrize("R,K,n,m", CASES)
def test_blocked_round_trip(R, K, n, m):
    rng = np.random.default_rng(7 * R + K)
    values, meta = random_rows(rng, R, K, n, m)
    v2, m2 = rows_from_blocked(*blocked_from_rows(values, meta, R, K, n, m), R, K, n, m)
    assert np.array_equal(v2, values) and np.array_equal(m2, meta)


@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (4, 8), (3, 8), (1, 8)])
def test_blocked_step_slices_hold_whole_fields(n, m):
    """Field j of step s, read from the block's byte slice at bit j*b, is field s*V + j of
    the oracle's row bitstream: a step's slice starts on a field boundary."""
    rng = np.random.default_rng(3)
    R, K = 20, 192
    W = rng.standard_normal((R, K)).astype(np.float32)
    vals, meta = oracle.compress(W, "f32", n, m)
    vb, mb = blocked_from_rows(vals.view(np.uint32), meta, R, K, n, m)
    G, S, V, B = blocked_dims(R, K, n, m)
    b = {2: 1, 4: 2, 8: 3}[m]
    mbytes = np.ascontiguousarray(mb.astype("<u4")).view(np.uint8).reshape(G, S, 16, B)
    rbytes = meta_row_bytes(meta)
    for row in range(R):
        stream = int.from_bytes(rbytes[row].tobytes(), "little")
        for s in range(S):
            chunk = int.from_bytes(mbytes[row // 16, s, row % 16].tobytes(), "little")
            for j in range(V):
                f = s * V + j
                assert (chunk >> (j * b)) & ((1 << b) - 1) == (stream >> (f * b)) & ((1 << b) - 1)
