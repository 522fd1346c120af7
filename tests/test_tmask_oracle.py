"""Pins for the oracle's transposable N:M masks, each computed here without the
oracle's code path.

Source: "[论文解读] Accelerated Sparse Neural Training: A Provable and Efficient
Method to Find N:M Transposable Masks", ABSTRACT and section "提出的方法": a mask
per M x M block with N kept per row and per column, so that W and its transpose
are both N:M; the optimum (maximal kept L1) is a minimum-cost flow, the fast method
a greedy 2-approximation.

Pins: hand-worked blocks (tests/golden/tmask_hand.txt); the greedy's output is a
valid, maximal b-matching within half of the optimum; it equals the ordinary
row-wise mask whenever that mask already fits the column caps; it commutes with
transposition for distinct magnitudes; the optimum's kept L1 equals brute force
(4 x 4) and scipy's linear programme (8 x 8, whose polytope is integral).
"""
import os
from itertools import product

import numpy as np
import pytest
from scipy.optimize import linprog

import oracle
import synth
from tests.helpers import GOLDEN, as_bits, encode

DTS = ["f32", "f16", "bf16"]
PATTERNS = [(2, 4), (1, 4), (3, 4), (1, 2), (4, 8), (2, 8), (1, 8)]


def read_tmask_hand():
    rows = []
    with open(os.path.join(GOLDEN, "tmask_hand.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, block, want, why = [p.strip() for p in line.split("|")]
            dt, n, m = head.split()
            vals = [[float(x) for x in r.split()] for r in block.split(";")]
            mask = [[int(ch) for ch in r.strip()] for r in want.split(";")]
            rows.append(dict(dtype=dt, n=int(n), m=int(m), block=vals, mask=mask, why=why))
    return rows


def magnitudes(W, dt):
    return np.abs(synth.bits_to_f64(as_bits(W), dt))


def blocks(a: np.ndarray, m: int):
    R, K = a.shape
    return a.reshape(R // m, m, K // m, m).transpose(0, 2, 1, 3).reshape(-1, m, m)


def random_w(R, K, dt, seed, ties=False):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((R, K)) * np.exp2(rng.integers(-6, 7, size=(R, K)))
    if ties:
        a = np.round(a * 2) / 2
    return encode(a, dt)


@pytest.mark.parametrize("case", read_tmask_hand(), ids=lambda c: c["why"][:40])
def test_hand_worked_blocks(case):
    W = encode(np.array(case["block"]), case["dtype"])
    got = oracle.tmask_greedy(W, case["dtype"], case["n"], case["m"])
    assert got.tolist() == case["mask"], case["why"]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("n,m", PATTERNS)
@pytest.mark.parametrize("ties", [False, True])
def test_greedy_is_a_valid_maximal_b_matching(dt, n, m, ties):
    W = random_w(4 * m, 6 * m, dt, seed=n * 10 + m, ties=ties)
    keep = blocks(oracle.tmask_greedy(W, dt, n, m).astype(int), m)
    rows, cols = keep.sum(axis=2), keep.sum(axis=1)
    assert rows.max() <= n and cols.max() <= n
    # maximal: every refused entry meets a full row or a full column
    refused = keep == 0
    full = (rows[:, :, None] == n) | (cols[:, None, :] == n)
    assert np.all(full[refused])


def brute_force_optimum(block_abs: np.ndarray, n: int) -> float:
    """Largest kept L1 over every 0/1 4x4 mask with at most n per row and column."""
    m = block_abs.shape[0]
    bits = ((np.arange(1 << (m * m))[:, None] >> np.arange(m * m)) & 1).reshape(-1, m, m)
    ok = (bits.sum(axis=2) <= n).all(axis=1) & (bits.sum(axis=1) <= n).all(axis=1)
    return float((bits[ok] * block_abs).sum(axis=(1, 2)).max())


def lp_optimum(block_abs: np.ndarray, n: int) -> float:
    m = block_abs.shape[0]
    A = np.zeros((2 * m, m * m))
    for i in range(m):
        A[i, i * m:(i + 1) * m] = 1          # row i
        A[m + i, i::m] = 1                   # column i
    res = linprog(-block_abs.ravel(), A_ub=A, b_ub=np.full(2 * m, n), bounds=(0, 1),
                  method="highs")
    assert res.status == 0
    return -res.fun


@pytest.mark.parametrize("n", [1, 2, 3])
def test_optimum_matches_brute_force_4x4(n):
    W = random_w(8, 12, "f32", seed=40 + n, ties=True)
    mask, l1 = oracle.tmask_optimal(W, "f32", n, 4)
    a = magnitudes(W, "f32")
    want = sum(brute_force_optimum(b, n) for b in blocks(a, 4))
    assert l1 == pytest.approx(want, rel=1e-12)
    assert (mask * a).sum() == pytest.approx(want, rel=1e-12)
    kb = blocks(mask.astype(int), 4)
    assert kb.sum(axis=2).max() <= n and kb.sum(axis=1).max() <= n


@pytest.mark.parametrize("n", [1, 2, 4, 6])
def test_optimum_matches_linear_programme_8x8(n):
    W = random_w(16, 24, "f32", seed=50 + n)
    mask, l1 = oracle.tmask_optimal(W, "f32", n, 8)
    a = magnitudes(W, "f32")
    want = sum(lp_optimum(b, n) for b in blocks(a, 8))
    assert l1 == pytest.approx(want, rel=1e-9)
    kb = blocks(mask.astype(int), 8)
    assert kb.sum(axis=2).max() <= n and kb.sum(axis=1).max() <= n


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 4), (2, 8)])
def test_greedy_within_half_of_the_optimum(dt, n, m):
    W = random_w(8 * m, 8 * m, dt, seed=60 + n + m)
    a = magnitudes(W, dt)
    g = blocks(oracle.tmask_greedy(W, dt, n, m) * a, m).sum(axis=(1, 2))
    o = blocks(oracle.tmask_optimal(W, dt, n, m)[0] * a, m).sum(axis=(1, 2))
    assert np.all(g <= o * (1 + 1e-12)) and np.all(2 * g >= o * (1 - 1e-12))


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 4), (3, 8), (1, 2)])
def test_greedy_equals_row_mask_when_that_fits_the_columns(dt, n, m):
    """Rows whose N largest sit in cyclically shifted columns: every column holds N of
    them, so the ordinary (pinned) row mask is already transposable and the greedy
    must return it."""
    R, K = 3 * m, 5 * m
    rng = np.random.default_rng(70 + n + m)
    a = rng.uniform(0.0, 1.0, size=(R, K))
    for r in range(R):
        for c0 in range(0, K, m):
            for j in range(n):
                a[r, c0 + (r + j + c0 // m) % m] += 2.0
    a *= np.where(rng.random((R, K)) < 0.5, -1.0, 1.0)
    W = encode(a, dt)
    assert np.array_equal(oracle.tmask_greedy(W, dt, n, m), oracle.mask(W, dt, n, m))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 2)])
def test_greedy_commutes_with_transposition(dt, n, m):
    """With distinct magnitudes the order of entries does not depend on positions."""
    R, K = 4 * m, 4 * m
    perm = np.random.default_rng(80).permutation(R * K).reshape(R, K) + 1
    W = encode(perm * np.where(perm % 3 == 0, -1.0, 1.0), dt)
    WT = np.ascontiguousarray(W.T)
    assert np.array_equal(oracle.tmask_greedy(WT, dt, n, m), oracle.tmask_greedy(W, dt, n, m).T)


@pytest.mark.parametrize("dt", DTS)
def test_n_equals_m_keeps_everything(dt):
    W = random_w(8, 16, dt, seed=90, ties=True)
    assert oracle.tmask_greedy(W, dt, 4, 4).all() and oracle.tmask_greedy(W, dt, 8, 8).all()


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 2)])
def test_tprune_is_select_of_the_greedy_mask(dt, n, m):
    W = random_w(4 * m, 6 * m, dt, seed=100, ties=True)
    keep = oracle.tmask_greedy(W, dt, n, m).astype(bool)
    want = as_bits(W).copy()
    want[~keep] = 0
    assert np.array_equal(as_bits(oracle.tprune(W, dt, n, m)), want)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 2)])
def test_one_mask_serves_both_products(dt, n, m):
    """The pruned weight survives compression along rows and along columns: both
    compressed pairs decompress to it (the point of a transposable mask)."""
    R, K = 4 * m, 8 * m
    W = random_w(R, K, dt, seed=110)
    P = oracle.tprune(W, dt, n, m)
    v, mt = oracle.compress(P, dt, n, m)
    vt, mtt = oracle.compress_t(P, dt, n, m)
    rows = synth.bits_to_f64(oracle.decompress(v, mt, dt, R, K, n, m), dt)
    cols = synth.bits_to_f64(oracle.decompress(vt, mtt, dt, K, R, n, m), dt).T
    p = synth.bits_to_f64(P, dt)
    assert np.array_equal(rows, p) and np.array_equal(cols, p)


def test_ordinary_mask_is_not_transposable_in_general():
    """Context for the pins above: the row-wise mask alone breaks the column caps."""
    W = random_w(16, 16, "f32", seed=120)
    keep = blocks(oracle.mask(W, "f32", 2, 4).astype(int), 4)
    assert keep.sum(axis=1).max() > 2


def test_shape_rules():
    W = np.zeros((6, 8), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.tmask_greedy(W, "f32", 2, 4)      # R % m != 0
    with pytest.raises(ValueError):
        oracle.tmask_optimal(np.zeros((8, 6), np.float32), "f32", 2, 4)


def test_optimum_keeps_non_finite_entries_first():
    """Inf and NaN outrank every finite magnitude (the mask's order), also in the optimum."""
    a = np.random.default_rng(130).uniform(1, 2, size=(8, 8))
    a[0, 0] = a[3, 1] = np.inf
    a[5, 6] = -np.inf
    W = a.astype(np.float32)
    W.view(np.uint32)[6, 2] = 0x7FC00000  # NaN
    mask, _ = oracle.tmask_optimal(W, "f32", 2, 4)
    assert mask[0, 0] and mask[3, 1] and mask[5, 6] and mask[6, 2]
    g = oracle.tmask_greedy(W, "f32", 2, 4)
    assert g[0, 0] and g[3, 1] and g[5, 6] and g[6, 2]
