"""Pins for the oracle's int8 path (mask, compress, decompress, exact product).

Sources: "[리뷰] Accelerating Sparse Deep Neural Networks", section "Tensor Scores
상에서 구조적인 sparse GEMM" (INT8 inputs to the sparse product) and
"量化友好的SR-STE稀疏化训练", section "NVIDA Apex内的静态掩码稀疏" (keep the N of
every M with the largest |w|).  Reading: |w| is the integer magnitude of the
two's-complement value (|-128| = 128), equal magnitudes go to the lower index,
and products are exact integers.

Pins: hand-worked groups (tests/golden/i8_groups.txt), brute force over every
group of a tie-heavy alphabet that includes -128 and 127, decompress(compress) =
select(mask, W, 0), and the product against numpy's int64 matrix product of the
masked weight.
"""
import os
from itertools import combinations, product

import numpy as np
import pytest

import oracle
import synth
from tests.helpers import GOLDEN


def read_i8_groups():
    rows = []
    with open(os.path.join(GOLDEN, "i8_groups.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, grp, kept, vals, why = [p.strip() for p in line.split("|", 4)]
            n, m = (int(x) for x in head.split())
            rows.append(dict(n=n, m=m, group=[int(x) for x in grp.split()],
                             kept=[int(x) for x in kept.split()],
                             vals=[int(x) for x in vals.split()], why=why))
    return rows


def brute_force_kept(group, n):
    mags = [abs(int(v)) for v in group]
    best, best_set = None, None
    for s in combinations(range(len(group)), n):
        score = sum(mags[i] for i in s)
        if best is None or score > best:
            best, best_set = score, s
    return best_set


@pytest.mark.parametrize("case", read_i8_groups(), ids=lambda c: c["why"][:40])
def test_hand_worked_groups(case):
    W = np.array([case["group"]], dtype=np.int8)
    n, m = case["n"], case["m"]
    assert np.nonzero(oracle.mask(W, "i8", n, m)[0])[0].tolist() == case["kept"], case["why"]
    vals, _ = oracle.compress(W, "i8", n, m)
    assert vals.view(np.int8)[0].tolist() == case["vals"], case["why"]


@pytest.mark.parametrize("n,m", [(1, 2), (1, 4), (2, 4), (3, 4)])
def test_mask_matches_brute_force_all_small_groups(n, m):
    alphabet = [0, 1, -1, 2, 127, -127, -128]
    groups = list(product(alphabet, repeat=m))
    W = np.array(groups, dtype=np.int8).reshape(1, -1)
    got = oracle.mask(W, "i8", n, m).reshape(-1, m)
    for g, row in zip(groups, got):
        assert tuple(np.nonzero(row)[0].tolist()) == brute_force_kept(g, n), g


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (2, 8), (1, 2)])
def test_mask_matches_brute_force_random(n, m):
    rng = np.random.default_rng(10 * n + m)
    W = rng.integers(-128, 128, size=(16, 8 * m)).astype(np.int8)
    W[::3] //= 16  # more ties
    got = oracle.mask(W, "i8", n, m).reshape(-1, m)
    for g, row in zip(W.reshape(-1, m), got):
        assert tuple(np.nonzero(row)[0].tolist()) == brute_force_kept(g, n)


@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (4, 8), (3, 8), (1, 4)])
def test_decompress_of_compress_is_select(n, m):
    W = synth.generate(synth.Dist("normal", 7, 40.0), (24, 16 * m), "i8")
    keep = oracle.mask(W, "i8", n, m).astype(bool)
    vals, meta = oracle.compress(W, "i8", n, m)
    dec = oracle.decompress(vals, meta, "i8", 24, 16 * m, n, m).view(np.int8)
    assert np.array_equal(dec, np.where(keep, W, 0).astype(np.int8))


@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (4, 8)])
def test_product_is_the_exact_integer_product(n, m):
    R, K, T = 40, 32 * m, 24
    W = synth.generate(synth.Dist("normal", 8, 60.0), (R, K), "i8")
    X = synth.generate(synth.Dist("normal", 9, 60.0), (K, T), "i8")
    keep = oracle.mask(W, "i8", n, m).astype(bool)
    Wm = np.where(keep, W, 0).astype(np.int64)
    vals, meta = oracle.compress(W, "i8", n, m)
    Y = oracle.spmm(vals, meta, R, K, n, m, X, "i8")
    assert np.array_equal(Y, (Wm @ X.astype(np.int64)).astype(np.float64))


def test_extreme_sums_stay_exact():
    """Every product -128 * -128 over 8192 kept terms: 2^27, exact in the double sum."""
    R, K, T = 2, 16384, 3
    W = np.full((R, K), -128, dtype=np.int8)
    X = np.full((K, T), -128, dtype=np.int8)
    vals, meta = oracle.compress(W, "i8", 2, 4)
    Y = oracle.spmm(vals, meta, R, K, 2, 4, X, "i8")
    assert np.all(Y == 16384 * 8192)


def test_int8_is_rejected_where_the_method_needs_floats():
    W = np.zeros((8, 8), dtype=np.int8)
    for f in (lambda: oracle.prune(W, "i8", 2, 4), lambda: oracle.srste_grad(W, W, "i8", 2, 4, 2e-4),
              lambda: oracle.tmask_greedy(W, "i8", 2, 4)):
        with pytest.raises(ValueError):
            f()
