"""Pins for the oracle's channel permutation (kept L1, swap gains, swap search).

Source: "[리뷰] Accelerating Sparse Deep Neural Networks", section "Step-2: Weight
Pruning" (Fig. 6): permuting the weight's columns before the 2:4 mask spreads the
large values over the groups, so that the mask keeps a larger total magnitude.
Reading (the pages give only the effect): the objective is the kept L1 of the N:M
mask of W[:, perm]; the search runs rounds of the best single swap per pair of
groups, applied to disjoint pairs in descending order of gain.

Pins: the kept L1 equals |W| summed under the (pinned) mask; it ignores the order
inside groups and of the groups; every gain equals a brute-force re-evaluation of
the swapped permutation; the search never lowers the kept L1, ends with no
improving swap, returns a bijection and reaches the brute-force optimum where a
single round suffices.
"""
from itertools import combinations

import numpy as np
import pytest

import oracle
from tests.helpers import encode


def kept_by_sorting(W: np.ndarray, n: int, m: int, perm) -> float:
    """Independent objective: sort each group's magnitudes, sum the n largest."""
    a = np.abs(W.astype(np.float64))[:, perm]
    g = np.sort(a.reshape(a.shape[0], -1, m), axis=2)[:, :, m - n:]
    return float(g.sum())


def matrix(R, K, seed, dt="f32", scale=1.0):
    rng = np.random.default_rng(seed)
    # integers times 2^-4: every sum below is exact in double and in fp32
    return encode(np.round(rng.standard_normal((R, K)) * 16 * scale) / 16, dt)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (4, 8), (1, 4)])
def test_kept_l1_is_the_masked_magnitude(dt, n, m):
    W = matrix(12, 8 * m, seed=n + m, dt=dt)
    keep = oracle.mask(W, dt, n, m).astype(bool)
    from synth import bits_to_f64
    a = np.abs(bits_to_f64(W if dt != "f32" else W.view(np.uint32), dt))
    assert oracle.kept_l1(W, dt, n, m) == pytest.approx(float(a[keep].sum()), rel=1e-12)


def test_kept_l1_ignores_order_inside_and_between_groups():
    W = matrix(10, 16, seed=3)
    rng = np.random.default_rng(4)
    base = oracle.kept_l1(W, "f32", 2, 4)
    for _ in range(5):
        groups = rng.permutation(4)
        perm = np.concatenate([rng.permutation(4) + 4 * g for g in groups]).astype(np.int32)
        assert oracle.kept_l1(W, "f32", 2, 4, perm) == base


@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (4, 8), (1, 2)])
def test_gains_match_brute_force(n, m):
    R, K = 9, 4 * m
    W = matrix(R, K, seed=10 * n + m)
    rng = np.random.default_rng(5)
    perm = rng.permutation(K).astype(np.int32)
    gain, pick = oracle.perm_gains(W, "f32", n, m, perm)
    base = kept_by_sorting(W, n, m, perm)
    G = K // m
    for g1, g2 in combinations(range(G), 2):
        deltas = []
        for a in range(m):
            for b in range(m):
                p = perm.copy()
                p[g1 * m + a], p[g2 * m + b] = p[g2 * m + b], p[g1 * m + a]
                deltas.append(kept_by_sorting(W, n, m, p) - base)
        assert gain[g1, g2] == pytest.approx(max(deltas), abs=1e-9)
        assert pick[g1, g2] == int(np.argmax(np.array(deltas) >= max(deltas) - 1e-12))


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 4)])
def test_search_is_monotone_and_ends_swap_optimal(n, m):
    W = matrix(16, 8 * m, seed=20 + n + m)
    K = W.shape[1]
    perm = np.arange(K, dtype=np.int32)
    last = oracle.kept_l1(W, "f32", n, m, perm)
    for _ in range(50):
        nxt, rounds = oracle.perm_search(W, "f32", n, m, max_rounds=1, perm=perm)
        now = oracle.kept_l1(W, "f32", n, m, nxt)
        assert now >= last
        if rounds == 0:
            break
        assert now > last
        perm, last = nxt, now
    assert sorted(perm.tolist()) == list(range(K))
    gain, _ = oracle.perm_gains(W, "f32", n, m, perm)
    assert np.triu(gain, 1).max() <= 0


def test_search_reaches_the_optimum_on_a_clustered_matrix():
    """Large values packed into the first group (the situation of Fig. 6): the best
    partition spreads them, and the search finds a partition as good as brute force."""
    R, K, n, m = 6, 8, 2, 4
    rng = np.random.default_rng(7)
    a = rng.uniform(0.0, 1.0, size=(R, K))
    a[:, :4] += 8.0  # the four largest columns share one group
    W = (np.round(a * 16) / 16).astype(np.float32)
    start = oracle.kept_l1(W, "f32", n, m)
    perm, _ = oracle.perm_search(W, "f32", n, m)
    found = oracle.kept_l1(W, "f32", n, m, perm)
    best = max(kept_by_sorting(W, n, m, list(c) + [j for j in range(K) if j not in c])
               for c in combinations(range(K), 4))
    assert found == pytest.approx(best, rel=1e-12) and found > start * 1.3


def test_identity_is_kept_when_nothing_improves():
    W = np.ones((4, 8), dtype=np.float32)
    perm, rounds = oracle.perm_search(W, "f32", 2, 4)
    assert rounds == 0 and perm.tolist() == list(range(8))
