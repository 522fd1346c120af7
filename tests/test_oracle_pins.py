"""Pins for the CPU oracle: facts fixed by the pages and by mathematics, each
computed here without the oracle's own code path.

Sources: "量化友好的SR-STE稀疏化训练" section "NVIDA Apex内的静态掩码稀疏"
(exhaustive best-pattern search); "[리뷰] Accelerating Sparse Deep Neural
Networks" sections "Step-2: Weight Pruning" (drop the smallest), "2:4 Sparsity의
benefits" (R*C/2 values, 2-bit positions, 36 vs 64 bits) and "Tensor Scores
상에서 구조적인 sparse GEMM" (sparse x dense = dense).
"""
from fractions import Fraction
from itertools import combinations, product

import numpy as np
import pytest

import oracle
import synth
from tests.helpers import as_bits, encode, normwise_rel_err, read_hand_groups, read_kv

DTS = ["f32", "f16", "bf16"]


def exact(vals_bits: np.ndarray, dtype: str):
    """Exact rational |value| of every element (numpy decode, then Fraction)."""
    return [abs(Fraction(float(x))) for x in synth.bits_to_f64(vals_bits, dtype).ravel()]


def brute_force_kept(group_exact, n: int):
    """All n-subsets in lexicographic order; first one with the largest exact sum."""
    best, best_set = None, None
    for s in combinations(range(len(group_exact)), n):
        score = sum((group_exact[i] for i in s), Fraction(0))
        if best is None or score > best:
            best, best_set = score, s
    return best_set


def rank_rule_kept(group_exact, n: int):
    """Drop the smallest: order by (magnitude descending, index ascending), keep n."""
    order = sorted(range(len(group_exact)), key=lambda i: (-group_exact[i], i))
    return tuple(sorted(order[:n]))


def mask_to_sets(mask: np.ndarray, m: int):
    g = mask.reshape(-1, m)
    return [tuple(np.nonzero(row)[0].tolist()) for row in g]


# --------------------------------------------------------------------------
# Selection
# --------------------------------------------------------------------------


@pytest.mark.parametrize("n,m", [(1, 2), (1, 4), (2, 4), (3, 4)])
def test_mask_matches_brute_force_all_small_groups(n, m):
    """Every group over a tie-heavy alphabet: exhaustive oracle == brute force."""
    alphabet = [0.0, -0.0, 1.0, -1.0, 2.0, 3.0, -3.0]
    groups = list(product(alphabet, repeat=m))
    W = encode(np.array(groups).reshape(1, -1), "f32")
    got = mask_to_sets(oracle.mask(W, "f32", n, m), m)
    for gi, grp in enumerate(groups):
        ex = [abs(Fraction(v)) for v in grp]
        assert got[gi] == brute_force_kept(ex, n), grp


@pytest.mark.parametrize("dtype", DTS)
@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (2, 8), (4, 8), (5, 16)])
def test_mask_matches_brute_force_random(dtype, n, m):
    rng = np.random.default_rng(1000 + 10 * n + m)
    # wide exponent range plus repeated values, so both rounding and ties matter
    base = rng.choice([0.0, 1.0, 2.0, 2.0**-20, 3.0 * 2.0**-21, 1.5, 2.0**10], size=(6, 64))
    base *= rng.choice([-1.0, 1.0], size=base.shape)
    W = encode(base, dtype)
    got = mask_to_sets(oracle.mask(W, dtype, n, m), m)
    ex = exact(as_bits(W), dtype)
    for gi in range(len(got)):
        grp = ex[gi * m : (gi + 1) * m]
        assert got[gi] == brute_force_kept(grp, n)


@pytest.mark.parametrize("dtype", DTS)
@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (4, 8), (3, 8)])
def test_exhaustive_equals_drop_smallest(dtype, n, m):
    """The exhaustive best pattern keeps the same set as dropping the M-N smallest."""
    rng = np.random.default_rng(7)
    W = encode(np.round(rng.standard_normal((32, 128)) * 4) / 4, dtype)  # many ties
    got = mask_to_sets(oracle.mask(W, dtype, n, m), m)
    ex = exact(as_bits(W), dtype)
    for gi in range(len(got)):
        assert got[gi] == rank_rule_kept(ex[gi * m : (gi + 1) * m], n)


def test_exact_scores_matter():
    """fp32 scoring would keep {0,1}; the exact optimum is {0,2}."""
    g = np.array([[1.0, 1e-8, 2e-8, 0.0]], dtype=np.float32)
    assert np.float32(1.0) + np.float32(1e-8) == np.float32(1.0) + np.float32(2e-8)
    assert mask_to_sets(oracle.mask(g, "f32", 2, 4), 4) == [(0, 2)]


def test_wide_exponent_sums():
    """A sum of two tiny values can beat one mid value only when compared exactly."""
    tiny = 2.0**-149  # smallest fp32 subnormal
    g = np.array([[2 * tiny, tiny, tiny, 3 * tiny]], dtype=np.float32)
    assert mask_to_sets(oracle.mask(g, "f32", 2, 4), 4) == [(0, 3)]
    big = np.array([[3e38, 3.1e38, 3.2e38, 1.0]], dtype=np.float32)  # sums overflow fp32
    assert mask_to_sets(oracle.mask(big, "f32", 2, 4), 4) == [(1, 2)]


def test_non_finite_reading():
    """Reading: magnitudes order by sign-cleared bits, so NaN > Inf > finite."""
    g = np.array([[np.inf, 1.0, np.nan, 2.0], [-np.inf, 5.0, np.inf, 7.0]], dtype=np.float32)
    assert mask_to_sets(oracle.mask(g, "f32", 2, 4), 4) == [(0, 2), (0, 2)]


@pytest.mark.parametrize("dtype", DTS)
def test_invariants(dtype):
    rng = np.random.default_rng(3)
    W = encode(rng.standard_normal((16, 64)), dtype)
    for n, m in [(1, 2), (2, 4), (4, 8), (1, 4), (3, 8)]:
        mk = oracle.mask(W, dtype, n, m)
        assert np.all(mk.reshape(-1, m).sum(axis=1) == n)  # exactly N kept per group
    assert np.all(oracle.mask(W, dtype, 4, 4) == 1)  # N = M keeps everything
    # a 1:2 mask is a valid 2:4 mask (one of each pair => two of each four)
    m12 = oracle.mask(W, dtype, 1, 2).reshape(-1, 4)
    assert np.all(m12.sum(axis=1) == 2)
    # distinct magnitudes: plain top-N by |w|
    ex = synth.bits_to_f64(as_bits(W), dtype).reshape(-1, 4)
    mk = oracle.mask(W, dtype, 2, 4).reshape(-1, 4)
    for gi in range(ex.shape[0]):
        mags = np.abs(ex[gi])
        if len(set(mags.tolist())) == 4:
            top = set(np.argsort(-mags)[:2].tolist())
            assert set(np.nonzero(mk[gi])[0].tolist()) == top


def test_hand_worked_groups():
    for case in read_hand_groups():
        W = encode(np.array([case["values"]]), case["dtype"])
        if case["dtype"] == "f32":  # keep -0 exactly
            W = np.array([case["values"]], dtype=np.float32)
        n, m = case["n"], case["m"]
        mk = oracle.mask(W, case["dtype"], n, m)
        assert np.nonzero(mk[0])[0].tolist() == case["kept"], case["why"]
        vals, meta = oracle.compress(W, case["dtype"], n, m)
        assert int(meta[0, 0]) == case["meta"], case["why"]
        # stored values are bitwise copies of the kept weights
        assert as_bits(vals)[0].tolist() == as_bits(W)[0][case["kept"]].tolist()


# --------------------------------------------------------------------------
# Compressed format
# --------------------------------------------------------------------------


def test_storage_closed_form_36_of_64_bits():
    sizes = read_kv("format_sizes.txt")
    R, K, n, m = 1, 4, 2, 4
    W = encode(np.array([[1.0, -2.0, 3.0, 0.5]]), "f16")
    vals, meta = oracle.compress(W, "f16", n, m)
    dense_bits = K * 16
    compressed_bits = vals.size * 16 + n * oracle.meta_bits(m) * (K // m)
    assert dense_bits == sizes["dense_bits"]
    assert compressed_bits == sizes["compressed_bits"]
    assert round(100 * (1 - compressed_bits / dense_bits)) == sizes["saving_percent"]
    assert vals.shape == (R, K * n // m)


@pytest.mark.parametrize("K,n,m,words", [(128, 2, 4, 4), (768, 2, 4, 24), (4096, 1, 2, 64),
                                          (4096, 2, 4, 128), (4096, 4, 8, 192), (11008, 2, 4, 344),
                                          (8, 4, 8, 1), (12, 2, 4, 1), (40, 2, 4, 2)])
def test_meta_words_closed_form(K, n, m, words):
    assert oracle.meta_words_per_row(K, n, m) == words


@pytest.mark.parametrize("dtype", DTS)
def test_2_4_nibbles_are_legal(dtype):
    rng = np.random.default_rng(5)
    W = encode(np.round(rng.standard_normal((16, 256)) * 2) / 2, dtype)
    _, meta = oracle.compress(W, dtype, 2, 4)
    nibbles = [(int(w) >> (4 * i)) & 0xF for w in meta.ravel() for i in range(8)]
    assert set(nibbles) <= {0x4, 0x8, 0xC, 0x9, 0xD, 0xE}


@pytest.mark.parametrize("dtype", DTS)
@pytest.mark.parametrize("n,m", [(1, 2), (2, 4), (4, 8), (3, 8), (2, 8)])
def test_decompress_of_compress_is_select(dtype, n, m):
    """decompress(compress(W)) == where(mask, W, +0), bitwise; meta decodes to the mask."""
    rng = np.random.default_rng(11)
    K = 8 * 13  # rows whose metadata ends mid-word for 3-bit fields
    raw = rng.standard_normal((9, K))
    raw[0, :8] = [-0.0, 0.0, -0.0, 0.0, -1.0, -1.0, 0.0, -0.0]
    W = encode(raw, dtype)
    mk = oracle.mask(W, dtype, n, m)
    vals, meta = oracle.compress(W, dtype, n, m)
    Wd = oracle.decompress(vals, meta, dtype, W.shape[0], K, n, m)
    expect = np.where(mk == 1, as_bits(W), 0).astype(as_bits(W).dtype)
    assert np.array_equal(as_bits(Wd), expect)
    # independent bit-level decode of the metadata
    b = oracle.meta_bits(m)
    for r in range(W.shape[0]):
        bits = 0
        for i, w in enumerate(meta[r].tolist()):
            bits |= int(w) << (32 * i)
        for g in range(K // m):
            pos = [(bits >> ((g * n + j) * b)) & ((1 << b) - 1) for j in range(n)]
            assert pos == np.nonzero(mk[r, g * m : (g + 1) * m])[0].tolist()
        assert bits >> ((K // m) * n * b) == 0  # pad bits are zero


def test_compressed_values_keep_negative_zero():
    W = np.array([[-0.0, 0.0, 0.0, 0.0]], dtype=np.float32)
    vals, meta = oracle.compress(W, "f32", 2, 4)
    assert vals.view(np.uint32)[0].tolist() == [0x80000000, 0]
    assert int(meta[0, 0]) == 0x4


# --------------------------------------------------------------------------
# Sparse x dense product
# --------------------------------------------------------------------------


@pytest.mark.parametrize("dtype", DTS)
@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (4, 8)])
def test_spmm_equals_dense_product_of_masked_weight(dtype, n, m):
    rng = np.random.default_rng(21)
    R, K, T = 24, 64, 40
    W = encode(rng.standard_normal((R, K)), dtype)
    X = encode(rng.standard_normal((K, T)), dtype)
    vals, meta = oracle.compress(W, dtype, n, m)
    Y = oracle.spmm(vals, meta, R, K, n, m, X, dtype)
    mk = oracle.mask(W, dtype, n, m)
    Wm = np.where(mk == 1, synth.bits_to_f64(as_bits(W), dtype), 0.0)
    ref = Wm @ synth.bits_to_f64(as_bits(X), dtype)  # numpy float64 GEMM
    assert normwise_rel_err(Y, ref) <= 1e-12


@pytest.mark.parametrize("dtype", DTS)
def test_spmm_identity_gives_masked_weight(dtype):
    rng = np.random.default_rng(22)
    K = 32
    W = encode(rng.standard_normal((8, K)), dtype)
    X = encode(np.eye(K), dtype)
    vals, meta = oracle.compress(W, dtype, 2, 4)
    Y = oracle.spmm(vals, meta, 8, K, 2, 4, X, dtype)
    Wd = oracle.decompress(vals, meta, dtype, 8, K, 2, 4)
    assert np.array_equal(Y, synth.bits_to_f64(as_bits(Wd), dtype))


def test_spmm_integer_inputs_exact():
    rng = np.random.default_rng(23)
    R, K, T = 16, 64, 24
    Wi = rng.integers(-8, 9, size=(R, K)).astype(np.float64)
    Xi = rng.integers(-8, 9, size=(K, T)).astype(np.float64)
    for dtype in DTS:
        W, X = encode(Wi, dtype), encode(Xi, dtype)
        vals, meta = oracle.compress(W, dtype, 2, 4)
        Y = oracle.spmm(vals, meta, R, K, 2, 4, X, dtype)
        mk = oracle.mask(W, dtype, 2, 4)
        assert np.array_equal(Y, np.where(mk == 1, Wi, 0.0) @ Xi)


def test_spmm_n_equals_m_is_dense_gemm():
    rng = np.random.default_rng(24)
    W = encode(rng.standard_normal((8, 16)), "bf16")
    X = encode(rng.standard_normal((16, 8)), "bf16")
    vals, meta = oracle.compress(W, "bf16", 4, 4)
    Y = oracle.spmm(vals, meta, 8, 16, 4, 4, X, "bf16")
    ref = synth.bits_to_f64(W, "bf16") @ synth.bits_to_f64(X, "bf16")
    assert normwise_rel_err(Y, ref) <= 1e-12


def test_spmm_rows_and_samples_agree_with_full():
    rng = np.random.default_rng(25)
    R, K, T = 12, 32, 20
    W = encode(rng.standard_normal((R, K)), "f16")
    X = encode(rng.standard_normal((K, T)), "f16")
    vals, meta = oracle.compress(W, "f16", 2, 4)
    Y = oracle.spmm(vals, meta, R, K, 2, 4, X, "f16")
    Yr = np.zeros_like(Y)
    oracle.spmm_rows(vals, meta, R, K, 2, 4, X, "f16", 3, 9, Yr)
    assert np.array_equal(Yr[3:9], Y[3:9]) and not Yr[:3].any()
    rs, ts = rng.integers(0, R, 30), rng.integers(0, T, 30)
    assert np.array_equal(oracle.spmm_sample(vals, meta, R, K, 2, 4, X, "f16", rs, ts), Y[rs, ts])


def test_oracle_rejects_bad_arguments():
    W = np.zeros((2, 6), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.mask(W, "f32", 2, 4)  # K % M != 0
    with pytest.raises(ValueError):
        oracle.mask(np.zeros((2, 8), np.float32), "f32", 5, 4)  # N > M
    with pytest.raises(ValueError):
        oracle.mask(np.zeros((2, 6), np.float32), "f32", 1, 3)  # M not a power of two
