"""Pins for the oracle's FP8 path (OCP E4M3 bytes: mask, compress, decompress, product)
and for the generator's rounding to E4M3.

FP8 is not among the pages' sparse input types (the ASDNN review, "Tensor Scores 상에서
구조적인 sparse GEMM", lists FP16, BF16 and INT8); it is the same selection
("量化友好的SR-STE稀疏化训练", "NVIDA Apex内的静态掩码稀疏": keep the N largest |w| of
every M) at a narrower floating type.  Pins: every code's value against torch's
float8_e4m3fn conversion, brute force over exact magnitudes (NaN > 448 > ... > 0),
decompress(compress) as a select, and the product against numpy's float64 product of
the masked, decoded weight.
"""
from fractions import Fraction
from itertools import combinations

import numpy as np
import pytest
import torch

import oracle
import synth


def decode_torch(b: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def test_every_code_decodes_as_torch_does():
    codes = np.arange(256, dtype=np.uint8)
    d, t = oracle.to_double(codes, "fp8"), decode_torch(codes)
    assert np.array_equal(np.isnan(d), np.isnan(t))
    assert np.array_equal(d[~np.isnan(d)], t[~np.isnan(t)])
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF]) and d[0x7E] == 448.0


def test_generator_rounds_to_nearest_even_like_torch():
    rng = np.random.default_rng(0)
    x = np.clip(rng.standard_normal(100000) * np.exp2(rng.integers(-12, 8, 100000)), -448, 448)
    x = x.astype(np.float32)
    assert np.array_equal(synth.f32_to_e4m3_bits(x),
                          torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def brute_force_kept(codes, n):
    mags = []
    for c in codes:
        v = decode_torch(np.array([c], dtype=np.uint8))[0]
        mags.append(Fraction(10 ** 9) if np.isnan(v) else abs(Fraction(float(v))))
    best, best_set = None, None
    for s in combinations(range(len(codes)), n):
        score = sum(mags[i] for i in s)
        if best is None or score > best:
            best, best_set = score, s
    return best_set


@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (4, 8), (3, 8)])
def test_mask_matches_brute_force(n, m):
    rng = np.random.default_rng(n * 10 + m)
    W = rng.integers(0, 256, size=(12, 4 * m)).astype(np.uint8)
    W[W & 0x7F == 0x7F] = 0x38            # mostly no NaN ...
    W[0, 0] = 0x7F                        # ... but one, which ranks first
    W[1, :m] = 0x40                       # an all-tied group
    got = oracle.mask(W, "fp8", n, m).reshape(-1, m)
    for g, row in zip(W.reshape(-1, m), got):
        assert tuple(np.nonzero(row)[0].tolist()) == brute_force_kept(g.tolist(), n)


@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (4, 8)])
def test_decompress_of_compress_is_select_and_product_exact(n, m):
    R, K, T = 24, 16 * m, 20
    W = synth.generate(synth.Dist("normal", 3, 2.0), (R, K), "fp8")
    X = synth.generate(synth.Dist("normal", 4, 2.0), (K, T), "fp8")
    keep = oracle.mask(W, "fp8", n, m).astype(bool)
    vals, meta = oracle.compress(W, "fp8", n, m)
    dec = oracle.decompress(vals, meta, "fp8", R, K, n, m)
    assert np.array_equal(dec, np.where(keep, W, 0).astype(np.uint8))
    Wm = np.where(keep, decode_torch(W), 0.0)
    Y = oracle.spmm(vals, meta, R, K, n, m, X, "fp8")
    assert np.array_equal(Y, Wm @ decode_torch(X))  # every product and sum is exact here
