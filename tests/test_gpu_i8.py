"""GPU parity of the int8 path (mask, compress, decompress, exact int32 product)
against the oracle.

Everything is compared exactly: masks, stored values, metadata, decompressed
weights, and the products (the oracle's double sums of int8 products are exact
integers, and so are the library's int32 sums).
"""
import numpy as np
import pytest
import torch

import masking_sparse_gemm_amd as nm
import oracle
import synth
from tests.helpers import blocked_from_rows

pytestmark = pytest.mark.gpu

PATTERNS = [(1, 2), (2, 2), (1, 4), (2, 4), (3, 4), (4, 4), (1, 8), (2, 8), (3, 8), (4, 8), (6, 8),
            (8, 8)]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nm.lib()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def dev8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int8)).cuda()


def host8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint8)


def blocked_ok(n, m):
    return (16 * n // m) % 4 == 0


def int8_matrix(rng, shape, ties=True):
    a = rng.integers(-128, 128, size=shape)
    if ties:
        a[rng.random(shape) < 0.3] //= 32
        a[rng.random(shape) < 0.05] = -128
    return a.astype(np.int8)


def check_select_i8(W: np.ndarray, n: int, m: int, label: str):
    R, K = W.shape
    Wd = dev8(W)
    vals_o, meta_o = oracle.compress(W, "i8", n, m)
    assert np.array_equal(nm.mask(Wd, n, m).cpu().numpy().astype(np.uint8),
                          oracle.mask(W, "i8", n, m)), f"mask {label}"
    v, mt = nm.compress(Wd, n, m)
    assert np.array_equal(host8(v), vals_o), f"values {label}"
    assert np.array_equal(mt.cpu().numpy().view(np.uint32), meta_o), f"meta {label}"
    dec_o = oracle.decompress(vals_o, meta_o, "i8", R, K, n, m)
    assert np.array_equal(host8(nm.decompress(v, mt, n, m, K)), dec_o), f"decompress {label}"
    if K % 64 == 0 and blocked_ok(n, m):
        vb, mb = nm.compress(Wd, n, m, layout="blocked")
        vb_o, mb_o = blocked_from_rows(vals_o, meta_o, R, K, n, m)
        assert np.array_equal(host8(vb), vb_o), f"blocked values {label}"
        assert np.array_equal(mb.cpu().numpy().view(np.uint32), mb_o), f"blocked meta {label}"
        dec = nm.decompress(vb, mb, n, m, K, layout="blocked", rows=R)
        assert np.array_equal(host8(dec), dec_o), f"blocked decompress {label}"
    return v, mt, vals_o, meta_o


@pytest.mark.parametrize("n,m", PATTERNS)
def test_i8_select_shapes(n, m):
    rng = np.random.default_rng(900 + 10 * n + m)
    for R, K in [(7, 128), (33, 96), (5, 24), (64, 8), (3, 1024), (17, 64), (9, 16 * 17)]:
        if K % m:
            continue
        check_select_i8(int8_matrix(rng, (R, K)), n, m, f"{R}x{K} {n}:{m}")


def test_i8_select_extremes():
    W = np.array([[-128, 127, 127, 0, -128, -128, 127, -127] * 8,
                  [0, 0, 0, -1, 1, -1, 1, -1] * 8], dtype=np.int8)
    for n, m in [(2, 4), (1, 2), (4, 8), (2, 8)]:
        check_select_i8(W, n, m, f"extremes {n}:{m}")


@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (4, 8), (1, 4), (3, 4), (2, 8)])
@pytest.mark.parametrize("layout", ["rows", "blocked"])
def test_i8_product_exact(n, m, layout):
    if layout == "blocked" and not blocked_ok(n, m):
        pytest.skip("pattern not stored in the blocked int8 layout")
    rng = np.random.default_rng(950 + n + m)
    # (70, 1280, 48): more than 512 of K, so the expansion kernel's exact fp32 chunks are
    # moved into int32 several times
    for R, K, T in [(200, 384, 264), (130, 256, 136), (16, 128, 8), (33, 64, 13), (257, 128, 520),
                    (70, 1280, 48)]:
        W = int8_matrix(rng, (R, K))
        X = int8_matrix(rng, (K, T), ties=False)
        vals_o, meta_o = oracle.compress(W, "i8", n, m)
        v, mt = nm.compress(dev8(W), n, m, layout=layout)
        Y = nm.spmm(v, mt, dev8(X), n, m, layout=layout, rows=R)
        assert Y.dtype == torch.int32
        y_ref = oracle.spmm(vals_o, meta_o, R, K, n, m, X, "i8")
        assert np.array_equal(Y.cpu().numpy().astype(np.float64), y_ref), f"{R}x{K}x{T} {n}:{m}"


@pytest.mark.parametrize("R,K,T", [(200, 384, 272), (300, 256, 144), (16, 128, 16), (513, 640, 400),
                                   (256, 1024, 256), (40, 128, 1040)])
@pytest.mark.parametrize("layout", ["rows", "blocked"])
@pytest.mark.parametrize("n,m", [(2, 4), (1, 2)])
def test_i8_matrix_core_product_exact(R, K, T, layout, n, m):
    """Shapes the int8 matrix-core kernel takes (2:4 or 1:2, K % 128 == 0, T % 16 == 0),
    several tiles with ragged row and column tails: exact against the oracle."""
    rng = np.random.default_rng(R + K + T)
    W = int8_matrix(rng, (R, K))
    X = int8_matrix(rng, (K, T), ties=False)
    vals_o, meta_o = oracle.compress(W, "i8", n, m)
    v, mt = nm.compress(dev8(W), n, m, layout=layout)
    Y = nm.spmm(v, mt, dev8(X), n, m, layout=layout, rows=R)
    y_ref = oracle.spmm(vals_o, meta_o, R, K, n, m, X, "i8")
    got = Y.cpu().numpy().astype(np.float64)
    bad = got != y_ref
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} differ, first at {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("n,m", [(4, 8), (1, 4), (3, 4)])
def test_i8_product_extremes_other_patterns(n, m):
    """All -128: every output is (K n/m) * 2^14, far past fp32's exact integers, through the
    expansion kernel's exact int32 totals."""
    R, K, T = 64, 4096, 64
    W = np.full((R, K), -128, dtype=np.int8)
    X = np.full((K, T), -128, dtype=np.int8)
    for layout in ["rows", "blocked"]:
        v, mt = nm.compress(dev8(W), n, m, layout=layout)
        Y = nm.spmm(v, mt, dev8(X), n, m, layout=layout, rows=R)
        assert bool((Y == K // m * n * 16384).all()), layout


def test_i8_product_extremes_and_empty():
    R, K, T = 64, 4096, 64
    W = np.full((R, K), -128, dtype=np.int8)
    X = np.full((K, T), -128, dtype=np.int8)
    v, mt = nm.compress(dev8(W), 2, 4)
    Y = nm.spmm(v, mt, dev8(X), 2, 4)
    assert bool((Y == 2048 * 16384).all())
    Z = nm.spmm(v, mt, dev8(np.zeros((K, 0), np.int8)), 2, 4)
    assert Z.shape == (R, 0)
    E = torch.zeros((0, 128), dtype=torch.int8, device="cuda")
    ve, me = nm.compress(E, 2, 4)
    assert nm.spmm(ve, me, dev8(np.zeros((128, 8), np.int8)), 2, 4).shape == (0, 8)


@pytest.mark.parametrize("name", ["llama_up_i8", "llama_down_i8"])
@pytest.mark.parametrize("layout", ["rows", "blocked"])
def test_i8_full_workloads(name, layout):
    """Selection bit for bit at full size; the product on sampled outputs, each an exact
    dot product in the oracle, launched as the benchmark launches it."""
    w = synth.WORKLOADS[name]
    W, X = w.W(), w.X()
    print(f"[i8] {name} {w.R}x{w.K} x {w.T} {layout}", flush=True)
    vals_o, meta_o = oracle.compress(W, "i8", 2, 4)
    v, mt = nm.compress(dev8(W), 2, 4, layout=layout)
    if layout == "rows":
        assert np.array_equal(host8(v), vals_o) and np.array_equal(mt.cpu().numpy().view(np.uint32), meta_o)
    else:
        vb_o, mb_o = blocked_from_rows(vals_o, meta_o, w.R, w.K, 2, 4)
        assert np.array_equal(host8(v), vb_o) and np.array_equal(mt.cpu().numpy().view(np.uint32), mb_o)
    Y = nm.spmm(v, mt, dev8(X), 2, 4, layout=layout, rows=w.R).cpu().numpy()
    rng = np.random.default_rng(3)
    rs = np.concatenate([rng.integers(0, w.R, 1500), [w.R - 1, 0]])
    ts = np.concatenate([rng.integers(0, w.T, 1500), [w.T - 1, w.T - 1]])
    want = oracle.spmm_sample(vals_o, meta_o, w.R, w.K, 2, 4, X, "i8", rs, ts)
    assert np.array_equal(Y[rs, ts].astype(np.float64), want)


def crafted_i8_case(n, m, R, K, T, seed):
    """W, X for test_i8_expansion_exact_past_fp32_integers: large same-sign products almost
    everywhere, +-1 entries where they are kept or multiplied."""
    rng = np.random.default_rng(seed)
    s = rng.choice([-1, 1], size=K)
    W = np.broadcast_to(s[None, :] * 127, (R, K)).copy()
    W[(s[None, :] < 0) & (rng.random((R, K)) < 0.3)] = -128
    # in one group in five, m - n + 1 entries become +-1: the group then keeps n - 1 large
    # values and one +-1 (the first of the tied small ones)
    G = K // m
    for r, g in zip(*np.nonzero(rng.random((R, G)) < 0.2)):
        pos = g * m + rng.choice(m, size=m - n + 1, replace=False)
        W[r, pos] = rng.choice([-1, 1], size=pos.size)
    X = np.broadcast_to(s[:, None] * 127, (K, T)).copy()
    X[(s[:, None] < 0) & (rng.random((K, T)) < 0.3)] = -128
    small = rng.random((K, T)) < 0.05
    X[small] = rng.choice([-1, 1], size=int(small.sum()))
    return W.astype(np.int8), X.astype(np.int8)


@pytest.mark.parametrize("n,m", [(4, 8), (1, 4), (3, 4)])
@pytest.mark.parametrize("layout", ["rows", "blocked"])
def test_i8_expansion_exact_past_fp32_integers(n, m, layout):
    """The expansion kernel's int8 product where rounding would show.  Most kept products
    are +127^2 .. +128^2 (W's column signs match X's row signs), so each 512-wide run of K
    sums to within a factor 4 of 2^23 and every total passes 2^24; +-1 entries kept in W
    and spread through X put odd products of +-1 and +-127 beside them in every 16-wide run.
    An fp32 total, a run summed past 2^24, or an adder that drops low bits against a large
    partial sum would lose them; the int32 totals must equal the oracle's exact integers."""
    R, K, T = 96, 6144, 80
    W, X = crafted_i8_case(n, m, R, K, T, 4000 + 10 * n + m)
    vals_o, meta_o = oracle.compress(W, "i8", n, m)
    y_ref = oracle.spmm(vals_o, meta_o, R, K, n, m, X, "i8")
    assert np.abs(y_ref).min() > 2 ** 24 and (y_ref % 2 == 1).any()   # the case is what it says
    v, mt = nm.compress(dev8(W), n, m, layout=layout)
    Y = nm.spmm(v, mt, dev8(X), n, m, layout=layout, rows=R)
    got = Y.cpu().numpy().astype(np.float64)
    bad = got != y_ref
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} differ, first at {np.argwhere(bad)[0]}"
