"""GPU parity of the transposable-mask path (nm_tmask, nm_tprune, nm_compress_t)
against the oracle, and of the backward product it enables.

Masks, pruned weights and both compressed pairs are compared bit for bit.  The
backward product W^T dY through nm_compress_t + nm_spmm is held to the product
tolerance and element bound of tests/test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

import masking_sparse_gemm_amd as nm
import oracle
import synth
from tests.helpers import as_bits, blocked_from_rows, encode
from tests.test_gpu_parity import check_product, dev, host_bits, reference_product, tie_heavy

pytestmark = pytest.mark.gpu

DTS = ["bf16", "f16", "f32"]
TPATTERNS = [(2, 4), (1, 4), (3, 4), (4, 4), (1, 2), (4, 8), (2, 8), (1, 8), (6, 8)]
# (R, K) with R and K multiples of 8: several blocks of 256 threads, ragged last block
TSHAPES = [(8, 16), (16, 264), (64, 1032), (40, 72), (136, 520), (8, 8)]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nm.lib()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def check_tmask(W: np.ndarray, dtype: str, n: int, m: int, label: str):
    Wd = dev(W, dtype)
    mask_o = oracle.tmask_greedy(W, dtype, n, m)
    got = nm.tmask(Wd, n, m).cpu().numpy().astype(np.uint8)
    assert np.array_equal(got, mask_o), f"tmask {label}"
    pr = nm.tprune(Wd, n, m)
    assert np.array_equal(host_bits(pr), as_bits(oracle.tprune(W, dtype, n, m))), f"tprune {label}"
    return pr


@pytest.mark.parametrize("dtype", DTS)
@pytest.mark.parametrize("n,m", TPATTERNS)
def test_tmask_small_shapes(dtype, n, m):
    rng = np.random.default_rng(500 + 10 * n + m)
    for R, K in TSHAPES:
        check_tmask(tie_heavy(rng, (R, K), dtype), dtype, n, m, f"{R}x{K} {n}:{m}")


@pytest.mark.parametrize("dtype", DTS)
def test_tmask_special_values(dtype):
    big = 65504.0 if dtype == "f16" else 3e38
    vals = [0.0, -0.0, 1.0, -1.0, big, 2.0 ** -24, np.inf, -np.inf, 5.0, 5.0]
    rng = np.random.default_rng(21)
    W = encode(rng.choice(vals, size=(32, 64)), dtype).copy()
    as_bits(W).reshape(-1)[7::23] = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}[dtype]
    for n, m in [(2, 4), (4, 8), (1, 2), (1, 8)]:
        check_tmask(W, dtype, n, m, f"special {n}:{m}")


def test_tprune_in_place_and_empty():
    rng = np.random.default_rng(22)
    W = tie_heavy(rng, (32, 96), "bf16")
    Wd = dev(W, "bf16")
    nm.tprune(Wd, 2, 4, out=Wd)
    assert np.array_equal(host_bits(Wd), as_bits(oracle.tprune(W, "bf16", 2, 4)))
    for R, K in [(0, 64), (8, 0)]:
        Z = torch.zeros((R, K), dtype=torch.bfloat16, device="cuda")
        assert nm.tmask(Z, 2, 4).shape == (R, K) and nm.tprune(Z, 2, 4).shape == (R, K)


def check_compress_t(W: np.ndarray, dtype: str, n: int, m: int, label: str):
    """compress_t on the GPU == oracle compress of W.T, in both layouts where allowed."""
    R, K = W.shape
    Wd = dev(W, dtype)
    vals_o, meta_o = oracle.compress_t(W, dtype, n, m)
    v, mt = nm.compress_t(Wd, n, m)
    assert np.array_equal(host_bits(v), as_bits(vals_o)), f"values_t {label}"
    assert np.array_equal(host_bits(mt), meta_o), f"meta_t {label}"
    if R % 64 == 0:
        vb, mb = nm.compress_t(Wd, n, m, layout="blocked")
        vb_o, mb_o = blocked_from_rows(as_bits(vals_o), meta_o, K, R, n, m)
        assert np.array_equal(host_bits(vb), vb_o), f"blocked values_t {label}"
        assert np.array_equal(host_bits(mb), mb_o), f"blocked meta_t {label}"
    return vals_o, meta_o


@pytest.mark.parametrize("dtype", DTS)
@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (4, 8), (3, 8), (1, 4)])
def test_compress_t_shapes(dtype, n, m):
    rng = np.random.default_rng(600 + 10 * n + m)
    # K not a multiple of 16 (padding rows of the transpose) and not of 8 (scalar loads)
    for R, K in [(64, 128), (128, 40), (64, 100), (192, 17 * m), (8, 24), (64, 8)]:
        if R % m:
            continue
        check_compress_t(tie_heavy(rng, (R, K), dtype), dtype, n, m, f"{R}x{K} {n}:{m}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 2)])
@pytest.mark.parametrize("layout", ["rows", "blocked"])
def test_backward_product_through_the_transposable_mask(dtype, n, m, layout):
    """dX = Wp^T dY with Wp = tprune(W): compress_t + spmm against the oracle."""
    rng = np.random.default_rng(700 + n + m)
    R, K, T = 192, 128, 72   # W is R x K; the backward product is K x R times R x T
    W = encode(rng.standard_normal((R, K)), dtype)
    dY = encode(rng.standard_normal((R, T)), dtype)
    Wp = nm.tprune(dev(W, dtype), n, m)
    Wp_o = oracle.tprune(W, dtype, n, m)
    assert np.array_equal(host_bits(Wp), as_bits(Wp_o))
    v, mt = nm.compress_t(Wp, n, m, layout=layout)
    Yt = nm.spmm(v, mt, dev(dY, dtype), n, m, layout=layout, rows=K)
    vals_o, meta_o = oracle.compress_t(Wp_o, dtype, n, m)
    y_ref, s = reference_product(vals_o, meta_o, K, R, n, m, dY, dtype)
    check_product(Yt, y_ref, s, R * n // m, dtype, dtype, f"backward {n}:{m} {layout}")
    # the same pruned weight also gives the forward operand
    X = encode(rng.standard_normal((K, T)), dtype)
    vf, mf = nm.compress(Wp, n, m, layout=layout)
    Yf = nm.spmm(vf, mf, dev(X, dtype), n, m, layout=layout, rows=R)
    vf_o, mf_o = oracle.compress(Wp_o, dtype, n, m)
    y_ref, s = reference_product(vf_o, mf_o, R, K, n, m, X, dtype)
    check_product(Yf, y_ref, s, K * n // m, dtype, dtype, f"forward {n}:{m} {layout}")


@pytest.mark.parametrize("name,n,m", [("llama_up", 2, 4), ("llama_down", 2, 4), ("bert_ffn", 2, 4),
                                      ("sweep_f16", 4, 8), ("sweep_f16", 2, 4), ("toy_f32", 2, 4)])
def test_tmask_full_workloads(name, n, m):
    """Whole matrices on the GPU; the oracle checks row bands (the mask is independent per
    band of m rows) at the top, middle and bottom, and the transposed compression of the
    pruned weight in full."""
    w = synth.WORKLOADS[name]
    W = w.W()
    Wd = dev(W, w.dtype)
    print(f"[tmask] {name} {w.R}x{w.K} {n}:{m}", flush=True)
    mask = nm.tmask(Wd, n, m).cpu().numpy().astype(np.uint8)
    pr = nm.tprune(Wd, n, m)
    prh = host_bits(pr)
    for a in (0, (w.R // 2) // 64 * 64, w.R - 64):
        b = min(w.R, a + 64)
        band = np.ascontiguousarray(W[a:b])
        assert np.array_equal(mask[a:b], oracle.tmask_greedy(band, w.dtype, n, m)), f"rows {a}"
        assert np.array_equal(prh[a:b], as_bits(oracle.tprune(band, w.dtype, n, m))), f"rows {a}"
    layout = "blocked" if w.R % 64 == 0 else "rows"
    v, mt = nm.compress_t(pr, n, m, layout=layout)
    vals_o, meta_o = oracle.compress_t(prh, w.dtype, n, m)
    if layout == "blocked":
        vals_o, meta_o = blocked_from_rows(as_bits(vals_o), meta_o, w.K, w.R, n, m)
    assert np.array_equal(host_bits(v), as_bits(vals_o)) and np.array_equal(host_bits(mt), meta_o)
