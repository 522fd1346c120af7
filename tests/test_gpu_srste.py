"""GPU parity of the SR-STE passes (nm_prune, nm_srste_grad) against the oracle.

Both outputs are compared bit for bit: the forward weight is a selection, and the
gradient is computed in the same fp32 order on both sides (product, then sum, then
one rounding to the element type).  Results that are NaN on one side must be NaN
on the other (payloads may differ).
"""
import numpy as np
import pytest
import torch

import masking_sparse_gemm_amd as nm
import oracle
import synth
from tests.helpers import as_bits, encode
from tests.test_gpu_parity import SELECT_PATTERNS, dev, host_bits, tie_heavy

pytestmark = pytest.mark.gpu

DTS = ["bf16", "f16", "f32"]
NAN = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nm.lib()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def is_nan(bits: np.ndarray, dtype: str) -> np.ndarray:
    b = as_bits(bits)
    if dtype == "f32":
        return (b & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if dtype == "f16":
        return (b & np.uint16(0x7FFF)) > np.uint16(0x7C00)
    return (b & np.uint16(0x7FFF)) > np.uint16(0x7F80)


def assert_same_bits(got: np.ndarray, want: np.ndarray, dtype: str, label: str):
    got, want = as_bits(got), as_bits(want)
    ng, nw = is_nan(got, dtype), is_nan(want, dtype)
    assert np.array_equal(ng, nw), f"NaN positions differ: {label}"
    bad = (got != want) & ~nw
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{label}: {int(bad.sum())} elements differ, first {idx}: "
                             f"got {got[bad][:5]} want {want[bad][:5]}")


def check_srste(W: np.ndarray, G: np.ndarray, dtype: str, n: int, m: int, decay: float,
                label: str):
    Wd, Gd = dev(W, dtype), dev(G, dtype)
    assert_same_bits(host_bits(nm.prune(Wd, n, m)), oracle.prune(W, dtype, n, m), dtype,
                     f"prune {label}")
    assert_same_bits(host_bits(nm.srste_grad(Wd, Gd, n, m, decay)),
                     oracle.srste_grad(W, G, dtype, n, m, decay), dtype, f"grad {label}")


def gradient(rng, shape, dtype, scale=1e-3):
    return encode(rng.standard_normal(shape) * scale, dtype)


# Shapes with ragged tails: R*K not a multiple of the 16-byte unit (8 x 16-bit or
# 4 x fp32 elements) for some patterns, and sizes spanning several blocks of
# 256 lanes x 4 units.
SRSTE_SHAPES = [(7, 128), (5, 24), (33, 96), (1, 8), (3, 1000), (129, 2056), (2, 8200), (3, 40),
                (65, 264)]


@pytest.mark.parametrize("dtype", DTS)
@pytest.mark.parametrize("n,m", SELECT_PATTERNS)
def test_srste_small_shapes(dtype, n, m):
    rng = np.random.default_rng(300 + 10 * n + m)
    for R, K in SRSTE_SHAPES:
        if K % m:
            continue
        W = tie_heavy(rng, (R, K), dtype)
        G = gradient(rng, (R, K), dtype)
        check_srste(W, G, dtype, n, m, 2e-4, f"{R}x{K} {n}:{m}")


@pytest.mark.parametrize("dtype", DTS)
@pytest.mark.parametrize("R,K,m", [(3, 12, 4), (5, 6, 2), (1, 4, 4), (1, 2, 2), (9, 20, 4)])
def test_srste_tail_only_and_ragged(dtype, R, K, m):
    """R*K below or not a multiple of one unit: the per-group tail kernel."""
    rng = np.random.default_rng(R * 100 + K)
    W = tie_heavy(rng, (R, K), dtype)
    G = gradient(rng, (R, K), dtype)
    for n in range(1, m + 1):
        check_srste(W, G, dtype, n, m, 2e-4, f"{R}x{K} {n}:{m}")


@pytest.mark.parametrize("dtype", DTS)
@pytest.mark.parametrize("decay", [0.0, 1.0, -0.5, float.fromhex("0x1.000002p-8"), 3.75, 1e-30])
def test_srste_grad_decays(dtype, decay):
    rng = np.random.default_rng(7)
    W = encode(rng.standard_normal((64, 256)), dtype)
    G = gradient(rng, (64, 256), dtype, scale=1.0)
    for n, m in [(2, 4), (4, 8), (1, 2)]:
        check_srste(W, G, dtype, n, m, decay, f"decay {decay} {n}:{m}")


@pytest.mark.parametrize("dtype", DTS)
def test_srste_special_values(dtype):
    """Signed zeros, subnormals, extremes, Inf and NaN in W and G."""
    big = 65504.0 if dtype == "f16" else 3e38
    tiny = 2.0 ** -24 if dtype == "f16" else 2.0 ** -133
    vals = [0.0, -0.0, 1.0, -1.0, big, -big, tiny, -tiny, np.inf, -np.inf, 2.0 ** -14, 7.0]
    rng = np.random.default_rng(11)
    for trial in range(2):
        W = encode(rng.choice(vals, size=(16, 256)), dtype).copy()
        G = encode(rng.choice(vals, size=(16, 256)), dtype).copy()
        as_bits(W).reshape(-1)[5::41] = NAN[dtype]
        as_bits(G).reshape(-1)[3::29] = NAN[dtype]
        for n, m in [(2, 4), (1, 2), (4, 8), (3, 8)]:
            for decay in (2e-4, 1.0, 1e30):
                check_srste(W, G, dtype, n, m, decay, f"special {n}:{m} decay {decay}")


@pytest.mark.parametrize("dtype", DTS)
def test_srste_subnormal_products(dtype):
    """decay * w and g + p in the fp32 subnormal range: no flush to zero."""
    rng = np.random.default_rng(12)
    scale = 2.0 ** -120 if dtype != "f16" else 2.0 ** -20
    W = encode(rng.standard_normal((32, 128)) * scale, dtype)
    G = encode(rng.standard_normal((32, 128)) * scale * 2.0 ** -10, dtype)
    check_srste(W, G, dtype, 2, 4, 2.0 ** -10, "subnormal")


@pytest.mark.parametrize("dtype", DTS)
def test_srste_in_place(dtype):
    rng = np.random.default_rng(13)
    R, K = 37, 520
    W = tie_heavy(rng, (R, K), dtype)
    G = gradient(rng, (R, K), dtype)
    Wd, Gd = dev(W, dtype), dev(G, dtype)
    out = nm.srste_grad(Wd, Gd, 2, 4, 2e-4, out=Gd)
    assert out.data_ptr() == Gd.data_ptr()
    assert_same_bits(host_bits(Gd), oracle.srste_grad(W, G, dtype, 2, 4, 2e-4), dtype, "grad in place")
    nm.prune(Wd, 2, 4, out=Wd)
    assert_same_bits(host_bits(Wd), oracle.prune(W, dtype, 2, 4), dtype, "prune in place")


def test_srste_empty():
    for R, K in [(0, 128), (16, 0)]:
        W = torch.zeros((R, K), dtype=torch.bfloat16, device="cuda")
        assert nm.prune(W, 2, 4).shape == (R, K)
        assert nm.srste_grad(W, W.clone(), 2, 4).shape == (R, K)


def test_srste_default_decay_is_the_pages():
    rng = np.random.default_rng(14)
    W = encode(rng.standard_normal((16, 64)), "f32")
    G = gradient(rng, (16, 64), "f32")
    got = host_bits(nm.srste_grad(dev(W, "f32"), dev(G, "f32"), 2, 4))
    assert_same_bits(got, oracle.srste_grad(W, G, "f32", 2, 4, 0.0002), "f32", "default decay")


@pytest.mark.parametrize("name", ["toy_f32", "bert_ffn", "resnet_conv3x3", "llama_up", "llama_down",
                                  "sweep_f16"])
def test_srste_full_workloads(name):
    """Whole weight matrices at their real shapes, every element against the oracle."""
    w = synth.WORKLOADS[name]
    W, G = w.W(), w.G()
    Wd, Gd = dev(W, w.dtype), dev(G, w.dtype)
    for n, m in w.patterns:
        print(f"[srste] {name} {w.R}x{w.K} {n}:{m}", flush=True)
        assert_same_bits(host_bits(nm.prune(Wd, n, m)), oracle.prune(W, w.dtype, n, m), w.dtype,
                         f"prune {name} {n}:{m}")
        assert_same_bits(host_bits(nm.srste_grad(Wd, Gd, n, m)),
                         oracle.srste_grad(W, G, w.dtype, n, m, nm.SRSTE_DECAY), w.dtype,
                         f"grad {name} {n}:{m}")
