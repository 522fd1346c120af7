"""GPU parity of nm_mask_compress (mask and compressed pair from one pass over W) against
the oracle, bit for bit, in both layouts: the mask equals nm_mask's rule, the pair equals
nm_compress's, for every element type, on ragged shapes (padding rows of the blocked
layout, odd and even step counts) and on a full LLaMA matrix."""
import numpy as np
import pytest
import torch

import masking_sparse_gemm_amd as nm
import oracle
import synth
from tests.helpers import as_bits, blocked_from_rows, encode
from tests.test_gpu_parity import dev, host_bits, tie_heavy

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nm.lib()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def to_dev(W, dtype):
    if dtype == "i8":
        return torch.from_numpy(np.ascontiguousarray(W)).cuda()
    if dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(W)).cuda().view(torch.float8_e4m3fn)
    return dev(W, dtype)


def raw(t):
    if t.dtype in (torch.int8, torch.float8_e4m3fn):
        return t.detach().view(torch.uint8).cpu().numpy()
    return host_bits(t)


def matrix(rng, shape, dtype):
    if dtype == "i8":
        a = rng.integers(-128, 128, size=shape)
        a[rng.random(shape) < 0.3] //= 32
        return a.astype(np.int8)
    if dtype == "fp8":
        a = rng.integers(0, 256, size=shape).astype(np.uint8)
        a[rng.random(shape) < 0.3] &= 0xF8
        return a
    return tie_heavy(rng, shape, dtype)


def check(W, dtype, n, m, layout, label):
    R, K = W.shape
    Wd = to_dev(W, dtype)
    mask, v, mt = nm.mask_compress(Wd, n, m, layout=layout)
    assert np.array_equal(mask.cpu().numpy().astype(np.uint8), oracle.mask(W, dtype, n, m)), \
        f"mask {label}"
    vals_o, meta_o = oracle.compress(W, dtype, n, m)
    vals_o = vals_o if dtype in ("i8", "fp8") else as_bits(vals_o)
    if dtype == "i8":
        vals_o = vals_o.view(np.uint8)
    if layout == "blocked":
        vals_o, meta_o = blocked_from_rows(vals_o, meta_o, R, K, n, m)
    assert np.array_equal(raw(v), vals_o), f"values {label}"
    assert np.array_equal(mt.cpu().numpy().view(np.uint32), meta_o), f"meta {label}"


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32", "i8", "fp8"])
@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (4, 8), (1, 4), (3, 8), (2, 8)])
@pytest.mark.parametrize("layout", ["rows", "blocked"])
def test_mask_compress_shapes(dtype, n, m, layout):
    one_byte = dtype in ("i8", "fp8")
    if layout == "blocked" and one_byte and (16 * n // m) % 4:
        pytest.skip("pattern not stored in the blocked 1-byte layout")
    rng = np.random.default_rng(1400 + 10 * n + m)
    # K = 64 and 192: odd step counts (one block per wave); 128, 256: even (two per wave)
    for R, K in [(7, 128), (33, 64), (20, 192), (16, 256), (45, 128), (5, 24 * m)]:
        if K % m or (layout == "blocked" and K % 64):
            continue
        check(matrix(rng, (R, K), dtype), dtype, n, m, layout, f"{dtype} {R}x{K} {n}:{m} {layout}")


def test_mask_compress_full_llama_blocked():
    w = synth.WORKLOADS["llama_up"]
    W = w.W()
    print(f"[mask_compress] llama_up {w.R}x{w.K}", flush=True)
    check(W, "bf16", 2, 4, "blocked", "llama_up")


def test_mask_compress_empty_and_alias():
    Z = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    mask, v, mt = nm.mask_compress(Z, 2, 4, layout="blocked")
    assert mask.shape == (0, 64)
    L = nm.lib()
    W = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    # the mask written over W: refused before any launch
    rc = L.nm_mask_compress(W.data_ptr(), nm.NM_BF16, 16, 64, 2, 4, 0, W.data_ptr(),
                            buf.data_ptr(), buf.data_ptr() + 8192, None)
    assert nm.STATUS[rc] == "alias"
