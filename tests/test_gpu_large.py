"""Sizes past 32-bit element and byte offsets, checked on samples against the oracle.

The inputs are seeded synthetic blocks tiled on the GPU (torch.repeat), so the oracle
only needs the base block: a tiled W compresses to tiled rows, and a product with a tiled
X has its column t equal to column t mod T0 of the product with the base block.
  * the fused mask + compress pass over W with R*K > 2^31 elements (4.3 GB of bf16);
  * the product with X of 2^31 bytes (8192 x 131072 bf16), sampled up to the last column.
"""
import numpy as np
import pytest
import torch

import masking_sparse_gemm_amd as nm
import oracle
import synth
from tests.helpers import as_bits
from tests.test_gpu_parity import host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nm.lib()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def bf16_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def test_mask_compress_past_2_pow_31_elements():
    R0, K, reps = 1024, 8192, 264  # R = 270336 rows: R * K = 2.21e9 elements
    base = synth.generate(synth.Dist("normal", 0, 0.02), (R0, K), "bf16")
    R = R0 * reps
    assert R * K > 2**31
    W = bf16_dev(base).repeat(reps, 1)
    print(f"[large] mask_compress {R}x{K}", flush=True)
    mask, v, mt = nm.mask_compress(W, 2, 4)
    torch.cuda.synchronize()
    del W
    vals_o, meta_o = oracle.compress(base, "bf16", 2, 4)
    mask_o = oracle.mask(base, "bf16", 2, 4)
    rows = [0, R0 - 1, R0 * 131 + 7, R - R0 + 100, R - 1]
    for r in rows:
        b = r % R0
        assert np.array_equal(host_bits(v[r]), as_bits(vals_o[b])), f"values row {r}"
        assert np.array_equal(mt[r].cpu().numpy().view(np.uint32), meta_o[b]), f"meta row {r}"
        assert np.array_equal(mask[r].cpu().numpy().astype(np.uint8), mask_o[b]), f"mask row {r}"
    del mask, v, mt
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layout", ["blocked", "rows"])
def test_product_with_2_pow_31_bytes_of_x(layout):
    R, K, T0, reps = 256, 8192, 1024, 128  # X: 8192 x 131072 bf16 = 2 GiB
    Wb = synth.generate(synth.Dist("normal", 0, 0.02), (R, K), "bf16")
    Xb = synth.generate(synth.Dist("normal", 1), (K, T0), "bf16")
    T = T0 * reps
    assert K * T * 2 >= 2**31
    X = bf16_dev(Xb).repeat(1, reps)
    v, mt = nm.compress(bf16_dev(Wb), 2, 4, layout=layout)
    print(f"[large] spmm {R}x{K} x {K}x{T} {layout}", flush=True)
    Y = nm.spmm(v, mt, X, 2, 4, layout=layout, rows=R)
    torch.cuda.synchronize()
    del X
    vals_o, meta_o = oracle.compress(Wb, "bf16", 2, 4)
    rng = np.random.default_rng(8)
    rs = np.concatenate([rng.integers(0, R, 300), [R - 1, 0, R - 1]])
    ts = np.concatenate([rng.integers(0, T, 300), [T - 1, T - 1, T0 * 77 + 5]])
    want = oracle.spmm_sample(vals_o, meta_o, R, K, 2, 4, Xb, "bf16", rs, ts % T0)
    got = Y[torch.from_numpy(rs).cuda(), torch.from_numpy(ts).cuda()].float().cpu().double().numpy()
    s = oracle.spmm_sample(as_bits(vals_o) & np.uint16(0x7FFF), meta_o, R, K, 2, 4,
                           as_bits(Xb) & np.uint16(0x7FFF), "bf16", rs, ts % T0)
    bound = 2.0 * (K // 2) * 2.0**-24 * s + 2.0**-8 * (np.abs(want) + np.abs(got)) + 1e-37
    bad = np.abs(got - want) > bound
    assert not bad.any(), f"{int(bad.sum())} samples off, first at {np.argwhere(bad)[0]}"
    del Y
    torch.cuda.empty_cache()
