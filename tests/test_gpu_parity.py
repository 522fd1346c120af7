"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on the
same seeded inputs.

Masks, stored values, metadata and decompressed weights must match bit for bit.
Products are checked two ways:
  * the stated tolerance, max|Y - Y_ref| / max|Y_ref| <= 2e-2 for 16-bit inputs
    and <= 1e-5 for fp32 inputs (fp32 accumulation in both cases);
  * an element-wise bound from the arithmetic: products of two bf16/fp16 (or
    fp32 pairs in the reference) are exact, so an fp32 sum of k terms in any order
    is off by at most about k * 2^-24 * sum|w_i x_i|; we allow 2 k 2^-24 (room for
    truncating adders), plus half an ulp of the output type for the final rounding.
    A single dropped or doubled term breaks this bound.
"""
import os

import numpy as np
import pytest
import torch

import masking_sparse_gemm_amd as nm
import oracle
import synth
from tests.helpers import as_bits, blocked_from_rows, encode, normwise_rel_err

pytestmark = pytest.mark.gpu

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ULP_HALF = {"f32": 2.0**-24, "f16": 2.0**-11, "bf16": 2.0**-8}
TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nm.lib()  # fails loudly if the library is not built
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(TORCH_DT[dtype])
    return t.cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32)
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def abs_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    b = as_bits(a)
    return b & (np.uint32(0x7FFFFFFF) if dtype == "f32" else np.uint16(0x7FFF))


def check_select(W: np.ndarray, dtype: str, n: int, m: int, label: str = ""):
    """mask / compress / decompress of W on the GPU == oracle, bitwise."""
    R, K = W.shape
    Wd = dev(W, dtype)
    vals_o, meta_o = oracle.compress(W, dtype, n, m)
    mask_o = oracle.mask(W, dtype, n, m)
    vals, meta = nm.compress(Wd, n, m)
    assert np.array_equal(host_bits(vals), as_bits(vals_o)), f"values {label}"
    assert np.array_equal(host_bits(meta), meta_o), f"meta {label}"
    assert np.array_equal(nm.mask(Wd, n, m).cpu().numpy().astype(np.uint8), mask_o), f"mask {label}"
    dec = nm.decompress(vals, meta, n, m, K)
    dec_o = oracle.decompress(vals_o, meta_o, dtype, R, K, n, m)
    assert np.array_equal(host_bits(dec), as_bits(dec_o)), f"decompress {label}"
    if K % 64 == 0:
        check_select_blocked(W, dtype, n, m, vals_o, meta_o, dec_o, label)
    return vals, meta, vals_o, meta_o


def check_select_blocked(W, dtype, n, m, vals_o, meta_o, dec_o=None, label=""):
    """compress / decompress in the blocked layout == the oracle's arrays regrouped, bitwise."""
    R, K = W.shape
    vb, mb = nm.compress(dev(W, dtype), n, m, layout="blocked")
    vb_o, mb_o = blocked_from_rows(as_bits(vals_o), meta_o, R, K, n, m)
    assert np.array_equal(host_bits(vb), vb_o), f"blocked values {label}"
    assert np.array_equal(host_bits(mb), mb_o), f"blocked meta {label}"
    if dec_o is None:
        dec_o = oracle.decompress(vals_o, meta_o, dtype, R, K, n, m)
    dec = nm.decompress(vb, mb, n, m, K, layout="blocked", rows=R)
    assert np.array_equal(host_bits(dec), as_bits(dec_o)), f"blocked decompress {label}"
    return vb, mb


def compressed(W, dtype, n, m, layout):
    """The checked compressed pair in `layout` and the oracle's (rows) pair."""
    vals, meta, vals_o, meta_o = check_select(W, dtype, n, m)
    if layout == "blocked":
        vals, meta = check_select_blocked(W, dtype, n, m, vals_o, meta_o)
    return vals, meta, vals_o, meta_o


def check_product(Y: torch.Tensor, y_ref: np.ndarray, abs_sum: np.ndarray, kept: int, dtype: str,
                  y_dtype: str, label: str = ""):
    y = host_f64(Y)
    assert normwise_rel_err(y, y_ref) <= TOL[dtype], f"tolerance {label}"
    bound = 2.0 * kept * 2.0**-24 * abs_sum + ULP_HALF[y_dtype] * np.abs(y_ref) + 1e-37
    if y_dtype != "f32":  # the rounded output may also sit half an ulp of itself away
        bound += ULP_HALF[y_dtype] * np.abs(y)
    bad = np.abs(y - y_ref) > bound
    assert not bad.any(), (f"element bound {label}: {int(bad.sum())} entries, first at "
                           f"{np.argwhere(bad)[0].tolist()}")


def reference_product(vals_o, meta_o, R, K, n, m, X, dtype):
    y_ref = oracle.spmm(vals_o, meta_o, R, K, n, m, X, dtype)
    s = oracle.spmm(abs_bits(vals_o, dtype), meta_o, R, K, n, m, abs_bits(X, dtype), dtype)
    return y_ref, s


def tie_heavy(rng, shape, dtype, scale=1.0):
    """Values on a coarse grid (many equal magnitudes), zeros of both signs."""
    a = np.round(rng.standard_normal(shape) * 3) / 3 * scale
    a[rng.random(shape) < 0.05] = -0.0
    return encode(a, dtype)


# ---------------------------------------------------------------------------
# mask / compress / decompress
# ---------------------------------------------------------------------------

SELECT_PATTERNS = [(1, 2), (2, 2), (1, 4), (2, 4), (3, 4), (4, 4), (1, 8), (2, 8), (3, 8), (4, 8),
                   (7, 8), (8, 8)]
SELECT_SHAPES = [(7, 128), (33, 96), (5, 24), (64, 8), (3, 1024), (1, 64 * 8), (33, 192),
                 (17, 64)]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("n,m", SELECT_PATTERNS)
def test_select_small_shapes(dtype, n, m):
    rng = np.random.default_rng(100 + 10 * n + m)
    for R, K in SELECT_SHAPES:
        if K % m:
            continue
        check_select(tie_heavy(rng, (R, K), dtype), dtype, n, m, f"{R}x{K}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_select_special_values(dtype):
    """Signed zeros, all-equal groups, extreme exponents, Inf and NaN: bitwise."""
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0 if dtype == "f16" else 3e38, 2.0**-24 if dtype != "f32"
            else 2.0**-149, np.inf, -np.inf, 2.0**-14, 7.0]
    rng = np.random.default_rng(5)
    a = rng.choice(vals, size=(16, 256))
    a[0, :] = 5.0  # all-equal groups
    a[1, :] = -0.0
    W = encode(a, dtype)
    if dtype == "f32":
        W = a.astype(np.float32)
    W = W.copy()
    flat = as_bits(W).reshape(-1)
    flat[7::37] = 0x7FC00000 if dtype == "f32" else (0x7E00 if dtype == "f16" else 0x7FC0)  # NaN
    for n, m in [(2, 4), (1, 2), (4, 8), (3, 8)]:
        check_select(W, dtype, n, m, f"special {n}:{m}")


@pytest.mark.parametrize("name", ["toy_f32", "bert_ffn", "resnet_conv3x3", "llama_up", "llama_down",
                                  "sweep_f16"])
def test_select_full_workloads(name):
    w = synth.WORKLOADS[name]
    W = w.W()
    for n, m in w.patterns:
        print(f"[select] {name} {w.R}x{w.K} {n}:{m}", flush=True)
        check_select(W, w.dtype, n, m, f"{name} {n}:{m}")


def test_select_empty():
    for R, K in [(0, 128), (16, 0)]:
        W = torch.zeros((R, K), dtype=torch.bfloat16, device="cuda")
        vals, meta = nm.compress(W, 2, 4)
        assert vals.shape == (R, K // 2) and meta.shape == (R, K // 32)
        assert nm.mask(W, 2, 4).shape == (R, K)
        assert nm.decompress(vals, meta, 2, 4, K).shape == (R, K)
        vb, mb = nm.compress(W, 2, 4, layout="blocked")
        assert nm.decompress(vb, mb, 2, 4, K, layout="blocked", rows=R).shape == (R, K)


# ---------------------------------------------------------------------------
# sparse x dense product
# ---------------------------------------------------------------------------

# (R, K, T): several tiles with ragged row and column tails.  16-bit: 2:4 and 1:2 with K a
# multiple of 64 and T of 8 take the structured-sparse kernels, 4:8 the expanded-group one,
# everything else the expansion kernel (K = 96 and 40: a K tail inside its 64-wide step;
# T = 13, 70 and 261: rows of X that are not whole 16-byte pieces, loaded element-wise).
PRODUCT_SHAPES = [(200, 384, 264), (130, 256, 136), (16, 128, 8), (257, 128, 520), (64, 96, 40),
                  (33, 40, 13), (70, 40, 24), (130, 256, 70), (129, 128, 261), (300, 192, 262),
                  (16, 64, 6), (40, 128, 2), (20, 64, 1)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (4, 8), (3, 4), (1, 8), (1, 4), (2, 8), (6, 8),
                                 (2, 2)])
@pytest.mark.parametrize("yf32", [False, True])
@pytest.mark.parametrize("layout", ["rows", "blocked"])
def test_spmm_elementwise(dtype, n, m, yf32, layout):
    rng = np.random.default_rng(7 + n + 3 * m)
    for R, K, T in PRODUCT_SHAPES:
        if K % m or (layout == "blocked" and K % 64):
            continue
        W = encode(rng.standard_normal((R, K)), dtype)
        X = encode(rng.standard_normal((K, T)), dtype)
        vals, meta, vals_o, meta_o = compressed(W, dtype, n, m, layout)
        y_dtype = "f32" if yf32 else dtype
        Y = nm.spmm(vals, meta, dev(X, dtype), n, m, out_dtype=TORCH_DT[y_dtype], layout=layout,
                    rows=R)
        y_ref, s = reference_product(vals_o, meta_o, R, K, n, m, X, dtype)
        check_product(Y, y_ref, s, K // m * n, dtype, y_dtype, f"{R}x{K}x{T} {n}:{m} {layout}")


@pytest.mark.parametrize("dtype,n,m", [("bf16", 2, 4), ("f16", 1, 2), ("bf16", 4, 8)])
@pytest.mark.parametrize("layout", ["rows", "blocked"])
def test_spmm_even_ragged_columns(dtype, n, m, layout):
    """Even T that is not a multiple of 8 (X rows not whole 16-byte pieces): the
    structured-sparse and 4:8 kernels with 4-byte X pieces, over many tiles, against the
    oracle."""
    rng = np.random.default_rng(67)
    R, K, T = 600, 512, 1022
    W = encode(rng.standard_normal((R, K)), dtype)
    X = encode(rng.standard_normal((K, T)), dtype)
    vals, meta, vals_o, meta_o = compressed(W, dtype, n, m, layout)
    Y = nm.spmm(vals, meta, dev(X, dtype), n, m, layout=layout, rows=R)
    y_ref, s = reference_product(vals_o, meta_o, R, K, n, m, X, dtype)
    check_product(Y, y_ref, s, K // m * n, dtype, dtype, f"{R}x{K}x{T} {layout}")


@pytest.mark.parametrize("tile", ["0", "1", "2", "3"])
@pytest.mark.parametrize("dtype,n,m", [("bf16", 2, 4), ("f16", 1, 2), ("f16", 2, 4)])
@pytest.mark.parametrize("layout", ["rows", "blocked"])
def test_spmm_every_tile_shape(tile, dtype, n, m, layout, monkeypatch):
    """Each matrix-core tile shape, pinned, on shapes with ragged row and column tiles.
    Tile 3 is the 256 x 256 kernel split over workgroups by K steps (2:4, blocked layout):
    on these small shapes every workgroup gets one or two steps, so tiles are cut into
    many parts whose partial sums are exchanged through the workspace."""
    monkeypatch.setenv("NM_SPMM_TILE", tile)
    rng = np.random.default_rng(61)
    for R, K, T in [(300, 192, 264), (520, 128, 136), (16, 64, 8), (33, 640, 392)]:
        W = encode(rng.standard_normal((R, K)), dtype)
        X = encode(rng.standard_normal((K, T)), dtype)
        vals, meta, vals_o, meta_o = compressed(W, dtype, n, m, layout)
        Y = nm.spmm(vals, meta, dev(X, dtype), n, m, out_dtype=torch.float32, layout=layout,
                    rows=R)
        y_ref, s = reference_product(vals_o, meta_o, R, K, n, m, X, dtype)
        check_product(Y, y_ref, s, K // m * n, dtype, "f32", f"tile {tile} {R}x{K}x{T} {layout}")


@pytest.mark.parametrize("dtype,ydt", [("bf16", "bf16"), ("f16", "f32")])
def test_spmm_split_kernel_whole_tiles(dtype, ydt, monkeypatch):
    """The 256 x 256 split kernel where every workgroup gets whole tiles in step (256 tiles
    of one or two K steps each, tiles taken in XCD blocks), with ragged edges: every output
    against the oracle."""
    monkeypatch.setenv("NM_SPMM_TILE", "3")
    rng = np.random.default_rng(71)
    for R, K, T in [(4000, 64, 4088), (2048, 128, 8192)]:
        W = encode(rng.standard_normal((R, K)), dtype)
        X = encode(rng.standard_normal((K, T)), dtype)
        vals, meta, vals_o, meta_o = compressed(W, dtype, 2, 4, "blocked")
        Y = nm.spmm(vals, meta, dev(X, dtype), 2, 4, out_dtype=TORCH_DT[ydt], layout="blocked",
                    rows=R)
        y_ref, s = reference_product(vals_o, meta_o, R, K, 2, 4, X, dtype)
        check_product(Y, y_ref, s, K // 2, dtype, ydt, f"split whole tiles {R}x{K}x{T}")


# fp32: the matrix-core expansion kernel for every pattern (K tails inside its 32-wide step:
# K = 200, 72, 8, 40; T = 13 and 261 load X element-wise)
F32_SHAPES = PRODUCT_SHAPES + [(70, 200, 132), (129, 72, 260), (1, 8, 4), (300, 320, 4)]


@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (4, 8), (1, 4), (3, 4), (2, 2), (1, 8), (6, 8),
                                 (8, 8)])
@pytest.mark.parametrize("layout", ["rows", "blocked"])
def test_spmm_f32_elementwise(n, m, layout):
    rng = np.random.default_rng(31)
    for R, K, T in F32_SHAPES:
        if K % m or (layout == "blocked" and K % 64):
            continue
        W = rng.standard_normal((R, K)).astype(np.float32)
        X = rng.standard_normal((K, T)).astype(np.float32)
        vals, meta, vals_o, meta_o = compressed(W, "f32", n, m, layout)
        Y = nm.spmm(vals, meta, dev(X, "f32"), n, m, layout=layout, rows=R)
        y_ref, s = reference_product(vals_o, meta_o, R, K, n, m, X, "f32")
        check_product(Y, y_ref, s, K // m * n, "f32", "f32", f"{R}x{K}x{T} {layout}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("n,m", [(2, 4), (1, 2), (3, 8)])
@pytest.mark.parametrize("layout", ["rows", "blocked"])
def test_spmm_identity_is_exact(dtype, n, m, layout):
    """X = I: every output is one product by 1, so Y equals the masked weight bitwise."""
    rng = np.random.default_rng(41)
    R, K = 72, 256
    W = encode(rng.standard_normal((R, K)), dtype)
    vals, meta = nm.compress(dev(W, dtype), n, m, layout=layout)
    Y = nm.spmm(vals, meta, dev(encode(np.eye(K), dtype), dtype), n, m, layout=layout, rows=R)
    dec = nm.decompress(vals, meta, n, m, K, layout=layout, rows=R)
    assert np.array_equal(host_bits(Y), host_bits(dec))


@pytest.mark.parametrize("layout", ["rows", "blocked"])
def test_spmm_integers_are_exact(layout):
    """Small integers: every partial sum is exact in fp32, so any order gives the oracle's value."""
    rng = np.random.default_rng(43)
    R, K, T = 96, 512, 72
    for dtype in ["bf16", "f16", "f32"]:
        W = encode(rng.integers(-8, 9, (R, K)).astype(np.float64), dtype)
        X = encode(rng.integers(-8, 9, (K, T)).astype(np.float64), dtype)
        vals, meta = nm.compress(dev(W, dtype), 2, 4, layout=layout)
        Y = nm.spmm(vals, meta, dev(X, dtype), 2, 4, out_dtype=torch.float32, layout=layout,
                    rows=R)
        vals_o, meta_o = oracle.compress(W, dtype, 2, 4)
        assert np.array_equal(host_f64(Y), oracle.spmm(vals_o, meta_o, R, K, 2, 4, X, dtype))


def test_spmm_empty():
    v = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    meta = torch.zeros((4, 4), dtype=torch.int32, device="cuda")
    assert nm.spmm(v, meta, torch.zeros((128, 0), dtype=torch.bfloat16, device="cuda")).shape == (4, 0)
    v0 = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    m0 = torch.zeros((0, 4), dtype=torch.int32, device="cuda")
    x = torch.ones((128, 16), dtype=torch.bfloat16, device="cuda")
    assert nm.spmm(v0, m0, x).shape == (0, 16)
    ve = torch.zeros((4, 0), dtype=torch.bfloat16, device="cuda")
    me = torch.zeros((4, 0), dtype=torch.int32, device="cuda")
    y = nm.spmm(ve, me, torch.zeros((0, 10), dtype=torch.bfloat16, device="cuda"))
    assert y.shape == (4, 10) and not y.float().abs().sum().item()
    # blocked: no rows, no columns, and an empty contraction (K = 0)
    vb, mb = nm.compress(torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda"), 2, 4,
                         layout="blocked")
    assert nm.spmm(vb, mb, x, layout="blocked", rows=0).shape == (0, 16)
    vb, mb = nm.compress(torch.ones((20, 128), dtype=torch.bfloat16, device="cuda"), 2, 4,
                         layout="blocked")
    y = nm.spmm(vb, mb, torch.zeros((128, 0), dtype=torch.bfloat16, device="cuda"),
                layout="blocked", rows=20)
    assert y.shape == (20, 0)
    vb, mb = nm.compress(torch.zeros((20, 0), dtype=torch.bfloat16, device="cuda"), 2, 4,
                         layout="blocked")
    y = nm.spmm(vb, mb, torch.zeros((0, 10), dtype=torch.bfloat16, device="cuda"),
                layout="blocked", rows=20)
    assert y.shape == (20, 10) and not y.float().abs().sum().item()


def sample_points(rng, R, T, count=1500):
    """Random outputs, the corners and edges of the matrix (ragged tiles live there), and one
    random output in every 32 x 32 block (the accumulator fragment of one matrix-core
    instruction), so every wave's share of every tile is checked."""
    rs = list(rng.integers(0, R, count)) + [0, R - 1, R - 1, 0] + [R - 1] * 64 + list(rng.integers(0, R, 64))
    ts = list(rng.integers(0, T, count)) + [0, T - 1, 0, T - 1] + list(rng.integers(0, T, 64)) + [T - 1] * 64
    br, bt = np.meshgrid(np.arange(0, R, 32), np.arange(0, T, 32), indexing="ij")
    br = br.reshape(-1) + rng.integers(0, 32, br.size)
    bt = bt.reshape(-1) + rng.integers(0, 32, bt.size)
    keep = (br < R) & (bt < T)
    rs += list(br[keep])
    ts += list(bt[keep])
    return np.array(rs, dtype=np.int64), np.array(ts, dtype=np.int64)


@pytest.mark.parametrize("name", ["toy_f32", "bert_ffn", "resnet_conv3x3", "llama_up", "llama_down",
                                  "sweep_f16", "sweep_f32"])
def test_spmm_full_workloads_sampled(name):
    """Full-size products, launched exactly as the benchmark launches them; the oracle
    computes sampled outputs one by one."""
    w = synth.WORKLOADS[name]
    W, X = w.W(), w.X()
    Xd = dev(X, w.dtype)
    rng = np.random.default_rng(55)
    for n, m in w.patterns:
        vals_o, meta_o = oracle.compress(W, w.dtype, n, m)
        rs, ts = sample_points(rng, w.R, w.T)
        y_ref = oracle.spmm_sample(vals_o, meta_o, w.R, w.K, n, m, X, w.dtype, rs, ts)
        s = oracle.spmm_sample(abs_bits(vals_o, w.dtype), meta_o, w.R, w.K, n, m,
                               abs_bits(X, w.dtype), w.dtype, rs, ts)
        for layout in ["blocked", "rows"]:
            print(f"[spmm] {name} {w.R}x{w.K}x{w.T} {n}:{m} {layout}", flush=True)
            vals, meta = nm.compress(dev(W, w.dtype), n, m, layout=layout)
            if layout == "rows":
                assert np.array_equal(host_bits(vals), as_bits(vals_o))
                assert np.array_equal(host_bits(meta), meta_o)
            else:
                vb_o, mb_o = blocked_from_rows(as_bits(vals_o), meta_o, w.R, w.K, n, m)
                assert np.array_equal(host_bits(vals), vb_o)
                assert np.array_equal(host_bits(meta), mb_o)
            Y = nm.spmm(vals, meta, Xd, n, m, layout=layout, rows=w.R)
            y = Y[torch.from_numpy(rs).cuda(), torch.from_numpy(ts).cuda()]
            check_product(y, y_ref, s, w.K // m * n, w.dtype, w.dtype, f"{name} {n}:{m} {layout}")
            if name == "toy_f32":  # small enough to compare every output
                y_full, s_full = reference_product(vals_o, meta_o, w.R, w.K, n, m, X, w.dtype)
                check_product(Y, y_full, s_full, w.K // m * n, w.dtype, w.dtype, "toy full")


def test_load_path_probe_runs_on_product_inputs():
    """The benchmark's load-path probe (libnm_probe: the product's direct loads alone) runs
    to completion on the product's own inputs, ragged tiles included, and writes nothing
    to them."""
    if not os.path.exists(nm.PROBE_LIB_PATH):
        pytest.skip("libnm_probe.so not built")
    P = nm.probe_lib()
    for i, (R, K, T) in enumerate([(512, 256, 256), (300, 192, 136), (16, 64, 8)]):
        print(f"[load-path probe] {R}x{K}x{T}", flush=True)
        W = synth.generate(synth.Dist("normal", 91 + 2 * i, 0.02), (R, K), "bf16")
        X = synth.generate(synth.Dist("normal", 92 + 2 * i), (K, T), "bf16")
        vals, meta = nm.compress(dev(W, "bf16"), 2, 4, layout="blocked")
        Xd = dev(X, "bf16")
        before = [host_bits(t) for t in (vals, meta, Xd)]
        assert P.nm_probe_load_path(vals.data_ptr(), meta.data_ptr(), Xd.data_ptr(), R, K, T,
                                    None) == 0
        torch.cuda.synchronize()
        for b, t in zip(before, (vals, meta, Xd)):
            assert np.array_equal(b, host_bits(t))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("n,m", [(1, 2), (2, 4), (4, 8), (3, 8)])
def test_decompress_trusts_metadata_later_value_wins(dtype, n, m):
    """Decompress trusts its metadata (include/nm.h): with arbitrary fields, repeated and
    descending positions included, value j of a group goes to its field's position in the
    order j = 0 .. n-1, so a repeated position keeps the later value and unnamed positions
    are +0.  Bitwise against the oracle, which writes them in that order, in both layouts."""
    rng = np.random.default_rng(700 + 10 * n + m)
    R, K = 40, 256  # whole metadata words per row for every pattern here; a ragged row block
    words = K // m * n * {2: 1, 4: 2, 8: 3}[m] // 32
    bits_t = np.uint32 if dtype == "f32" else np.uint16
    vals_o = rng.integers(0, np.iinfo(bits_t).max, size=(R, K // m * n), dtype=np.uint64).astype(bits_t)
    meta_o = rng.integers(0, 1 << 32, size=(R, words), dtype=np.uint64).astype(np.uint32)
    dec_o = oracle.decompress(vals_o, meta_o, dtype, R, K, n, m)
    dec = nm.decompress(dev(vals_o, dtype), torch.from_numpy(meta_o.view(np.int32)).cuda(), n, m, K)
    assert np.array_equal(host_bits(dec), as_bits(dec_o)), "rows"
    vb, mb = blocked_from_rows(vals_o, meta_o, R, K, n, m)
    decb = nm.decompress(dev(vb, dtype), torch.from_numpy(mb.view(np.int32)).cuda(), n, m, K,
                         layout="blocked", rows=R)
    assert np.array_equal(host_bits(decb), as_bits(dec_o)), "blocked"
