"""Host-only checks of the C ABI: it loads, exports what include/nm.h declares,
computes its size helpers, and rejects bad arguments before touching a device.
No kernel is launched here."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import masking_sparse_gemm_amd as nm
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nm.h")

needs_lib = pytest.mark.skipif(not os.path.exists(nm.LIB_PATH), reason="libnm.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nm_[a-z_]+)\s*\(", text)))


def test_header_lists_the_binding_exports():
    assert header_functions() == sorted(nm.EXPORTS)


@needs_lib
def test_library_exports_every_declared_symbol():
    L = nm.lib()
    for name in header_functions():
        assert hasattr(L, name), name
    assert L.nm_abi_version() == nm.ABI_VERSION == 10


@needs_lib
def test_library_has_no_undefined_symbols_of_its_own():
    """Every kernel launch stub and internal function is defined inside libnm.so."""
    out = subprocess.run(["nm", "-D", "--undefined-only", nm.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    names = [l.split()[-1] for l in out.splitlines() if l.strip()]
    own = [s for s in names if s.startswith(("_ZN2nm", "nm_")) or "device_stub" in s]
    assert not own, own


@needs_lib
def test_status_strings():
    for code in range(11):
        s = nm.status_str(code)
        assert s and s != "unknown status"
    assert nm.status_str(99) == "unknown status"


@needs_lib
@pytest.mark.parametrize("K,n,m", [(128, 2, 4), (768, 2, 4), (4096, 1, 2), (4096, 4, 8),
                                    (11008, 2, 4), (8, 4, 8), (12, 2, 4), (40, 2, 4), (0, 2, 4),
                                    (96, 3, 8), (64, 8, 8), (16, 1, 4)])
def test_meta_words_per_row_matches_oracle(K, n, m):
    assert nm.meta_words_per_row(K, n, m) == oracle.meta_words_per_row(K, n, m)


@needs_lib
def test_size_helpers_reject_bad_arguments():
    L = nm.lib()
    assert L.nm_meta_words_per_row(6, 2, 4) == -1
    assert L.nm_meta_words_per_row(16, 2, 16) == -1  # M = 16 is not a GPU pattern
    assert L.nm_meta_words_per_row(16, 0, 4) == -1
    ROWS, BLOCKED = nm.LAYOUTS["rows"], nm.LAYOUTS["blocked"]
    assert L.nm_values_bytes(3072, 768, 2, 4, nm.NM_BF16, ROWS) == 3072 * 384 * 2
    assert L.nm_values_bytes(64, 128, 2, 4, nm.NM_F32, ROWS) == 64 * 64 * 4
    assert L.nm_values_bytes(64, 130, 2, 4, nm.NM_F32, ROWS) == 0
    assert L.nm_values_bytes(64, 128, 2, 4, 7, ROWS) == 0
    assert L.nm_values_bytes(64, 128, 2, 4, nm.NM_BF16, 2) == 0
    # blocked: rows padded to 16, K in steps of 64
    assert L.nm_values_bytes(17, 128, 2, 4, nm.NM_BF16, BLOCKED) == 32 * 64 * 2
    assert L.nm_values_bytes(17, 96, 2, 4, nm.NM_BF16, BLOCKED) == 0
    assert L.nm_meta_bytes(17, 128, 2, 4, ROWS) == 17 * 4 * 4
    assert L.nm_meta_bytes(17, 128, 2, 4, BLOCKED) == 32 * 2 * 8
    assert L.nm_meta_bytes(17, 128, 4, 8, BLOCKED) == 32 * 2 * 12
    assert L.nm_meta_bytes(17, 128, 1, 2, BLOCKED) == 32 * 2 * 4
    assert L.nm_meta_bytes(17, 128, 3, 8, BLOCKED) == 32 * 2 * 9
    assert L.nm_meta_bytes(17, 96, 2, 4, BLOCKED) == 0


FAKE = 0x10000  # aligned, never dereferenced: validation fails before any device access


@needs_lib
@pytest.mark.parametrize("case,expect", [
    (dict(W=0), "null"),
    (dict(out=0), "null"),
    (dict(dt=6), "dtype"),
    (dict(n=3, m=3), "pattern"),
    (dict(n=0), "pattern"),
    (dict(n=5), "pattern"),
    (dict(m=16, n=2), "pattern"),
    (dict(K=130), "shape"),
    (dict(R=-1), "shape"),
    (dict(W=FAKE + 8), "align"),
    (dict(out=FAKE + 4), "align"),
    (dict(layout=2), "layout"),
    (dict(layout=1, K=96), "layout"),
])
def test_mask_compress_argument_errors(case, expect):
    L = nm.lib()
    a = dict(W=FAKE, dt=nm.NM_BF16, R=64, K=128, n=2, m=4, out=FAKE, layout=0)
    a.update(case)
    if "layout" not in case:  # nm_mask has no layout argument
        code = L.nm_mask(a["W"], a["dt"], a["R"], a["K"], a["n"], a["m"], a["out"], None)
        assert nm.STATUS[code] == expect
    code = L.nm_compress(a["W"], a["dt"], a["R"], a["K"], a["n"], a["m"], a["layout"], a["out"],
                         FAKE, None)
    assert nm.STATUS[code] == expect
    code = L.nm_decompress(a["W"], FAKE, a["dt"], a["R"], a["K"], a["n"], a["m"], a["layout"],
                           a["out"], None)
    assert nm.STATUS[code] == expect


@needs_lib
@pytest.mark.parametrize("case,expect", [
    (dict(X=0), "null"),
    (dict(meta=0), "null"),
    (dict(y_dt=nm.NM_F16), "dtype"),   # bf16 in, fp16 out is not offered
    (dict(dt=9), "dtype"),
    (dict(T=-3), "shape"),
    (dict(K=126), "shape"),
    (dict(n=3, m=5), "pattern"),
    (dict(Y=FAKE + 2), "align"),
    (dict(meta=FAKE + 4), "align"),
    (dict(layout=7), "layout"),
    (dict(layout=1, K=96), "layout"),
])
def test_spmm_argument_errors(case, expect):
    L = nm.lib()
    a = dict(values=FAKE, meta=FAKE, R=64, K=128, n=2, m=4, layout=0, X=FAKE, T=32,
             dt=nm.NM_BF16, Y=FAKE, y_dt=nm.NM_BF16)
    a.update(case)
    code = L.nm_spmm(a["values"], a["meta"], a["R"], a["K"], a["n"], a["m"], a["layout"], a["X"],
                     a["T"], a["dt"], a["Y"], a["y_dt"], None)
    assert nm.STATUS[code] == expect


@needs_lib
def test_empty_arrays_may_be_null():
    L = nm.lib()
    assert L.nm_mask(None, nm.NM_BF16, 0, 128, 2, 4, None, None) == 0
    for layout in (0, 1):
        assert L.nm_compress(None, nm.NM_F16, 16, 0, 2, 4, layout, None, None, None) == 0
        assert L.nm_compress(None, nm.NM_F16, 0, 64, 2, 4, layout, None, None, None) == 0
        assert L.nm_spmm(FAKE, FAKE, 8, 128, 2, 4, layout, FAKE, 0, nm.NM_BF16, None, nm.NM_BF16,
                         None) == 0


@needs_lib
@pytest.mark.parametrize("case,expect", [
    (dict(W=0), "null"),
    (dict(G=0), "null"),
    (dict(out=0), "null"),
    (dict(dt=4), "dtype"),
    (dict(n=0), "pattern"),
    (dict(m=16, n=2), "pattern"),
    (dict(K=130), "shape"),
    (dict(R=-2), "shape"),
    (dict(W=FAKE + 8, out=FAKE + 0x100000), "align"),
    (dict(G=FAKE + 2), "align"),
    (dict(out=FAKE + 0x100008), "align"),
    (dict(out=FAKE), "alias"),                     # G_out on top of W
    (dict(out=FAKE + 0x2000), "alias"),            # G_out overlapping W's second half
    # G_out just past W does not overlap it: the alias check passes and the
    # (later) alignment check of G reports instead
    (dict(out=FAKE + 0x4000, G=FAKE + 0x80002), "align"),
    (dict(out=FAKE + 0x80000 + 64), "alias"),      # G_out partly over G
])
def test_srste_argument_errors(case, expect):
    """W at FAKE (64 x 128 bf16 = 16 KiB), G at FAKE + 512 KiB, G_out at FAKE + 1 MiB."""
    L = nm.lib()
    a = dict(W=FAKE, G=FAKE + 0x80000, out=FAKE + 0x100000, dt=nm.NM_BF16, R=64, K=128, n=2, m=4)
    a.update(case)
    code = L.nm_srste_grad(a["W"], a["G"], a["dt"], a["R"], a["K"], a["n"], a["m"], 2e-4,
                           a["out"], None)
    assert nm.STATUS[code] == expect


@needs_lib
@pytest.mark.parametrize("case,expect", [
    (dict(W=0), "null"),
    (dict(out=0), "null"),
    (dict(dt=3), "dtype"),
    (dict(n=9, m=8), "pattern"),
    (dict(K=6), "shape"),
    (dict(W=FAKE + 4), "align"),
    (dict(out=FAKE + 0x2000), "alias"),            # half way into W
])
def test_prune_argument_errors(case, expect):
    L = nm.lib()
    a = dict(W=FAKE, out=FAKE + 0x100000, dt=nm.NM_F16, R=64, K=128, n=2, m=4)
    a.update(case)
    code = L.nm_prune(a["W"], a["dt"], a["R"], a["K"], a["n"], a["m"], a["out"], None)
    assert nm.STATUS[code] == expect


@needs_lib
@pytest.mark.parametrize("case,expect", [
    (dict(W=0), "null"),
    (dict(out=0), "null"),
    (dict(dt=6), "dtype"),
    (dict(n=3, m=6), "pattern"),
    (dict(R=62), "shape"),                           # R % m != 0
    (dict(K=66, m=4), "shape"),
    (dict(W=FAKE + 8), "align"),
    (dict(out=FAKE + 0x100004), "align"),
])
def test_tmask_tprune_argument_errors(case, expect):
    L = nm.lib()
    a = dict(W=FAKE, out=FAKE + 0x100000, dt=nm.NM_BF16, R=64, K=128, n=2, m=4)
    a.update(case)
    for fn in (L.nm_tmask, L.nm_tprune):
        code = fn(a["W"], a["dt"], a["R"], a["K"], a["n"], a["m"], a["out"], None)
        assert nm.STATUS[code] == expect, fn.__name__


@needs_lib
def test_tmask_tprune_aliasing():
    L = nm.lib()
    # W: 64 x 128 bf16 = 16 KiB at FAKE; the mask is 8 KiB
    assert nm.STATUS[L.nm_tmask(FAKE, nm.NM_BF16, 64, 128, 2, 4, FAKE + 0x3000, None)] == "alias"
    # a mask ending exactly where W starts does not overlap it: the (later) alignment
    # check of a misaligned W reports instead
    assert nm.STATUS[L.nm_tmask(FAKE + 0x2008, nm.NM_BF16, 64, 128, 2, 4, FAKE + 8, None)] == "align"
    assert nm.STATUS[L.nm_tprune(FAKE, nm.NM_BF16, 64, 128, 2, 4, FAKE + 0x10, None)] == "alias"


@needs_lib
@pytest.mark.parametrize("case,expect", [
    (dict(W=0), "null"),
    (dict(values=0), "null"),
    (dict(dt=3), "dtype"),
    (dict(R=66), "shape"),                           # groups run along R
    (dict(layout=1, R=96), "layout"),                # blocked needs R % 64 == 0
    (dict(layout=1, K=100), "align"),                # K is free: reaches the alignment check
    (dict(values=FAKE + 0x1000), "alias"),
    (dict(meta=FAKE), "alias"),
    (dict(meta=FAKE + 0x200004), "align"),
])
def test_compress_t_argument_errors(case, expect):
    L = nm.lib()
    a = dict(W=FAKE, values=FAKE + 0x100000, meta=FAKE + 0x200000, dt=nm.NM_BF16, R=64, K=128,
             n=2, m=4, layout=0)
    a.update(case)
    if case == dict(layout=1, K=100):
        a["W"] = FAKE + 8
    code = L.nm_compress_t(a["W"], a["dt"], a["R"], a["K"], a["n"], a["m"], a["layout"],
                           a["values"], a["meta"], None)
    assert nm.STATUS[code] == expect


@needs_lib
def test_int8_argument_rules():
    L = nm.lib()
    I8, I32, BF16, ROWS, BLOCKED = nm.NM_I8, nm.NM_I32, nm.NM_BF16, 0, 1
    assert L.nm_values_bytes(64, 128, 2, 4, I8, ROWS) == 64 * 64
    assert L.nm_values_bytes(64, 128, 1, 8, I8, BLOCKED) == 0       # 2 bytes per lane share
    assert L.nm_values_bytes(64, 128, 2, 8, I8, BLOCKED) == 64 * 32
    st = lambda code: nm.STATUS[code]
    # products: int8 in, int32 out, and nothing else mixes with int8
    spmm = lambda dt, ydt, K=128, layout=ROWS, n=2, m=4: L.nm_spmm(
        FAKE, FAKE, 64, K, n, m, layout, FAKE, 32, dt, FAKE + 0x100000, ydt, None)
    assert st(spmm(I8, nm.NM_F32)) == "dtype"
    assert st(spmm(I8, I8)) == "dtype"
    assert st(spmm(BF16, I32)) == "dtype"
    assert st(spmm(I8, I32, K=1 << 17)) == "shape"
    assert st(spmm(I8, I32, layout=BLOCKED, n=3, m=8)) == "unsupported"
    assert st(L.nm_compress(FAKE, I8, 64, 128, 1, 8, BLOCKED, FAKE, FAKE, None)) == "unsupported"
    assert st(L.nm_decompress(FAKE, FAKE, I8, 64, 128, 5, 8, BLOCKED, FAKE, None)) == "unsupported"
    # the training-side calls need floating-point weights
    assert st(L.nm_tmask(FAKE, I8, 64, 128, 2, 4, FAKE + 0x100000, None)) == "dtype"
    assert st(L.nm_prune(FAKE, I8, 64, 128, 2, 4, FAKE + 0x100000, None)) == "dtype"
    assert st(L.nm_mask(FAKE, I32, 64, 128, 2, 4, FAKE + 0x100000, None)) == "dtype"


@needs_lib
def test_fp8_argument_rules():
    L = nm.lib()
    F8, ROWS, BLOCKED = nm.NM_FP8, 0, 1
    st = lambda code: nm.STATUS[code]
    assert L.nm_values_bytes(64, 128, 2, 4, F8, ROWS) == 64 * 64
    assert L.nm_values_bytes(64, 128, 1, 8, F8, BLOCKED) == 0
    assert L.nm_values_bytes(64, 128, 4, 8, F8, BLOCKED) == 64 * 64
    spmm = lambda ydt, layout=ROWS, n=2, m=4: L.nm_spmm(
        FAKE, FAKE, 64, 128, n, m, layout, FAKE, 32, F8, FAKE + 0x100000, ydt, None)
    assert st(spmm(F8)) == "dtype"            # fp8 products come out in fp32 or bf16
    assert st(spmm(nm.NM_F16)) == "dtype"
    assert st(spmm(nm.NM_I32)) == "dtype"
    assert st(spmm(nm.NM_F32, layout=BLOCKED, n=3, m=8)) == "unsupported"
    assert st(L.nm_compress(FAKE, F8, 64, 128, 1, 8, BLOCKED, FAKE, FAKE, None)) == "unsupported"
    for call in (L.nm_tmask, L.nm_prune, L.nm_tprune):
        assert st(call(FAKE, F8, 64, 128, 2, 4, FAKE + 0x100000, None)) == "dtype"
    assert st(L.nm_mask(FAKE, F8, 64, 130, 2, 4, FAKE + 0x100000, None)) == "shape"


@needs_lib
def test_perm_argument_rules():
    L = nm.lib()
    st = lambda code: nm.STATUS[code]
    need = L.nm_perm_workspace_bytes(64, 128, 2, 4)
    assert need >= 64 * 128 * 4 + 128 * 4 + 2 * 32 * 32 * 4
    assert L.nm_perm_workspace_bytes(64, 130, 2, 4) == 0
    gains = lambda **kw: L.nm_perm_gains(kw.get("W", FAKE), kw.get("dt", nm.NM_BF16), 64,
                                         kw.get("K", 128), 2, 4, FAKE, FAKE, FAKE,
                                         kw.get("ws", FAKE + 0x100000), kw.get("wsb", need), None)
    assert st(gains(ws=0)) == "null"
    assert st(gains(wsb=need - 1)) == "shape"
    assert st(gains(dt=nm.NM_I32)) == "dtype"
    assert st(gains(K=126)) == "shape"
    assert st(gains(W=FAKE + 2)) == "align"
    perm = (ctypes.c_int32 * 128)(*range(128))
    perm[5] = 7  # 7 twice: not a permutation
    assert st(L.nm_perm_search(FAKE, nm.NM_BF16, 64, 128, 2, 4, 10, perm, None, FAKE, need,
                               None)) == "shape"
    perm[5] = 5
    assert st(L.nm_perm_search(FAKE, nm.NM_BF16, 64, 128, 2, 4, -1, perm, None, FAKE, need,
                               None)) == "shape"


@needs_lib
def test_srste_empty_arrays_may_be_null():
    L = nm.lib()
    assert L.nm_prune(None, nm.NM_BF16, 0, 128, 2, 4, None, None) == 0
    assert L.nm_srste_grad(None, None, nm.NM_F32, 16, 0, 2, 4, 2e-4, None, None) == 0


def test_binding_shapes_follow_the_layout_definition():
    """compressed_shapes() agrees with the header's byte counts (no GPU needed)."""
    if not os.path.exists(nm.LIB_PATH):
        pytest.skip("libnm.so not built")
    for R, K, n, m in [(17, 128, 2, 4), (300, 256, 4, 8), (16, 64, 1, 2), (5, 192, 3, 8)]:
        (G, S, r16, V), (G2, S2, words) = nm.compressed_shapes(R, K, n, m, "blocked")
        assert (G, S, r16, V) == ((R + 15) // 16, K // 64, 16, 64 // m * n) and (G2, S2) == (G, S)
        b = {2: 1, 4: 2, 8: 3}[m]
        assert 4 * words == 16 * V * b // 8


def test_product_path_does_not_load_the_oracle():
    """Importing and using the binding never pulls in the CPU oracle."""
    code = ("import sys, masking_sparse_gemm_amd as nm; "
            "assert not any(k == 'oracle' or k.startswith('oracle.') for k in sys.modules); "
            "print('clean')")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert out.returncode == 0 and "clean" in out.stdout, out.stderr


def test_binding_has_no_cpu_fallback():
    src = open(os.path.join(ROOT, "masking_sparse_gemm_amd", "__init__.py")).read()
    assert "import oracle" not in src and "from oracle" not in src
    for f in os.listdir(os.path.join(ROOT, "masking_sparse_gemm_amd", "csrc")):
        text = open(os.path.join(ROOT, "masking_sparse_gemm_amd", "csrc", f)).read()
        assert "nm_oracle" not in text and "nmo_" not in text, f


@needs_lib
def test_mask_compress_argument_rules():
    L = nm.lib()
    st = lambda code: nm.STATUS[code]
    mc = lambda **kw: L.nm_mask_compress(
        kw.get("W", FAKE), kw.get("dt", nm.NM_BF16), kw.get("R", 64), kw.get("K", 128), 2, 4,
        kw.get("layout", 0), kw.get("mask", FAKE + 0x100000), kw.get("values", FAKE + 0x200000),
        kw.get("meta", FAKE + 0x300000), None)
    assert st(mc(dt=6)) == "dtype"
    assert st(mc(K=130)) == "shape"
    assert st(mc(layout=1, K=96)) == "layout"
    assert st(mc(mask=0)) == "null"
    assert st(mc(values=FAKE + 0x200008)) == "align"
    assert st(mc(mask=FAKE)) == "alias"                       # the mask over W
    assert st(mc(values=FAKE + 0x100000 + 64 * 64)) == "alias"  # values inside the mask
    assert st(mc(meta=FAKE + 0x200000 + 16)) == "alias"       # meta inside the values
    assert st(mc(R=0)) == "ok"


@needs_lib
def test_outputs_overlapping_inputs_are_rejected():
    """nm_mask, nm_compress, nm_decompress and nm_spmm refuse an output that overlaps an input
    (other workgroups would still be reading it); disjoint arrays pass every check and reach
    the device check, which fails on a host without a GPU."""
    L = nm.lib()
    MB = 0x100000
    R, K, T = 64, 128, 32   # bf16: W 16 KiB, mask 8 KiB, values 8 KiB, meta 1 KiB, X 8 KiB, Y 4 KiB
    BF = nm.NM_BF16
    st = lambda c: nm.STATUS[c]
    no_alias = {"device"}   # what a disjoint call returns here
    # nm_mask: the mask over W
    assert st(L.nm_mask(FAKE, BF, R, K, 2, 4, FAKE + 0x3000, None)) == "alias"
    assert st(L.nm_mask(FAKE, BF, R, K, 2, 4, FAKE + MB, None)) in no_alias
    for layout in (0, 1):
        # nm_compress: values or meta over W, or over each other
        comp = lambda W, v, mt: st(L.nm_compress(W, BF, R, K, 2, 4, layout, v, mt, None))
        assert comp(FAKE, FAKE + 0x1000, FAKE + 2 * MB) == "alias"
        assert comp(FAKE, FAKE + MB, FAKE + 0x3f00) == "alias"
        assert comp(FAKE, FAKE + MB, FAKE + MB + 0x1000) == "alias"
        assert comp(FAKE, FAKE + MB, FAKE + 2 * MB) in no_alias
        # nm_decompress: W_out over values or over meta
        dec = lambda v, mt, W: st(L.nm_decompress(v, mt, BF, R, K, 2, 4, layout, W, None))
        assert dec(FAKE, FAKE + MB, FAKE + 0x1000) == "alias"
        assert dec(FAKE, FAKE + MB, FAKE + MB - 0x2000) == "alias"
        assert dec(FAKE, FAKE + MB, FAKE + 2 * MB) in no_alias
        # nm_spmm: Y over X, values or meta
        sp = lambda v, mt, X, Y: st(L.nm_spmm(v, mt, R, K, 2, 4, layout, X, T, BF, Y, BF, None))
        assert sp(FAKE, FAKE + MB, FAKE + 2 * MB, FAKE + 2 * MB + 0x1ff0) == "alias"
        assert sp(FAKE, FAKE + MB, FAKE + 2 * MB, FAKE + 0x1000) == "alias"
        assert sp(FAKE, FAKE + MB, FAKE + 2 * MB, FAKE + MB + 0x100) == "alias"
        assert sp(FAKE, FAKE + MB, FAKE + 2 * MB, FAKE + 3 * MB) in no_alias
        # Y ending exactly where X starts does not overlap it
        assert sp(FAKE, FAKE + MB, FAKE + 2 * MB, FAKE + 2 * MB - 0x1000) in no_alias
    # fp32 output: Y is twice as large
    assert st(L.nm_spmm(FAKE, FAKE + MB, R, K, 2, 4, 0, FAKE + 2 * MB, T, BF,
                        FAKE + 2 * MB - 0x1000, nm.NM_F32, None)) == "alias"


@needs_lib
def test_perm_gains_static_checks_its_scratch_limit():
    """nm_perm_gains_static needs R*K*4 bytes of the 64 MiB static scratch buffer: one element
    more than fits returns NM_ERR_SCRATCH before any device access; a call that fits passes
    every host check and reaches the device check, which fails on a host without a GPU."""
    L = nm.lib()
    st = lambda c: nm.STATUS[c]
    BF = nm.NM_BF16
    limit = nm.STATIC_SCRATCH_BYTES // 4          # fp32 elements of the permuted copy
    K = 4096
    R_fit = limit // K                            # 4096 x 4096 fills the buffer exactly
    args = lambda R: (FAKE, BF, R, K, 2, 4, FAKE + 0x4000000 * 3, FAKE + 0x4000000 * 4,
                      FAKE + 0x4000000 * 5, None)
    assert st(L.nm_perm_gains_static(*args(R_fit + 1))) == "scratch"
    assert st(L.nm_perm_gains_static(*args(R_fit))) == "device"
    assert st(L.nm_perm_gains_static(FAKE, BF, 64, 130, 2, 4, FAKE, FAKE, FAKE, None)) == "shape"
    assert st(L.nm_perm_gains_static(None, BF, 64, 128, 2, 4, FAKE, FAKE, FAKE, None)) == "null"
    assert st(L.nm_perm_gains_static(FAKE, BF, 64, 128, 2, 4, None, FAKE, FAKE, None)) == "null"
    assert st(L.nm_perm_gains_static(FAKE, nm.NM_I32, 64, 128, 2, 4, FAKE, FAKE, FAKE,
                                     None)) == "dtype"
    assert st(L.nm_perm_gains_static(FAKE + 8, BF, 64, 128, 2, 4, FAKE, FAKE, FAKE,
                                     None)) == "align"
    # empty inputs and a single group are no-ops that touch nothing
    assert st(L.nm_perm_gains_static(None, BF, 0, 128, 2, 4, FAKE, FAKE, FAKE, None)) == "ok"
    assert st(L.nm_perm_gains_static(FAKE, BF, 64, 4, 2, 4, FAKE, FAKE, FAKE, None)) == "ok"


@needs_lib
def test_shape_limit_is_2_pow_36_elements():
    """Below 2^36 elements every launch of the element-wise passes fits the 2^32 work-items
    of one dispatch; R*K = 2^36 is refused before any device access, one row less passes
    every host check (and stops at the device check on a host without a GPU)."""
    L = nm.lib()
    st = lambda c: nm.STATUS[c]
    K = 1 << 20
    R = (1 << 36) // K
    assert st(L.nm_mask(FAKE, nm.NM_BF16, R, K, 2, 4, FAKE + (1 << 40), None)) == "shape"
    assert st(L.nm_mask(FAKE, nm.NM_BF16, R - 1, K, 2, 4, FAKE + (1 << 40), None)) == "device"
    assert st(L.nm_mask(FAKE, nm.NM_BF16, 3, ((1 << 36) + 2) // 3, 2, 2, FAKE + (1 << 40), None)) == "shape"
    assert L.nm_values_bytes(R, K, 2, 4, nm.NM_BF16, 0) == 0
    assert L.nm_values_bytes(R - 1, K, 2, 4, nm.NM_BF16, 0) == (R - 1) * K // 2 * 2


@needs_lib
def test_out_of_range_enum_values_are_rejected():
    """Unknown dtype, layout and status values are ordinary ints to the library (its
    enumerations have int as their underlying type), refused by the checks."""
    L = nm.lib()
    assert nm.STATUS[L.nm_mask(FAKE, 99, 64, 128, 2, 4, FAKE + (1 << 30), None)] == "dtype"
    assert nm.STATUS[L.nm_mask(FAKE, -1, 64, 128, 2, 4, FAKE + (1 << 30), None)] == "dtype"
    assert L.nm_values_bytes(64, 128, 2, 4, nm.NM_BF16, 7) == 0
    assert nm.status_str(-5) == "unknown status" and nm.status_str(1 << 30) == "unknown status"


@pytest.mark.skipif(not os.path.exists(nm.PROBE_LIB_PATH), reason="libnm_probe.so not built")
def test_probe_library_exports_every_declared_symbol():
    """libnm_probe.so (the benchmark's rate probes) exports what include/nm_probe.h declares
    and rejects bad arguments before any launch."""
    text = open(os.path.join(os.path.dirname(HEADER), "nm_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(nm_[a-z_]+)\s*\(", text)))
    assert names == ["nm_probe_copy", "nm_probe_load_path", "nm_probe_matrix_core",
                     "nm_probe_operand_bytes", "nm_probe_valu"]
    P = nm.probe_lib()
    for name in names:
        assert hasattr(P, name), name
    assert P.nm_probe_operand_bytes() == 4 * 64 * 24 * 2
    assert P.nm_probe_matrix_core(2, FAKE, 256, 2, 10, FAKE, FAKE, None) == 1
    assert P.nm_probe_valu(3, 256, 2, 10, FAKE, FAKE, None) == 1
    assert P.nm_probe_valu(0, 256, 9, 10, FAKE, FAKE, None) == 1
    assert P.nm_probe_copy(FAKE, FAKE + 4096, 24, None) == 1      # not a multiple of 16
    assert P.nm_probe_copy(FAKE + 8, FAKE + 4096, 32, None) == 1  # misaligned
    # the load-path probe: shapes the product's 256 x 128 loads take, 16-byte alignment
    assert P.nm_probe_load_path(FAKE, FAKE, FAKE, 256, 100, 128, None) == 1  # K % 64
    assert P.nm_probe_load_path(FAKE, FAKE, FAKE, 256, 128, 12, None) == 1   # T % 8
    assert P.nm_probe_load_path(FAKE, FAKE, FAKE, 0, 128, 128, None) == 1    # empty
    assert P.nm_probe_load_path(FAKE + 4, FAKE, FAKE, 256, 128, 128, None) == 1
    assert P.nm_probe_load_path(None, FAKE, FAKE, 256, 128, 128, None) == 1
    assert P.nm_probe_load_path(FAKE, FAKE, FAKE, 1 << 28, 128, 128, None) == 1
