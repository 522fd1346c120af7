"""nm_perm_gains_static, the permutation-gains entry point that allocates nothing (its
workspace is the library's static per-device scratch buffer), against nm_perm_gains with a
caller workspace: two calls in a row, the second on a smaller input, each compared entry by
entry (the same kernels run on the same inputs, so the results must be identical, including
the entries the call leaves untouched)."""
import ctypes

import numpy as np
import pytest
import torch

import masking_sparse_gemm_amd as nm
from tests.helpers import encode
from tests.test_gpu_parity import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nm.lib()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def gains_both_ways(W, perm, n, m):
    """(gain, pick) from nm_perm_gains (caller workspace) and from nm_perm_gains_static,
    called on the same stream, both output pairs pre-filled with the same sentinels."""
    L = nm.lib()
    R, K = W.shape
    G = K // m
    dt = nm.NM_BF16
    s = torch.cuda.current_stream().cuda_stream
    outs = []
    for static in (False, True):
        gain = torch.full((G, G), -7.5, dtype=torch.float32, device=W.device)
        pick = torch.full((G, G), -3, dtype=torch.int32, device=W.device)
        if static:
            rc = L.nm_perm_gains_static(W.data_ptr(), dt, R, K, n, m, perm.data_ptr(),
                                        gain.data_ptr(), pick.data_ptr(), s)
        else:
            nbytes = int(L.nm_perm_workspace_bytes(R, K, n, m))
            ws = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
            rc = L.nm_perm_gains(W.data_ptr(), dt, R, K, n, m, perm.data_ptr(), gain.data_ptr(),
                                 pick.data_ptr(), ws.data_ptr(), nbytes, s)
        assert nm.STATUS[rc] == "ok", (static, nm.STATUS[rc])
        torch.cuda.synchronize()
        outs.append((gain.cpu().numpy(), pick.cpu().numpy()))
    return outs


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_static_scratch_gains_match_workspace_gains(n, m):
    rng = np.random.default_rng(1234 + m)
    # the larger case fills 94 % of the static buffer; the second call is smaller
    for R, K in ((3072, 5120), (200, 328)):
        print(f"perm_gains_static bf16 {n}:{m} R={R} K={K}", flush=True)
        W = dev(encode(rng.standard_normal((R, K)), "bf16"), "bf16")
        perm = torch.from_numpy(rng.permutation(K).astype(np.int32)).cuda()
        (g_ref, p_ref), (g, p) = gains_both_ways(W, perm, n, m)
        assert np.array_equal(g.view(np.uint32), g_ref.view(np.uint32))
        assert np.array_equal(p, p_ref)
        G = K // m
        iu = np.triu_indices(G, 1)
        assert (g[iu] != -7.5).all()          # every pair g1 < g2 was written
        assert (g[np.tril_indices(G)] == -7.5).all()   # the rest left as it was


def test_static_scratch_rejects_beyond_its_size():
    """R*K*4 above NM_STATIC_SCRATCH_BYTES is refused before any launch."""
    L = nm.lib()
    R, K = 4097, 4096
    W = torch.zeros(16, dtype=torch.bfloat16, device="cuda")   # never read: rejected first
    perm = torch.zeros(16, dtype=torch.int32, device="cuda")
    out = torch.zeros(16, dtype=torch.float32, device="cuda")
    rc = L.nm_perm_gains_static(W.data_ptr(), nm.NM_BF16, R, K, 2, 4, perm.data_ptr(),
                                out.data_ptr(), out.data_ptr(), None)
    assert nm.STATUS[rc] == "scratch"
