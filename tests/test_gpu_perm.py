"""GPU parity of the channel-permutation search (nm_perm_gains, nm_perm_search)
against the oracle.

Inputs are multiples of 1/16 with small integer parts, so every magnitude sum the
search forms is exact in fp32 (the library) and in double (the oracle): gains must
be equal, picks identical and the searched permutations the same.
"""
import numpy as np
import pytest
import torch

import masking_sparse_gemm_amd as nm
import oracle
from tests.helpers import as_bits, encode
from tests.test_gpu_parity import dev, host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nm.lib()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def exact_matrix(rng, shape, dt):
    a = np.round(rng.standard_normal(shape) * 24) / 16
    if dt == "i8":
        return np.clip(np.round(a * 16), -128, 127).astype(np.int8)
    return encode(a, dt)


def to_dev(W, dt):
    if dt == "i8":
        return torch.from_numpy(W).cuda()
    return dev(W, dt)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32", "i8"])
@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (4, 8), (1, 2), (3, 8)])
def test_perm_gains_match_oracle(dt, n, m):
    rng = np.random.default_rng(40 + n + m)
    for R, K in [(37, 16 * m), (70, 34 * m), (5, 3 * m)]:
        W = exact_matrix(rng, (R, K), dt)
        perm = rng.permutation(K).astype(np.int32)
        gain_o, pick_o = oracle.perm_gains(W, dt, n, m, perm)
        gain, pick = nm.perm_gains(to_dev(W, dt), torch.from_numpy(perm).cuda(), n, m)
        G = K // m
        iu = np.triu_indices(G, 1)
        assert np.array_equal(gain.cpu().numpy().astype(np.float64)[iu], gain_o[iu]), f"{R}x{K}"
        assert np.array_equal(pick.cpu().numpy()[iu], pick_o[iu]), f"{R}x{K}"


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 4)])
def test_perm_search_matches_oracle(dt, n, m):
    rng = np.random.default_rng(50 + n + m)
    R, K = 48, 32 * m
    W = exact_matrix(rng, (R, K), dt)
    W = W.copy()
    p_o, rounds_o = oracle.perm_search(W, dt, n, m)
    p, rounds = nm.perm_search(to_dev(W, dt), n, m)
    assert rounds == rounds_o and np.array_equal(p.numpy(), p_o)
    assert oracle.kept_l1(W, dt, n, m, p_o) > oracle.kept_l1(W, dt, n, m)
    # a given start and a round limit
    start = rng.permutation(K).astype(np.int32)
    p_o, rounds_o = oracle.perm_search(W, dt, n, m, max_rounds=2, perm=start)
    p, rounds = nm.perm_search(to_dev(W, dt), n, m, max_rounds=2, perm=start)
    assert rounds == rounds_o and np.array_equal(p.numpy(), p_o)


def test_perm_search_edge_cases():
    W = torch.ones((8, 16), dtype=torch.bfloat16, device="cuda")
    p, rounds = nm.perm_search(W, 2, 4)           # all equal: nothing improves
    assert rounds == 0 and p.tolist() == list(range(16))
    p, rounds = nm.perm_search(W[:, :4].contiguous(), 2, 4)   # a single group
    assert rounds == 0 and p.tolist() == [0, 1, 2, 3]
    p, rounds = nm.perm_search(torch.zeros((0, 16), dtype=torch.bfloat16, device="cuda"), 2, 4)
    assert rounds == 0
    with pytest.raises(nm.NMError):
        nm.perm_search(W, 2, 4, perm=[0] * 16)     # not a permutation


@pytest.mark.parametrize("R,K", [(11008, 4096), (4096, 11008)])
def test_perm_gains_full_size_sampled(R, K):
    """The LLaMA MLP shapes with exact bf16 data: the gains of the pairs among 8 groups
    spread over the matrix against the oracle on just those groups' columns."""
    rng = np.random.default_rng(R)
    W = exact_matrix(rng, (R, K), "bf16")
    perm = rng.permutation(K).astype(np.int32)
    print(f"[perm] {R}x{K}", flush=True)
    gain, pick = nm.perm_gains(dev(W, "bf16"), torch.from_numpy(perm).cuda(), 2, 4)
    gain, pick = gain.cpu().numpy(), pick.cpu().numpy()
    G = K // 4
    groups = np.sort(rng.choice(G, size=8, replace=False))
    cols = np.concatenate([perm[4 * g:4 * g + 4] for g in groups])
    sub = np.ascontiguousarray(W[:, cols])
    g_o, p_o = oracle.perm_gains(sub, "bf16", 2, 4)
    for i in range(8):
        for j in range(i + 1, 8):
            assert gain[groups[i], groups[j]] == g_o[i, j]
            assert pick[groups[i], groups[j]] == p_o[i, j]
