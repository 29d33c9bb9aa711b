"""GPU parity of moe_router_bwd (through the C ABI) against the oracle's router
backward, on the same fp32 inputs (indices and probabilities from the GPU routing,
d_prob seeded).

Bar: exact zeros where no slot selects the expert; elsewhere the fp32 result of
p_i (d_p_i - s) with s = sum_j p_j d_p_j (k fused multiply-adds, then a subtract and a
multiply) is within (k + 3) unit roundoffs of the scale p_i (|d_p_i| + sum_j p_j |d_p_j|),
bounded here by 1e-6 times that scale per element."""
import numpy as np
import pytest
import torch

from oracle import route as rt

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import moe_grouped_expert_amd as mge
    return mge


def check(m, idx, p, dp, E):
    from tests.gpu_helpers import npy
    got = npy(m.moe_router_bwd(idx, p, dp, E)).astype(np.float64)
    i_, p_, d_ = npy(idx), npy(p).astype(np.float64), npy(dp).astype(np.float64)
    ref = rt.router_bwd(i_, p_, d_, E)
    T, k = i_.shape
    scale = np.zeros((T, E))
    sabs = (p_ * np.abs(d_)).sum(axis=1)
    hit = np.zeros((T, E), bool)
    for i in range(k):
        e = i_[:, i]
        ok = (e >= 0) & (e < E)
        rows = np.nonzero(ok)[0]
        scale[rows, e[ok]] += p_[ok, i] * (np.abs(d_[ok, i]) + sabs[ok])
        hit[rows, e[ok]] = True
    assert np.all(got[~hit] == 0.0)
    assert np.all(np.abs(got - ref) <= 1e-6 * scale + 1e-30)
    return got, ref


@pytest.mark.parametrize("T,E,k", [(300, 8, 2), (1000, 16, 4), (513, 6, 3), (64, 8, 1), (1, 4, 4),
                                   (2000, 256, 8), (8192, 8, 2)])
def test_router_bwd_after_routing(m, T, E, k):
    from tests.gpu_helpers import say
    say("[gpu] router_bwd", T, E, k)
    rng = np.random.default_rng(T * 7 + E * 3 + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    g = m.moe_route_permute(torch.from_numpy(logits).cuda(), None, k, align=32)
    dp = torch.from_numpy(rng.standard_normal((T, k)).astype(np.float32)).cuda()
    got, ref = check(m, g.topk_idx, g.topk_prob, dp, E)
    if k == 1:
        assert np.all(got == 0.0)   # p = 1: nothing flows back to the logits
    # each token's gradient sums to zero (shift invariance of the softmax)
    assert np.max(np.abs(got.sum(axis=1))) <= 1e-5


def test_router_bwd_repeated_and_out_of_range_indices(m):
    """Slots that share an expert add up; an index outside [0, E) adds to nothing."""
    from tests.gpu_helpers import say
    say("[gpu] router_bwd repeated / out-of-range indices")
    rng = np.random.default_rng(11)
    T, E, k = 257, 6, 3
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[::5, 1] = idx[::5, 0]
    idx[1::7, 2] = E
    idx[2::9, 0] = -1
    p = rng.random((T, k)).astype(np.float32)
    dp = rng.standard_normal((T, k)).astype(np.float32)
    check(m, torch.from_numpy(idx).cuda(), torch.from_numpy(p).cuda(), torch.from_numpy(dp).cuda(), E)


def test_router_bwd_empty(m):
    z = torch.zeros((0, 2), device="cuda")
    out = m.moe_router_bwd(z.int(), z, z, 8)
    assert out.shape == (0, 8)
