"""GPU parity of moe_route_permute (through the C ABI) against the oracle.

Bit-exact: topk_idx, split_sizes, group_offsets, perm_src, perm_pos, the gathered
bf16 rows and the MXFP8 codes/scales of x (row and column form).  Probabilities:
fp32 on the GPU vs fp64 in the oracle, |diff| <= 2e-6 and each token's sum within
1e-6 of 1."""
import numpy as np
import pytest
import torch

import synth
from oracle import mx
from oracle import route as rt

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import moe_grouped_expert_amd as mge
    return mge


def check_maps(g, logits, k, E, align):
    from tests.gpu_helpers import npy
    idx, p = rt.route(logits, k)
    np.testing.assert_array_equal(npy(g.topk_idx), idx)
    gp = npy(g.topk_prob).astype(np.float64)
    assert np.max(np.abs(gp - p)) <= 2e-6
    assert np.max(np.abs(gp.sum(1) - 1)) <= 1e-6
    sizes = rt.split_sizes(idx, E)
    np.testing.assert_array_equal(npy(g.split_sizes), sizes)
    np.testing.assert_array_equal(npy(g.group_offsets), rt.group_offsets(sizes, align))
    ps, pp = rt.permutation(idx, E, align)
    np.testing.assert_array_equal(npy(g.perm_src), ps)
    np.testing.assert_array_equal(npy(g.perm_pos), pp)
    gpp = npy(g.prob_perm)
    np.testing.assert_array_equal(gpp, rt.prob_permuted(npy(g.topk_prob).astype(np.float64), pp, len(ps)).astype(np.float32))
    return idx, ps


CASES = [
    # (T, E, k, H, align)
    (256, 4, 2, 64, 32),
    (1000, 8, 2, 128, 32),
    (300, 16, 4, 96, 32),
    (37, 1, 1, 64, 32),
    (64, 5, 5, 32, 32),
    (1, 8, 2, 64, 32),
    (777, 8, 2, 64, 1),
    (513, 6, 3, 64, 8),
    (2000, 256, 8, 32, 32),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
def test_route_permute(m, case, prec):
    from tests.gpu_helpers import gpu_bf16, npy, say
    T, E, k, H, align = case
    if prec == "mxfp8" and align % 32:
        pytest.skip("column form needs align % 32 == 0")
    say("[gpu] route", case, prec)
    rng = np.random.default_rng(T * 31 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, H)).astype(np.float32)
    gx = gpu_bf16(x)
    g = m.moe_route_permute(torch.from_numpy(logits).cuda(), gx, k, align=align, prec=prec, want_col=True)
    idx, ps = check_maps(g, logits, k, E, align)
    xb = gx.float().cpu().numpy().astype(np.float64)
    X = np.zeros((len(ps), H))
    X[ps >= 0] = xb[ps[ps >= 0]]
    if prec == "bf16":
        np.testing.assert_array_equal(g.x_perm.float().cpu().numpy(), X)
        np.testing.assert_array_equal(g.x_col.float().cpu().numpy(), X.T)
    else:
        q, s = mx.quantize_rows(X)
        np.testing.assert_array_equal(npy(g.x_perm), q)
        np.testing.assert_array_equal(npy(g.x_perm_scale), s)
        qc, sc = mx.quantize_cols(X)
        np.testing.assert_array_equal(npy(g.x_col), qc)
        np.testing.assert_array_equal(npy(g.x_col_scale), sc)


def test_route_ties_and_signed_zero(m):
    from tests.gpu_helpers import say
    say("[gpu] route ties")
    rng = np.random.default_rng(3)
    l = (np.round(rng.standard_normal((700, 8)) * 2) / 2).astype(np.float32)
    l[::5] = 0.0
    l[1::5, 0] = -0.0
    l[2::5, :] = 1.0
    for k in (1, 2, 3, 8):
        g = m.moe_route_permute(torch.from_numpy(l).cuda(), None, k, align=32)
        check_maps(g, l, k, 8, 32)


def test_route_skewed_long_sequence(m):
    """The Zipf-skewed 32768-token workload: two experts receive nothing."""
    from tests.gpu_helpers import npy, say
    w = synth.WORKLOADS[3]
    say("[gpu] route skewed", w.T)
    l = synth.logits(w)
    g = m.moe_route_permute(torch.from_numpy(l).cuda(), None, w.k, align=32)
    check_maps(g, l, w.k, w.E, 32)
    s = npy(g.split_sizes)
    assert s[2] == 0 and s[5] == 0 and s.sum() == w.T * w.k


def test_route_prob_given_and_device_flag(m):
    from tests.gpu_helpers import npy, say
    say("[gpu] route prob given")
    T, E, k = 300, 6, 2
    rng = np.random.default_rng(8)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    p = rng.random((T, k)).astype(np.float32)
    gi, gp = torch.from_numpy(idx).cuda(), torch.from_numpy(p).cuda()
    g = m.moe_route_permute(None, None, k, E=E, align=32, topk_idx=gi, topk_prob=gp)
    assert m.check_device_errors(g) == 0
    ps, pp = rt.permutation(idx, E, 32)
    np.testing.assert_array_equal(npy(g.perm_src), ps)
    np.testing.assert_array_equal(npy(g.perm_pos), pp)
    bad = idx.copy()
    bad[5, 1] = E + 3
    g2 = m.moe_route_permute(None, None, k, E=E, align=32, topk_idx=torch.from_numpy(bad).cuda(), topk_prob=gp)
    assert m.check_device_errors(g2) == 5   # MGE_ERR_DEVICE_CHECK
    assert m.check_device_errors(g2) == 0   # the flag is cleared after being read


def test_route_deterministic(m):
    from tests.gpu_helpers import gpu_bf16, npy
    rng = np.random.default_rng(12)
    l = torch.from_numpy(rng.standard_normal((5000, 8)).astype(np.float32)).cuda()
    x = gpu_bf16(rng.standard_normal((5000, 256)).astype(np.float32))
    a = m.moe_route_permute(l, x, 2, prec="mxfp8", want_col=True)
    b = m.moe_route_permute(l, x, 2, prec="mxfp8", want_col=True)
    for f in ("topk_idx", "topk_prob", "perm_src", "perm_pos", "x_perm", "x_perm_scale", "x_col", "x_col_scale"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


def _repeat_case(T, E, k, seed):
    """Caller-given top-k with repeated experts inside tokens and a few out-of-range
    indices (each sets the device flag and is clamped into [0, E))."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[::7, :] = idx[::7, :1]                 # every slot of these tokens on one expert
    bad = idx.copy()
    bad[3, 0] = E + 5
    bad[10, k - 1] = -2
    bad[11, :] = -1                            # clamps to expert 0 in every slot
    clamped = np.clip(bad, 0, E - 1).astype(np.int32)
    p = rng.random((T, k)).astype(np.float32)
    return bad, clamped, p


@pytest.mark.parametrize("T,E,k", [(300, 6, 2), (1000, 8, 4), (129, 3, 3), (64, 2, 2)])
def test_route_given_repeated_experts_maps_only(m, T, E, k):
    """Maps only (x = NULL): every row of perm_src is written, in [-1, T), and the maps
    equal the oracle's stable counting sort of the clamped indices."""
    from tests.gpu_helpers import npy, say
    say("[gpu] route repeated experts, maps only", T, E, k)
    bad, clamped, p = _repeat_case(T, E, k, T + E)
    g = m.moe_route_permute(None, None, k, E=E, align=32, topk_idx=torch.from_numpy(bad).cuda(),
                            topk_prob=torch.from_numpy(p).cuda())
    assert m.check_device_errors(g) == 5
    ps = npy(g.perm_src)
    assert ps.min() >= -1 and ps.max() < T
    sizes = rt.split_sizes(clamped, E)
    np.testing.assert_array_equal(npy(g.split_sizes), sizes)
    np.testing.assert_array_equal(npy(g.group_offsets), rt.group_offsets(sizes, 32))
    ops, opp = rt.permutation(clamped, E, 32)
    np.testing.assert_array_equal(ps, ops)
    np.testing.assert_array_equal(npy(g.perm_pos), opp)
    np.testing.assert_array_equal(npy(g.prob_perm), rt.prob_permuted(p.astype(np.float64), opp, len(ops)).astype(np.float32))


@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
def test_route_given_repeated_experts_with_x(m, prec):
    """The same inputs with x: the gathered rows (and MXFP8 codes) follow the oracle's
    permutation (regression test of the repeated-slot rank)."""
    from tests.gpu_helpers import gpu_bf16, npy, say
    T, E, k, H = 300, 6, 2, 64
    say("[gpu] route repeated experts with x", prec)
    bad, clamped, p = _repeat_case(T, E, k, 77)
    x = np.random.default_rng(78).standard_normal((T, H)).astype(np.float32)
    gx = gpu_bf16(x)
    g = m.moe_route_permute(None, gx, k, E=E, align=32, prec=prec, want_col=True,
                            topk_idx=torch.from_numpy(bad).cuda(), topk_prob=torch.from_numpy(p).cuda())
    assert m.check_device_errors(g) == 5
    ops, _ = rt.permutation(clamped, E, 32)
    np.testing.assert_array_equal(npy(g.perm_src), ops)
    xb = gx.float().cpu().numpy().astype(np.float64)
    X = np.zeros((len(ops), H))
    X[ops >= 0] = xb[ops[ops >= 0]]
    if prec == "bf16":
        np.testing.assert_array_equal(g.x_perm.float().cpu().numpy(), X)
        np.testing.assert_array_equal(g.x_col.float().cpu().numpy(), X.T)
    else:
        q, s = mx.quantize_rows(X)
        np.testing.assert_array_equal(npy(g.x_perm), q)
        np.testing.assert_array_equal(npy(g.x_perm_scale), s)
        qc, sc = mx.quantize_cols(X)
        np.testing.assert_array_equal(npy(g.x_col), qc)
        np.testing.assert_array_equal(npy(g.x_col_scale), sc)
