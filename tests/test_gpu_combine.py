"""unpermute_combine on its own: unweighted (the method's combine, the probability having
been applied inside the forward) and weighted, bf16 and f32 in and out, and slots whose
perm_pos entry names no row of the input (-1, or past its rows) adding nothing.

Reference: the combine's definition in fp64, out[t] = sum over the slots i whose entry
lies in [0, rows) of w[t, i] * in[perm_pos[t, i]].  The GPU sums k products in fp32 in
slot order, at most two roundings per slot, so each element is within 2k * 2^-24 of the
sum of the terms' magnitudes, plus half a bf16 ulp of the result (at most 2^-8 of it)
for a bf16 output; a token with no valid slot gets exactly zero.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import moe_grouped_expert_amd as mge
    return mge


def _ref(inp, pos, w):
    rows = inp.shape[0]
    out = np.zeros((pos.shape[0], inp.shape[1]), dtype=np.float64)
    for i in range(pos.shape[1]):
        ok = (pos[:, i] >= 0) & (pos[:, i] < rows)
        wi = np.ones(pos.shape[0]) if w is None else w[:, i]
        out[ok] += wi[ok, None] * inp[pos[ok, i]]
    return out


@pytest.mark.parametrize("weighted", [False, True], ids=["unweighted", "weighted"])
@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
@pytest.mark.parametrize("in_dt", ["bf16", "f32"])
def test_combine_with_dropped_slots(m, in_dt, out_dt, weighted):
    from tests.gpu_helpers import say
    T, k, H, rows = 300, 3, 256, 1000
    say("[gpu] combine", in_dt, out_dt, "weighted" if weighted else "unweighted", T, k, H, rows)
    g = torch.Generator().manual_seed(71 + 2 * weighted + 4 * (in_dt == "f32") + 8 * (out_dt == "f32"))
    inp = torch.randn(rows, H, generator=g)
    if in_dt == "bf16":
        inp = inp.to(torch.bfloat16)
    pos = torch.randint(0, rows, (T, k), generator=g, dtype=torch.int32)
    pos[::7, 1] = -1            # dropped slots
    pos[::11, 2] = rows + 5     # past the rows of the input
    pos[5, :] = -1              # a token with no valid slot
    w = torch.rand(T, k, generator=g) * 2 - 0.5 if weighted else None
    out = m.unpermute_combine(inp.cuda(), pos.cuda(), None if w is None else w.cuda(), out_dtype=out_dt)
    torch.cuda.synchronize()
    assert out.shape == (T, H) and out.dtype == (torch.bfloat16 if out_dt == "bf16" else torch.float32)
    x = inp.float().numpy().astype(np.float64)
    pn = pos.numpy()
    wn = None if w is None else w.numpy().astype(np.float64)
    ref = _ref(x, pn, wn)
    mag = _ref(np.abs(x), pn, None if wn is None else np.abs(wn))
    got = out.float().cpu().numpy().astype(np.float64)
    err32 = 2 * k * 2.0 ** -24 * mag
    tol = err32 + (2.0 ** -8 * (np.abs(ref) + err32) if out_dt == "bf16" else 0.0)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (int(bad.sum()), float(np.abs(got - ref)[bad].max()))
    assert np.all(got[5] == 0.0)
