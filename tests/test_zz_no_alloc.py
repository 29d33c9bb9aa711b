"""moe_route_permute_noalloc (the routing/permutation call whose workspace is the
library's fixed per-GPU scratch, for callers that cannot allocate) against
moe_route_permute with a caller workspace, through the C ABI: every output bit-exact,
on two calls in a row, the second with a smaller input (the scratch keeps the first
call's contents)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

FIELDS = ("topk_idx", "topk_prob", "split_sizes", "group_offsets", "perm_src", "perm_pos", "prob_perm",
          "x_perm", "x_perm_scale", "x_col", "x_col_scale")


def _same(a, b):
    for f in FIELDS:
        u, v = getattr(a, f), getattr(b, f)
        assert (u is None) == (v is None), f
        if u is not None:
            assert torch.equal(u, v), f


def test_noalloc_route_equals_workspace_route():
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import gpu_bf16, say
    rng = np.random.default_rng(31337)
    # (T, E, k, H, prec, given top-k): the second call is smaller than the first
    calls = [(6000, 8, 2, 256, "mxfp8", False), (700, 16, 4, 128, "bf16", False), (300, 6, 2, 64, "mxfp8", True)]
    for T, E, k, H, prec, given in calls:
        say("[gpu] noalloc route", T, E, k, H, prec, "given" if given else "logits")
        x = gpu_bf16(rng.standard_normal((T, H)).astype(np.float32))
        if given:
            idx = torch.from_numpy(rng.integers(0, E, (T, k)).astype(np.int32)).cuda()
            p = torch.from_numpy(rng.random((T, k)).astype(np.float32)).cuda()
            kw = dict(E=E, topk_idx=idx, topk_prob=p)
            lg = None
        else:
            lg = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).cuda()
            kw = {}
        ref = m.moe_route_permute(lg, x, k, align=32, prec=prec, want_col=True, **kw)
        if given:   # the noalloc call writes its own copies of the outputs
            kw = dict(E=E, topk_idx=idx.clone(), topk_prob=p.clone())
        got = m.moe_route_permute(lg, x, k, align=32, prec=prec, want_col=True, noalloc=True, **kw)
        assert got.workspace is None
        torch.cuda.synchronize()
        _same(got, ref)


def test_noalloc_route_rejects_sizes_beyond_the_scratch():
    import moe_grouped_expert_amd as m
    from moe_grouped_expert_amd import _binding as b
    lg = torch.zeros((300000, 256), dtype=torch.float32, device="cuda:0")
    with pytest.raises(b.MgeError) as ei:
        m.moe_route_permute(lg, None, 2, align=32, noalloc=True)
    assert "scratch" in str(ei.value)
