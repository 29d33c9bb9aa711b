"""Routing maps other than the routing call's.  split_sizes and group_offsets live on the
device, where the host cannot check them; the grouped GEMMs clamp every group's span into
the R permuted rows, and the other kernels of the path bound their own accesses (record-
bounded buffer resources, gathers that take a row outside [0, T) as zeros, segment maps
clamped into [0, R], combine and d_prob skipping entries outside the rows).  Such maps
give wrong results but touch nothing outside the buffers: the grouped forward and
backward must complete on them, and a correct step run afterwards must reproduce the one
run before bit for bit.
"""
import dataclasses

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import moe_grouped_expert_amd as mge
    return mge


def _weights(m, inp, prec):
    if prec == "mxfp8":
        wq = m.mxfp8_quantize(inp.g_wgu, "both")
        dq = m.mxfp8_quantize(inp.g_wd, "both")
        return (wq[0], dq[0], wq[1], dq[1]), (wq[2], dq[2], wq[3], dq[3])
    return (inp.g_wgu, inp.g_wd), (inp.g_wgu, inp.g_wd)


def _step(m, inp, g, prec):
    fw, bw = _weights(m, inp, prec)
    f = m.grouped_mlp_fwd(g, *fw, train=True)
    b = m.grouped_mlp_bwd(inp.g_dy, g, f, *bw)
    y = m.unpermute_combine(f.y_perm, g.perm_pos)
    dx = m.unpermute_combine(b.dx_perm, g.perm_pos)
    return [y, dx, b.d_prob, *b.dw_gate_up, *b.dw_down]


@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
def test_grouped_calls_with_maps_outside_the_rows(m, prec):
    from tests.gpu_helpers import Inputs, say
    w = synth.custom(241, T=300, E=4, H=128, F=256, k=2, prec=prec)
    say("[gpu] grouped calls on corrupt routing maps", prec, w)
    inp = Inputs(w)
    g = m.moe_route_permute(inp.g_logits, inp.g_x, w.k, align=32, prec=prec, want_col=True)
    ref = [t.clone() for t in _step(m, inp, g, prec)]
    torch.cuda.synchronize()
    R = g.perm_src.numel()
    dev = inp.g_x.device
    # a group larger than all the rows, a negative size, a size near 2^30; offsets negative,
    # past the rows and near 2^31 (E + 1 entries)
    bad_sizes = torch.tensor([R + 5000, -7, 2 ** 30, 33], dtype=torch.int32, device=dev)
    bad_offs = torch.tensor([0, -64, R + 100, 2 ** 31 - 1, 5], dtype=torch.int32, device=dev)
    gb = dataclasses.replace(g, split_sizes=bad_sizes, group_offsets=bad_offs)
    out = _step(m, inp, gb, prec)
    torch.cuda.synchronize()
    assert all(t.is_cuda for t in out)
    again = _step(m, inp, g, prec)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(ref, again)):
        assert torch.equal(a, b), i
