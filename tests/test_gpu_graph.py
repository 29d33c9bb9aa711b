"""The training step captured in a HIP graph and replayed.

Every call of the step (routing and permutation, the weight quantization, the grouped
forward and backward, both combines, the router backward) only launches kernels: no
device allocation, memset, copy or host synchronisation happens inside them, and the
per-expert pointer tables go up as kernel arguments.  The whole step can therefore be
captured (torch.cuda.graph; its memory pool provides the outputs and workspaces the
binding allocates) and replayed, with the routing workspace either in that pool or in
the library's fixed scratch (moe_route_permute_noalloc).  Each replay must reproduce the
eager step bit for bit; eager steps run between the replays, on the same stream.
"""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import moe_grouped_expert_amd as mge
    return mge


def _step(m, inp, prec, noalloc):
    """One training step; returns every output that is fully written (permuted buffers'
    padding rows are not, so those leave through the combines)."""
    w = inp.w
    g = m.moe_route_permute(inp.g_logits, inp.g_x, w.k, align=32, prec=prec, want_col=True, noalloc=noalloc)
    if prec == "mxfp8":
        wq = m.mxfp8_quantize(inp.g_wgu, "both")
        dq = m.mxfp8_quantize(inp.g_wd, "both")
        f = m.grouped_mlp_fwd(g, wq[0], dq[0], wq[1], dq[1], train=True)
        b = m.grouped_mlp_bwd(inp.g_dy, g, f, wq[2], dq[2], wq[3], dq[3])
    else:
        f = m.grouped_mlp_fwd(g, inp.g_wgu, inp.g_wd, train=True)
        b = m.grouped_mlp_bwd(inp.g_dy, g, f, inp.g_wgu, inp.g_wd)
    y = m.unpermute_combine(f.y_perm, g.perm_pos)
    dx = m.unpermute_combine(b.dx_perm, g.perm_pos)
    d_logits = m.moe_router_bwd(g.topk_idx, g.topk_prob, b.d_prob, w.E)
    return [g.topk_idx, g.topk_prob, g.perm_src, g.perm_pos, y, dx, b.d_prob, d_logits, *b.dw_gate_up, *b.dw_down]


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
def test_training_step_graph_replay(m, prec, noalloc):
    from tests.gpu_helpers import Inputs, say
    w = synth.custom(230, T=700, E=6, H=256, F=384, k=2, prec=prec)
    say("[gpu] graph replay", prec, "noalloc" if noalloc else "workspace", w)
    inp = Inputs(w)
    ref = [t.clone() for t in _step(m, inp, prec, noalloc)]
    torch.cuda.synchronize()
    # warm-up on a side stream (default priority), as torch's capture expects
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(m, inp, prec, noalloc)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = _step(m, inp, prec, noalloc)
    torch.cuda.synchronize()
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, out)):
            assert torch.equal(a, b), (rep, i)
        eager = _step(m, inp, prec, noalloc)   # eager work between the replays
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, eager)):
            assert torch.equal(a, b), ("eager", rep, i)
    del graph
