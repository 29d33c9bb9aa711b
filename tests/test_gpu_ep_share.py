"""One expert-parallel rank's share and the per-expert launch loop, through the C ABI.

Both replay the grouped call on a subset of the experts with the same kernels, so
they are checked for exact equality with the grouped call over all experts:
  * expert loop: one single-group grouped_mlp_fwd per expert (sizes and offsets are
    the e-th entries of the device arrays) gives the grouped call's h codes, scales and
    y_perm bit for bit;
  * rank share: the assignments routed to a rank's experts, received in (token, slot)
    order with their expert and probability and permuted locally with k = 1, give the
    global call's h, y_perm, d_prob and dx_perm of those experts bit for bit (a group's
    row tiles and 32-token scale blocks start at its first row in both calls); their
    weight gradients too in BF16, and in MXFP8 up to the grouping of the token sums
    into 64-token MFMA steps (rel_F 1e-6);
  * at full size (Mixtral shape, 8 ranks of 16384 tokens, rank 0 holding expert 0) the
    rank's received rows match the oracle's routing, and sampled rows of h and y_perm
    match the oracle fed the GPU's codes (rel_F 2e-3).
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import mlp, mx
from oracle import route as rt
from oracle.metrics import rel_f

pytestmark = pytest.mark.gpu


def _valid_rows(g):
    return torch.nonzero(g.perm_src >= 0).flatten()


def _inputs(w, empty=()):
    from tests.gpu_helpers import dev, gpu_bf16

    logits = synth.logits(w)
    for e in empty:
        logits[:, e] = np.float32(-1e30)
    return dict(logits=torch.from_numpy(logits).to(dev()), x=gpu_bf16(synth.x(w)), wgu=gpu_bf16(synth.w_gate_up(w)),
                wd=gpu_bf16(synth.w_down(w)), dy=gpu_bf16(synth.dy(w)) if w.backward else None)


@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
def test_expert_loop_equals_grouped(prec):
    import bench
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import say

    w = synth.custom(1100, T=700, E=5, H=128, F=320, k=2, prec=prec, backward=False)
    inp = _inputs(w, empty=(2,))
    say("[gpu] expert loop vs grouped", prec)
    a = bench.Step(m, w, inp, train=False, variant="grouped")
    a()
    b = bench.Step(m, w, inp, train=False, variant="expert_loop")
    b()
    torch.cuda.synchronize()
    assert int(a.g.split_sizes[2]) == 0
    rows = _valid_rows(a.g)
    assert torch.equal(a.f.y_perm[rows], b.f.y_perm[rows])
    assert torch.equal(a.f.h[rows], b.f.h[rows])
    if prec == "mxfp8":
        assert torch.equal(a.f.h_scale[rows], b.f.h_scale[rows])


def _rank_inputs(g_global, inp, lo, hi):
    """What rank [lo, hi) receives: its assignments in (token, slot) order, their local
    expert and probability, and the token rows of x and dy."""
    mask = (g_global.topk_idx >= lo) & (g_global.topk_idx < hi)
    tok = torch.nonzero(mask)[:, 0]
    idx = (g_global.topk_idx[mask] - lo).to(torch.int32).reshape(-1, 1).contiguous()
    prob = g_global.topk_prob[mask].reshape(-1, 1).contiguous()
    out = dict(logits=None, idx=idx, prob=prob, x=inp["x"][tok].contiguous(), wgu=inp["wgu"][lo:hi].contiguous(),
               wd=inp["wd"][lo:hi].contiguous(), dy=None if inp["dy"] is None else inp["dy"][tok].contiguous())
    return out, mask


@pytest.mark.parametrize("prec,train", [("bf16", False), ("mxfp8", False), ("bf16", True), ("mxfp8", True)])
def test_rank_share_equals_global(prec, train):
    import bench
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import say

    w = synth.custom(1200, T=1000, E=8, H=128, F=256, k=2, prec=prec, backward=train)
    inp = _inputs(w, empty=(5,))
    glob = bench.Step(m, w, inp, train=train)
    glob()
    torch.cuda.synchronize()
    gg = glob.g
    for ep in (8, 4):
        e_loc = w.E // ep
        for r in range(ep):
            lo, hi = r * e_loc, (r + 1) * e_loc
            say("[gpu] rank share", prec, "train" if train else "fwd", f"ep={ep} rank={r}")
            rin, mask = _rank_inputs(gg, inp, lo, hi)
            n = int(rin["idx"].shape[0])
            if n == 0:
                assert all(int(gg.split_sizes[e]) == 0 for e in range(lo, hi))
                continue
            wl = dataclasses.replace(w, T=n, E=e_loc, k=1)
            st = bench.Step(m, wl, rin, train=train)
            st()
            torch.cuda.synchronize()
            rows_g = gg.perm_pos[mask]                 # the received rows' global rows
            rows_l = st.g.perm_pos[:, 0]
            assert torch.equal(st.g.split_sizes.cpu(), gg.split_sizes[lo:hi].cpu())
            assert torch.equal(st.f.h[rows_l], glob.f.h[rows_g])
            assert torch.equal(st.f.y_perm[rows_l], glob.f.y_perm[rows_g])
            if prec == "mxfp8":
                assert torch.equal(st.f.h_scale[rows_l], glob.f.h_scale[rows_g])
            if train:
                assert torch.equal(st.b.d_prob[:, 0], glob.b.d_prob[mask])
                assert torch.equal(st.b.dx_perm[rows_l], glob.b.dx_perm[rows_g])
                for le in range(e_loc):
                    for got, ref in ((st.b.dw_down[le], glob.b.dw_down[lo + le]),
                                     (st.b.dw_gate_up[le], glob.b.dw_gate_up[lo + le])):
                        if prec == "bf16":
                            assert torch.equal(got, ref)
                        else:
                            # the token (K) axis is cut into 64-token MFMA steps from the
                            # 128-token slice below the group's first row: the same sums,
                            # grouped differently when the two first rows differ mod 64
                            g64, r64 = got.double().cpu().numpy(), ref.double().cpu().numpy()
                            assert rel_f(g64, r64) <= 1e-6 if np.any(r64) else not np.any(g64)


def test_mixtral_ep8_rank_share_forward_sampled():
    """Rank 0 of 8 (expert 0) at the Mixtral shape: 8 x 16384 tokens routed, the rank's
    received rows run through bench.Step as bench.py times them."""
    import bench
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import layout_from_gpu, npy, say

    w = synth.WORKLOADS[5]
    assert (w.ep, w.T, w.E, w.H, w.F, w.k, w.prec, w.backward) == (8, 16384, 8, 4096, 14336, 2, "mxfp8", False)
    dev = torch.device("cuda:0")
    say("[gpu] full-size EP=8 rank share: inputs")
    inp, wl = bench.make_ep_share_inputs(m, w, dev)
    idx, prob = rt.route(synth.logits(w), w.k)
    hit = idx == 0
    assert wl.T == int(hit.sum()) and wl.E == 1 and wl.k == 1
    np.testing.assert_allclose(npy(inp["prob"])[:, 0], prob[hit], rtol=2e-6, atol=0)
    step = bench.Step(m, wl, inp, train=False)
    step()
    torch.cuda.synchronize()
    g, f = step.g, step.f
    lay = layout_from_gpu(g, 1, 32)
    assert int(npy(g.split_sizes)[0]) == wl.T
    F = w.F
    rng = np.random.default_rng(5500)
    r = lay.rows(0)
    rows = np.array(sorted({r.start, r.stop - 1, min(r.start + 256, r.stop - 1)} |
                           set(int(v) for v in rng.integers(r.start, r.stop, 5))))
    sel = torch.as_tensor(rows, device=dev, dtype=torch.long)
    perm_src = npy(g.perm_src)
    x = inp["x"].index_select(0, torch.as_tensor(perm_src[rows], device=dev, dtype=torch.long))
    q, s = mx.quantize_rows(x.float().cpu().numpy().astype(np.float64))
    np.testing.assert_array_equal(npy(g.x_perm.index_select(0, sel)), q)
    np.testing.assert_array_equal(npy(g.x_perm_scale.index_select(0, sel)), s)
    xd = mx.dequantize_rows(q, s)
    GU = xd @ mx.dequantize_rows(npy(step.wq[0][0]), npy(step.wq[1][0])).T
    p = npy(g.prob_perm).astype(np.float64)[rows]
    h = p[:, None] * mlp.silu(GU[:, :F]) * GU[:, F:]
    hq, hs = mx.quantize_rows(h)
    hg = mx.dequantize_rows(npy(f.h.index_select(0, sel)), npy(f.h_scale.index_select(0, sel)))
    Y = hg @ mx.dequantize_rows(npy(step.dq[0][0]), npy(step.dq[1][0])).T
    yg = f.y_perm.index_select(0, sel).float().cpu().numpy().astype(np.float64)
    errs = {"h": rel_f(hg, mx.dequantize_rows(hq, hs)), "y_perm": rel_f(yg, Y)}
    say("[gpu] EP=8 rank share rows", wl.T, {kk: f"{v:.2e}" for kk, v in errs.items()})
    for key, v in errs.items():
        assert v <= 2e-3, (key, v)


def test_mixtral_expert_loop_equals_grouped():
    """The Mixtral-shaped MXFP8 forward (16384 tokens) as bench.py times both variants:
    every valid row of h and y_perm is bit-equal."""
    import bench
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import say

    w = synth.WORKLOADS[2]
    dev = torch.device("cuda:0")
    say("[gpu] full-size expert loop vs grouped")
    inp = bench.make_inputs(w, dev)
    a = bench.Step(m, w, inp, train=False)
    a()
    ya, ha, sa = a.f.y_perm.clone(), a.f.h.clone(), a.f.h_scale.clone()
    rows = _valid_rows(a.g)
    del a
    b = bench.Step(m, w, inp, train=False, variant="expert_loop")
    b()
    torch.cuda.synchronize()
    assert torch.equal(ya[rows], b.f.y_perm[rows])
    assert torch.equal(ha[rows], b.f.h[rows])
    assert torch.equal(sa[rows], b.f.h_scale[rows])
