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
  * at full size (Mixtral shape, 8 or 4 ranks of 16384 tokens, rank 0 holding expert 0
    or experts 0 and 1) the rank's received rows match the oracle's routing, and sampled
    rows of h and y_perm of every local expert match the oracle fed the GPU's codes
    (rel_F 2e-3).
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


@pytest.mark.parametrize("cfg", [5, 6])
def test_mixtral_rank_share_forward_sampled(cfg):
    """Rank 0 of 8 (expert 0) or of 4 (experts 0, 1) at the Mixtral shape: 8 x 16384 or
    4 x 16384 tokens routed, the rank's received rows run through bench.Step as bench.py
    times them; sampled rows of every local expert against the oracle."""
    import bench
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import layout_from_gpu, npy, say

    w = synth.WORKLOADS[cfg]
    assert (w.T, w.E, w.H, w.F, w.k, w.prec, w.backward) == (16384, 8, 4096, 14336, 2, "mxfp8", False)
    dev = torch.device("cuda:0")
    say("[gpu] full-size rank share: inputs", w.name)
    inp, wl = bench.make_ep_share_inputs(m, w, dev)
    e_loc = w.E // w.ep
    idx, prob = rt.route(synth.logits(w), w.k)
    hit = idx < e_loc
    assert wl.T == int(hit.sum()) and wl.E == e_loc and wl.k == 1
    np.testing.assert_array_equal(npy(inp["idx"])[:, 0], idx[hit])
    np.testing.assert_allclose(npy(inp["prob"])[:, 0], prob[hit], rtol=2e-6, atol=0)
    step = bench.Step(m, wl, inp, train=False)
    step()
    torch.cuda.synchronize()
    g, f = step.g, step.f
    lay = layout_from_gpu(g, e_loc, 32)
    np.testing.assert_array_equal(npy(g.split_sizes), [int((idx[hit] == e).sum()) for e in range(e_loc)])
    F = w.F
    rng = np.random.default_rng(5500 + cfg)
    perm_src = npy(g.perm_src)
    errs = {"h": [[], []], "y_perm": [[], []]}
    for e in range(e_loc):
        r = lay.rows(e)
        rows = np.array(sorted({r.start, r.stop - 1, min(r.start + 256, r.stop - 1)} |
                               set(int(v) for v in rng.integers(r.start, r.stop, 4))))
        sel = torch.as_tensor(rows, device=dev, dtype=torch.long)
        x = inp["x"].index_select(0, torch.as_tensor(perm_src[rows], device=dev, dtype=torch.long))
        q, s = mx.quantize_rows(x.float().cpu().numpy().astype(np.float64))
        np.testing.assert_array_equal(npy(g.x_perm.index_select(0, sel)), q)
        np.testing.assert_array_equal(npy(g.x_perm_scale.index_select(0, sel)), s)
        GU = mx.dequantize_rows(q, s) @ mx.dequantize_rows(npy(step.wq[0][e]), npy(step.wq[1][e])).T
        p = npy(g.prob_perm).astype(np.float64)[rows]
        h = p[:, None] * mlp.silu(GU[:, :F]) * GU[:, F:]
        hq, hs = mx.quantize_rows(h)
        hg = mx.dequantize_rows(npy(f.h.index_select(0, sel)), npy(f.h_scale.index_select(0, sel)))
        errs["h"][0].append(hg)
        errs["h"][1].append(mx.dequantize_rows(hq, hs))
        errs["y_perm"][0].append(f.y_perm.index_select(0, sel).float().cpu().numpy().astype(np.float64))
        errs["y_perm"][1].append(hg @ mx.dequantize_rows(npy(step.dq[0][e]), npy(step.dq[1][e])).T)
    res = {k: rel_f(np.concatenate(a), np.concatenate(b)) for k, (a, b) in errs.items()}
    say("[gpu] rank share", w.name, "rows", wl.T, {kk: f"{v:.2e}" for kk, v in res.items()})
    for key, v in res.items():
        assert v <= 2e-3, (key, v)


def test_mixtral_ep8_rank_share_training_sampled():
    """Rank 0 of 8 (expert 0) at the Mixtral shape, the training step of 8 x 8192 tokens'
    expert-0 rows as bench.py times it (the backward keeps its dY and dGU codes in caller
    buffers, the same kernels): sampled rows of d_prob and of the dGU codes from the
    oracle's dh stage on the GPU's dY codes and saved G, U; dx_perm rows from the GPU's dGU
    codes; dW_down entries over the whole token span from the oracle's column forms of dY
    (bit-exact with the GPU's) and the GPU's column form of h.  rel_F 2e-3 each."""
    import bench
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import npy, say

    w = synth.WORKLOADS[7]
    assert (w.ep, w.T, w.E, w.H, w.F, w.k, w.prec, w.backward) == (8, 8192, 8, 4096, 14336, 2, "mxfp8", True)
    dev = torch.device("cuda:0")
    say("[gpu] full-size EP=8 training share: inputs")
    inp, wl = bench.make_ep_share_inputs(m, w, dev)
    step = bench.Step(m, wl, inp, train=True)
    step.keep_intermediates = True
    step()
    torch.cuda.synchronize()
    g, f, b = step.g, step.f, step.b
    F, H = w.F, w.H
    off, n = int(npy(g.group_offsets)[0]), int(npy(g.split_sizes)[0])
    assert off == 0 and n == wl.T
    perm_src = npy(g.perm_src)
    rng = np.random.default_rng(7700)
    rows = np.array(sorted({0, n - 1, 255, 256} | set(int(v) for v in rng.integers(0, n, 4))))
    sel = torch.as_tensor(rows, device=dev, dtype=torch.long)
    dy = inp["dy"].index_select(0, torch.as_tensor(perm_src[rows], device=dev, dtype=torch.long))
    dyq, dys = mx.quantize_rows(dy.float().cpu().numpy().astype(np.float64))
    np.testing.assert_array_equal(npy(b.dy_row.index_select(0, sel)), dyq)
    np.testing.assert_array_equal(npy(b.dy_row_scale.index_select(0, sel)), dys)
    dh = mx.dequantize_rows(dyq, dys) @ mx.dequantize_rows(npy(step.dq[2][0]), npy(step.dq[3][0])).T
    gu = f.saved_gu.index_select(0, sel).float().cpu().numpy().astype(np.float64)
    G, U = gu[:, :F], gu[:, F:]
    p = npy(g.prob_perm).astype(np.float64)[rows][:, None]
    dG = dh * p * U * mlp.dsilu(G)
    dU = dh * p * mlp.silu(G)
    gq, gs = mx.quantize_rows(np.concatenate([dG, dU], axis=1))
    gq_gpu, gs_gpu = npy(b.dgu_row.index_select(0, sel)), npy(b.dgu_row_scale.index_select(0, sel))
    flips = float(np.mean(gq_gpu != gq))
    dX = mx.dequantize_rows(gq_gpu, gs_gpu) @ mx.dequantize_rows(npy(step.wq[2][0]), npy(step.wq[3][0])).T
    errs = {"dgu_row": rel_f(mx.dequantize_rows(gq_gpu, gs_gpu), mx.dequantize_rows(gq, gs)),
            "dx_perm": rel_f(b.dx_perm.index_select(0, sel).float().cpu().numpy().astype(np.float64), dX),
            "d_prob": rel_f(npy(b.d_prob)[perm_src[rows], 0].astype(np.float64), np.sum(dh * mlp.silu(G) * U, axis=1))}
    # dW_down[h][f] = sum over the expert's tokens of dY[t][h] h[t][f], from the column forms
    hs, fs = rng.integers(0, H, 6), rng.integers(0, F, 6)
    span = (n + 31) // 32 * 32
    DYc = np.zeros((span, len(hs)))
    hs_t = torch.as_tensor(hs, device=dev, dtype=torch.long)
    fs_t = torch.as_tensor(fs, device=dev, dtype=torch.long)
    dy_rows = inp["dy"].index_select(0, torch.as_tensor(perm_src[:n], device=dev, dtype=torch.long))
    DYc[:n] = dy_rows.index_select(1, hs_t).float().cpu().numpy()
    cq, cs = mx.quantize_cols(DYc)
    hc = mx.dequantize_rows(npy(f.h_col.index_select(0, fs_t)[:, :span]),
                            npy(f.h_col_scale.index_select(0, fs_t)[:, :span // 32]))
    dWd = mx.dequantize_rows(cq, cs) @ hc.T
    got = b.dw_down[0].index_select(0, hs_t).index_select(1, fs_t)
    errs["dw_down"] = rel_f(got.double().cpu().numpy(), dWd)
    say("[gpu] EP=8 training share rows", n, {kk: f"{v:.2e}" for kk, v in errs.items()}, f"dGU flips {flips:.1e}")
    for key, v in errs.items():
        assert v <= 2e-3, (key, v)
    assert flips <= 2e-3, flips


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
