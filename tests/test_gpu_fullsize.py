"""Full-size parity of the Mixtral-shaped MXFP8 training step (8 experts, H = 4096,
F = 14336, 8192 tokens, top-2), run through the same calls and buffers as bench.py
times (bench.make_inputs + bench.Step; the backward keeps its dY and dGU codes in
caller buffers, the same kernels), on sampled outputs that the oracle computes one by
one in fp64.  Every expert is sampled: the first and last rows of its first and last
256-row M-tile, and a few rows in between.

Every sampled output is recomputed from the operands the stage consumes:
  * bit-exact: routing, the weight codes (row and column forms) on sampled rows, the
    permuted x and dY codes (row and column forms) on sampled rows / columns;
  * gate-up stage: G, U (saved bf16), h after quantization, and the column form of h
    on sampled 32-row blocks, from the GPU's x and weight codes;
  * down stage: y_perm rows from the GPU's h codes; the combine of sampled tokens;
  * dh stage: dG, dU (row codes, and column codes on sampled 32-row blocks) and d_prob
    from the GPU's dY codes, the W_down column codes and the saved G, U;
  * dX rows (on sampled columns) from the GPU's dGU row codes and the W_gate_up column
    codes; dW_down and dW_gate_up entries over the expert's whole token span from the
    GPU's column codes (dY, h; dGU, x).
Tolerance: rel_F 2e-3 everywhere (each stage reads only the GPU's own codes); code flips
of h and dGU (quantized by the GPU from fp32, by the oracle from fp64) within the same
bounds as the small-size staged tests.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import mlp, mx
from oracle import route as rt
from oracle.metrics import rel_f

pytestmark = pytest.mark.gpu

TOL = 2e-3
H_FLIP_MAX = 4e-3
DGU_FLIP_MAX = 2e-3


def _deq(codes, scales):
    return mx.dequantize_rows(codes, scales)


def _bf16_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _take(t, *idx):
    """t indexed on the GPU by numpy index arrays / slices (one dimension each)."""
    for d, i in enumerate(idx):
        if isinstance(i, np.ndarray):
            t = t.index_select(d, torch.as_tensor(i, device=t.device, dtype=torch.long))
        else:
            t = t[(slice(None),) * d + (i,)]
    return t


def _tile_rows(r, rng, n_random=2):
    """Rows of a group to sample: first and last rows of its first and last 256-row
    M-tile, and n_random rows in between."""
    last = r.stop - 1
    lt0 = r.start + (r.stop - 1 - r.start) // 256 * 256       # first row of the last M-tile
    pick = {r.start, min(r.start + 255, last), lt0, last}
    pick |= set(int(v) for v in rng.integers(r.start, r.stop, n_random))
    return np.array(sorted(pick))


def test_mixtral_mxfp8_train_step_sampled():
    import bench
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import layout_from_gpu, npy, say

    w = synth.WORKLOADS[4]
    assert (w.T, w.E, w.H, w.F, w.k, w.prec, w.backward) == (8192, 8, 4096, 14336, 2, "mxfp8", True)
    dev = torch.device("cuda:0")
    say("[gpu] full-size MXFP8 training step: inputs")
    inp = bench.make_inputs(w, dev)
    step = bench.Step(m, w, inp, train=True)
    step.keep_intermediates = True
    step()
    torch.cuda.synchronize()
    say("[gpu] full-size step done; sampling")
    g, f, b, wq, dq = step.g, step.f, step.b, step.wq, step.dq
    assert b.dgu_row is not None and b.dy_col is not None
    E, H, F, k = w.E, w.H, w.F, w.k
    F2 = 2 * F
    rng = np.random.default_rng(4040)

    lay = layout_from_gpu(g, E, 32)
    idx, _ = rt.route(synth.logits(w), k)
    np.testing.assert_array_equal(lay.topk_idx, idx)
    np.testing.assert_array_equal(npy(g.group_offsets), lay.off)
    perm_src = npy(g.perm_src)
    prob = npy(g.prob_perm).astype(np.float64)
    x = _bf16_np(inp["x"])
    dy = _bf16_np(inp["dy"])
    pp_all = npy(g.perm_pos)
    slot = {int(pp_all[t, i]): (t, i) for t in range(w.T) for i in range(k)}
    dpg = npy(b.d_prob)
    acc = {key: [[], []] for key in ("G", "U", "h", "h_col", "y_perm", "dgu_row", "dgu_col", "d_prob", "dx_perm",
                                      "dw_down", "dw_gate_up")}
    flips = {"h": [0, 0], "dgu": [0, 0]}

    def add(key, got, ref):
        acc[key][0].append(np.asarray(got, dtype=np.float64).ravel())
        acc[key][1].append(np.asarray(ref, dtype=np.float64).ravel())

    for e in range(E):
        say(f"[gpu] full-size sampling expert {e} ({int(lay.sizes[e])} rows)")
        r = lay.rows(e)
        span = lay.kspan(e)
        rows = _tile_rows(r, rng)
        wgu = _bf16_np(inp["wgu"][e])
        wd = _bf16_np(inp["wd"][e])
        # weight codes, both forms, on sampled rows
        wr = rng.integers(0, F2, 4)
        q, s_ = mx.quantize_rows(wgu[wr])
        np.testing.assert_array_equal(npy(_take(wq[0][e], wr)), q)
        np.testing.assert_array_equal(npy(_take(wq[1][e], wr)), s_)
        hc = rng.integers(0, H, 4)
        q, s_ = mx.quantize_rows(wgu[:, hc].T)
        np.testing.assert_array_equal(npy(_take(wq[2][e], hc)), q)
        np.testing.assert_array_equal(npy(_take(wq[3][e], hc)), s_)
        q, s_ = mx.quantize_rows(wd[hc])
        np.testing.assert_array_equal(npy(_take(dq[0][e], hc)), q)
        fc = rng.integers(0, F, 4)
        q, s_ = mx.quantize_rows(wd[:, fc].T)
        np.testing.assert_array_equal(npy(_take(dq[2][e], fc)), q)
        np.testing.assert_array_equal(npy(_take(dq[3][e], fc)), s_)
        del wgu, wd
        # x and dY row codes on the sampled rows
        q, s_ = mx.quantize_rows(x[perm_src[rows]])
        np.testing.assert_array_equal(npy(_take(g.x_perm, rows)), q)
        np.testing.assert_array_equal(npy(_take(g.x_perm_scale, rows)), s_)
        q, s_ = mx.quantize_rows(dy[perm_src[rows]])
        np.testing.assert_array_equal(npy(_take(b.dy_row, rows)), q)
        np.testing.assert_array_equal(npy(_take(b.dy_row_scale, rows)), s_)

        # ---- forward: gate-up + SwiGLU x p (+ quantize h), down
        wgu_d = _deq(npy(wq[0][e]), npy(wq[1][e]))          # [2F][H], from the GPU's codes
        xd = _deq(npy(_take(g.x_perm, rows)), npy(_take(g.x_perm_scale, rows)))
        GU = xd @ wgu_d.T
        G, U = GU[:, :F], GU[:, F:]
        gu_gpu = _bf16_np(_take(f.saved_gu, rows))
        add("G", gu_gpu[:, :F], G)
        add("U", gu_gpu[:, F:], U)
        h = prob[rows][:, None] * mlp.silu(G) * U
        hq, hs = mx.quantize_rows(h)
        hq_gpu = npy(_take(f.h, rows))
        add("h", _deq(hq_gpu, npy(_take(f.h_scale, rows))), _deq(hq, hs))
        flips["h"][0] += int(np.count_nonzero(hq_gpu != hq)); flips["h"][1] += hq.size
        wd_d = _deq(npy(dq[0][e]), npy(dq[1][e]))           # [H][F]
        add("y_perm", _bf16_np(_take(f.y_perm, rows)), _deq(hq_gpu, npy(_take(f.h_scale, rows))) @ wd_d.T)
        del wd_d
        # column form of h: the 32-row blocks holding the first and the last sampled row
        for rr in (rows[0], rows[-1]):
            blk = (rr - lay.off[e]) // 32 * 32 + lay.off[e]
            br = np.arange(blk, blk + 32)
            fcol = int(rng.integers(0, F))
            inside = br < r.stop
            xb = _deq(npy(_take(g.x_perm, br)), npy(_take(g.x_perm_scale, br)))
            hb = np.where(inside, prob[br] * mlp.silu(xb @ wgu_d[fcol]) * (xb @ wgu_d[F + fcol]), 0.0)
            cq, cs = mx.quantize_rows(hb[None, :])
            got = _deq(npy(f.h_col[fcol, blk:blk + 32])[None, :],
                       npy(f.h_col_scale[fcol, blk // 32:blk // 32 + 1])[None, :])
            add("h_col", got, _deq(cq, cs))
        del wgu_d

        # ---- dh stage: dh = dY W_down (GPU's dY row codes, W_down column codes), the
        # SwiGLU backward with the saved G, U and p, d_prob
        wdc_d = _deq(npy(dq[2][e]), npy(dq[3][e]))          # [F][H]
        dyd = _deq(npy(_take(b.dy_row, rows)), npy(_take(b.dy_row_scale, rows)))
        dh = dyd @ wdc_d.T                                   # [n][F]
        Gs, Us = gu_gpu[:, :F], gu_gpu[:, F:]
        pr = prob[rows][:, None]
        dGU = np.concatenate([dh * pr * Us * mlp.dsilu(Gs), dh * pr * mlp.silu(Gs)], axis=1)
        gq, gs_ = mx.quantize_rows(dGU)
        gq_gpu = npy(_take(b.dgu_row, rows))
        add("dgu_row", _deq(gq_gpu, npy(_take(b.dgu_row_scale, rows))), _deq(gq, gs_))
        flips["dgu"][0] += int(np.count_nonzero(gq_gpu != gq)); flips["dgu"][1] += gq.size
        dp = np.sum(dh * mlp.silu(Gs) * Us, axis=1)
        add("d_prob", [float(dpg[slot[int(rr)]]) for rr in rows], dp)
        # column form of dGU: the 32-row block of the last sampled row, two columns (dG, dU)
        blk = (rows[-1] - lay.off[e]) // 32 * 32 + lay.off[e]
        br = np.arange(blk, blk + 32)
        inside = (br < r.stop)[:, None]
        fcol = int(rng.integers(0, F))
        dhb = _deq(npy(_take(b.dy_row, br)), npy(_take(b.dy_row_scale, br))) @ wdc_d[fcol]
        gub = _bf16_np(_take(f.saved_gu, br))
        Gb, Ub = gub[:, fcol], gub[:, F + fcol]
        cols = {fcol: dhb * prob[br] * Ub * mlp.dsilu(Gb), F + fcol: dhb * prob[br] * mlp.silu(Gb)}
        for j, v in cols.items():
            v = np.where(inside[:, 0], v, 0.0)
            cq, cs = mx.quantize_rows(v[None, :])
            got = _deq(npy(b.dgu_col[j, blk:blk + 32])[None, :], npy(b.dgu_col_scale[j, blk // 32:blk // 32 + 1])[None, :])
            add("dgu_col", got, _deq(cq, cs))
        del wdc_d

        # ---- dX rows on sampled columns: the GPU's dGU row codes x the W_gate_up column codes
        hcols = np.unique(np.concatenate([[0, 255, H - 256, H - 1], rng.integers(0, H, 60)]))
        wgc_d = _deq(npy(_take(wq[2][e], hcols)), npy(_take(wq[3][e], hcols)))   # [n_h][2F]
        add("dx_perm", _bf16_np(_take(_take(b.dx_perm, rows), slice(None), hcols)),
            _deq(gq_gpu, npy(_take(b.dgu_row_scale, rows))) @ wgc_d.T)

        # ---- weight gradients: entries over the expert's token span from the GPU's
        # column codes (dY, h for dW_down; dGU, x for dW_gate_up); the dY column codes
        # bit-exact on the sampled columns
        sb = slice(span.start // 32, span.stop // 32)
        hh = np.unique(np.concatenate([[0, H - 1], rng.integers(0, H, 10)]))
        ff = np.unique(np.concatenate([[0, F - 1], rng.integers(0, F, 10)]))
        valid = perm_src[span] >= 0
        DYc = np.where(valid[None, :], dy[np.maximum(perm_src[span], 0)][:, hh].T, 0.0)
        q, s_ = mx.quantize_rows(DYc)
        dyc_q = npy(_take(b.dy_col, hh, span))
        np.testing.assert_array_equal(dyc_q, q)
        np.testing.assert_array_equal(npy(_take(b.dy_col_scale, hh, sb)), s_)
        hcd = _deq(npy(_take(f.h_col, ff, span)), npy(_take(f.h_col_scale, ff, sb)))
        add("dw_down", npy(_take(b.dw_down[e], hh, ff)), _deq(dyc_q, s_) @ hcd.T)
        jj = np.unique(np.concatenate([[0, F - 1, F, F2 - 1], rng.integers(0, F2, 8)]))
        gcd = _deq(npy(_take(b.dgu_col, jj, span)), npy(_take(b.dgu_col_scale, jj, sb)))
        xcd = _deq(npy(_take(g.x_col, hh, span)), npy(_take(g.x_col_scale, hh, sb)))
        add("dw_gate_up", npy(_take(b.dw_gate_up[e], jj, hh)), gcd @ xcd.T)

    errs = {key: rel_f(np.concatenate(a), np.concatenate(ref)) for key, (a, ref) in acc.items()}
    # combine of sampled tokens (y and dx are the unweighted slot sums of the permuted rows)
    toks = rng.integers(0, w.T, 8)
    pp = pp_all[toks]
    yp = _bf16_np(_take(f.y_perm, pp.ravel())).reshape(len(toks), k, H)
    errs["y"] = rel_f(_bf16_np(_take(step.y, toks)), yp.sum(axis=1))
    dxp = _bf16_np(_take(b.dx_perm, pp.ravel())).reshape(len(toks), k, H)
    errs["dx"] = rel_f(_bf16_np(_take(step.dx, toks)), dxp.sum(axis=1))
    fr = {key: v[0] / v[1] for key, v in flips.items()}
    say("[gpu] full-size sampled rel_F", {kk: f"{v:.2e}" for kk, v in errs.items()},
        "flips", {kk: f"{v:.1e}" for kk, v in fr.items()})
    for key, v in errs.items():
        assert v <= TOL, (key, v)
    assert fr["h"] <= H_FLIP_MAX and fr["dgu"] <= DGU_FLIP_MAX, fr


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_mixtral_forward_sampled(cfg):
    """The three forward-only workloads at full size (BF16 and MXFP8 with 16384 tokens,
    MXFP8 with 32768 tokens and a Zipf-skewed router whose experts 2 and 5 get no
    tokens), through bench.Step: sampled rows of the largest and the smallest non-empty
    expert.  BF16: h and y_perm end to end against fp64 on the same bf16 inputs
    (rel_F 1e-2), and y per token from the per-token definition on sampled tokens.  MXFP8: x codes bit-exact, h from the GPU's x and weight codes and
    y_perm from the GPU's h codes (rel_F 2e-3)."""
    import bench
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import layout_from_gpu, npy, say

    w = synth.WORKLOADS[cfg]
    assert not w.backward and w.H == 4096 and w.F == 14336
    dev = torch.device("cuda:0")
    say("[gpu] full-size forward", w.name)
    inp = bench.make_inputs(w, dev)
    step = bench.Step(m, w, inp, train=False)
    step()
    torch.cuda.synchronize()
    g, f = step.g, step.f
    E, H, F, k = w.E, w.H, w.F, w.k
    mx8 = w.prec == "mxfp8"
    rng = np.random.default_rng(5050 + cfg)
    lay = layout_from_gpu(g, E, 32)
    idx, _ = rt.route(synth.logits(w), k)
    np.testing.assert_array_equal(lay.topk_idx, idx)
    np.testing.assert_array_equal(npy(g.split_sizes), lay.sizes)
    if w.skew:
        assert lay.sizes[2] == 0 and lay.sizes[5] == 0
    perm_src = npy(g.perm_src)
    prob = npy(g.prob_perm).astype(np.float64)
    x = _bf16_np(inp["x"])
    nonempty = [e for e in range(E) if lay.sizes[e] > 0]
    experts = sorted({max(nonempty, key=lambda e: lay.sizes[e]), min(nonempty, key=lambda e: lay.sizes[e])})
    got = {"h": [[], []], "y_perm": [[], []]}
    for e in experts:
        r = lay.rows(e)
        rows = np.array(sorted({r.start, r.stop - 1, min(r.start + 256, r.stop - 1)} |
                               set(int(v) for v in rng.integers(r.start, r.stop, 3))))
        if mx8:
            q, s = mx.quantize_rows(x[perm_src[rows]])
            np.testing.assert_array_equal(npy(_take(g.x_perm, rows)), q)
            np.testing.assert_array_equal(npy(_take(g.x_perm_scale, rows)), s)
            xd = _deq(npy(_take(g.x_perm, rows)), npy(_take(g.x_perm_scale, rows)))
            wgu_d = _deq(npy(step.wq[0][e]), npy(step.wq[1][e]))
            GU = xd @ wgu_d.T
            del wgu_d
            h = prob[rows][:, None] * mlp.silu(GU[:, :F]) * GU[:, F:]
            hq, hs = mx.quantize_rows(h)
            hg = _deq(npy(_take(f.h, rows)), npy(_take(f.h_scale, rows)))
            got["h"][0].append(hg)
            got["h"][1].append(_deq(hq, hs))
            Y = hg @ _deq(npy(step.dq[0][e]), npy(step.dq[1][e])).T
        else:
            GU = x[perm_src[rows]] @ _bf16_np(inp["wgu"][e]).T
            h = prob[rows][:, None] * mlp.silu(GU[:, :F]) * GU[:, F:]
            got["h"][0].append(_bf16_np(_take(f.h, rows)))
            got["h"][1].append(h)
            Y = h @ _bf16_np(inp["wd"][e]).T
        got["y_perm"][0].append(_bf16_np(_take(f.y_perm, rows)))
        got["y_perm"][1].append(Y)
    errs = {key: rel_f(np.concatenate(a), np.concatenate(ref)) for key, (a, ref) in got.items()}
    if not mx8:
        # end to end, per token: the oracle's own routing and the per-token definition
        # (each slot's expert applied to the token, weighted by its probability) against
        # the combined bf16 output, on sampled tokens
        _, p_or = rt.route(synth.logits(w), k)
        toks = np.sort(rng.choice(w.T, 12, replace=False))
        y_ref = np.zeros((len(toks), H))
        for e in sorted(set(int(v) for v in idx[toks].ravel())):
            wgu_e, wd_e = _bf16_np(inp["wgu"][e])[None], _bf16_np(inp["wd"][e])[None]
            for i in range(k):
                hit = np.where(idx[toks, i] == e)[0]
                if len(hit):
                    y_ref[hit] += mlp.fwd_per_token(x[toks[hit]], wgu_e, wd_e, np.zeros((len(hit), 1), np.int32),
                                                    p_or[toks[hit], i][:, None])
            del wgu_e, wd_e
        errs["y_per_token"] = rel_f(_bf16_np(_take(step.y, toks)), y_ref)
    say("[gpu] full-size forward", w.name, "experts", experts, "sizes", [int(lay.sizes[e]) for e in experts],
        {kk: f"{v:.2e}" for kk, v in errs.items()})
    tol = TOL if mx8 else 1e-2
    for key, v in errs.items():
        assert v <= tol, (key, v)
