"""Full-size parity of the Mixtral-shaped MXFP8 training step (8 experts, H = 4096,
F = 14336, 8192 tokens, top-2), run through the same calls and buffers as bench.py
times (bench.make_inputs + bench.Step), on sampled outputs that the oracle computes
one by one in fp64.

Every sampled output is recomputed from the operands the stage consumes:
  * bit-exact: routing, the weight codes (row and column forms) on sampled rows, the
    permuted x codes on sampled rows;
  * gate-up stage on sampled rows of two experts (the last one ends the grid): G, U
    (saved bf16), h after quantization, and the column form of h on sampled 32-row
    blocks, from the GPU's x and weight codes;
  * down stage: y_perm rows from the GPU's h codes; the combine of sampled tokens;
  * backward on one expert: dh from dY (quantized by the oracle, the same codes as the
    GPU's by the bit-exact quantizer tests) and the W_down column codes; d_prob; dX rows
    from the oracle's quantization of its dG, dU; dW_down and dW_gate_up entries over
    the expert's whole token span.
Tolerances: rel_F 2e-3 where the stage reads only the GPU's own codes; 5e-3 where the
oracle quantizes dG, dU itself (a few E4M3 code flips between fp32 and fp64 values).
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
TOL_REQ = 5e-3


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
    step()
    torch.cuda.synchronize()
    say("[gpu] full-size step done; sampling")
    g, f, b, wq, dq = step.g, step.f, step.b, step.wq, step.dq
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
    errs = {}

    def rows_of(e, n):
        r = lay.rows(e)
        pick = {r.start, r.stop - 1, min(r.start + 255, r.stop - 1), min(r.start + 256, r.stop - 1)}
        pick |= set(int(v) for v in rng.integers(r.start, r.stop, n))
        return np.array(sorted(pick))

    # ---------------------------------------------------------------- forward, two experts
    fw = {"G": [[], []], "U": [[], []], "h": [[], []], "y_perm": [[], []], "h_col": [[], []]}
    for e in (0, E - 1):
        wgu = _bf16_np(inp["wgu"][e])
        wd = _bf16_np(inp["wd"][e])
        wr = rng.integers(0, F2, 6)
        q, s = mx.quantize_rows(wgu[wr])
        np.testing.assert_array_equal(npy(_take(wq[0][e], wr)), q)
        np.testing.assert_array_equal(npy(_take(wq[1][e], wr)), s)
        hc = rng.integers(0, H, 6)
        q, s = mx.quantize_rows(wgu[:, hc].T)
        np.testing.assert_array_equal(npy(_take(wq[2][e], hc)), q)
        np.testing.assert_array_equal(npy(_take(wq[3][e], hc)), s)
        q, s = mx.quantize_rows(wd[hc])
        np.testing.assert_array_equal(npy(_take(dq[0][e], hc)), q)
        np.testing.assert_array_equal(npy(_take(dq[1][e], hc)), s)
        rows = rows_of(e, 4)
        q, s = mx.quantize_rows(x[perm_src[rows]])
        np.testing.assert_array_equal(npy(_take(g.x_perm, rows)), q)
        np.testing.assert_array_equal(npy(_take(g.x_perm_scale, rows)), s)
        wgu_d = _deq(npy(wq[0][e]), npy(wq[1][e]))          # [2F][H], from the GPU's codes
        xd = _deq(npy(_take(g.x_perm, rows)), npy(_take(g.x_perm_scale, rows)))
        GU = xd @ wgu_d.T
        G, U = GU[:, :F], GU[:, F:]
        gu_gpu = _bf16_np(_take(f.saved_gu, rows))
        fw["G"][0].append(gu_gpu[:, :F]); fw["G"][1].append(G)
        fw["U"][0].append(gu_gpu[:, F:]); fw["U"][1].append(U)
        h = prob[rows][:, None] * mlp.silu(G) * U
        hq, hs = mx.quantize_rows(h)
        fw["h"][0].append(_deq(npy(_take(f.h, rows)), npy(_take(f.h_scale, rows)))); fw["h"][1].append(_deq(hq, hs))
        wd_d = _deq(npy(dq[0][e]), npy(dq[1][e]))           # [H][F]
        Y = _deq(npy(_take(f.h, rows)), npy(_take(f.h_scale, rows))) @ wd_d.T
        fw["y_perm"][0].append(_bf16_np(_take(f.y_perm, rows))); fw["y_perm"][1].append(Y)
        # column form of h: a few (column, 32-row block) pairs
        for r in rows[:3]:
            blk = (r - lay.off[e]) // 32 * 32 + lay.off[e]
            br = np.arange(blk, blk + 32)
            fc = int(rng.integers(0, F))
            inside = br < lay.rows(e).stop
            xb = _deq(npy(_take(g.x_perm, br)), npy(_take(g.x_perm_scale, br)))
            gb = xb @ wgu_d[fc]
            ub = xb @ wgu_d[F + fc]
            hb = np.where(inside, prob[br] * mlp.silu(gb) * ub, 0.0)
            cq, cs = mx.quantize_rows(hb[None, :])
            got = _deq(npy(f.h_col[fc, blk:blk + 32])[None, :], npy(f.h_col_scale[fc, blk // 32:blk // 32 + 1])[None, :])
            fw["h_col"][0].append(got); fw["h_col"][1].append(_deq(cq, cs))
        del wgu_d, wd_d
    for key, (a, ref) in fw.items():
        errs[key] = rel_f(np.concatenate(a), np.concatenate(ref))
    # combine of sampled tokens
    toks = rng.integers(0, w.T, 8)
    y_gpu = _bf16_np(_take(step.y, toks))
    pp = npy(g.perm_pos)[toks]
    yp = _bf16_np(_take(f.y_perm, pp.ravel())).reshape(len(toks), k, H)
    errs["y"] = rel_f(y_gpu, yp.sum(axis=1))
    say("[gpu] forward sampled rel_F", {kk: f"{v:.2e}" for kk, v in errs.items()})

    # ---------------------------------------------------------------- backward, one expert
    e = E - 1
    span = lay.kspan(e)
    rows_all = np.arange(span.start, span.stop)
    valid_e = perm_src[rows_all] >= 0
    DY = np.where(valid_e[:, None], dy[np.maximum(perm_src[rows_all], 0)], 0.0)    # [span][H]
    dyq, dys = mx.quantize_rows(DY)
    wdc_d = _deq(npy(dq[2][e]), npy(dq[3][e]))          # [F][H]: W_down column codes
    wgc_d = _deq(npy(wq[2][e]), npy(wq[3][e]))          # [H][2F]: W_gate_up column codes
    gu_e = _bf16_np(f.saved_gu[span])                    # [span][2F]
    p_e = prob[rows_all]
    rows = rows_of(e, 3) - span.start
    dh = _deq(dyq[rows], dys[rows]) @ wdc_d.T            # [n][F]
    G, U = gu_e[rows, :F], gu_e[rows, F:]
    dU = dh * p_e[rows, None] * mlp.silu(G)
    dG = dh * p_e[rows, None] * U * mlp.dsilu(G)
    dp = np.sum(dh * mlp.silu(G) * U, axis=1)
    pp_all = npy(g.perm_pos)
    slot = {int(pp_all[t, i]): (t, i) for t in range(w.T) for i in range(k)}
    dpg = npy(b.d_prob)
    dp_gpu = np.array([float(dpg[slot[int(r + span.start)]]) for r in rows])
    errs["d_prob"] = rel_f(dp_gpu, dp)
    gq, gs = mx.quantize_rows(np.concatenate([dG, dU], axis=1))
    dX = _deq(gq, gs) @ wgc_d.T
    errs["dx_perm"] = rel_f(_bf16_np(_take(b.dx_perm, rows + span.start)), dX)
    # dW_down entries: sum over the expert's token span of dY (column codes) x h (GPU column codes)
    hh = rng.integers(0, H, 16)
    ff = rng.integers(0, F, 16)
    dyc_q, dyc_s = mx.quantize_rows(DY[:, hh].T)          # column form of dY for columns hh
    hc = _deq(npy(_take(f.h_col, ff, span)), npy(_take(f.h_col_scale, ff, slice(span.start // 32, span.stop // 32))))
    dWd = _deq(dyc_q, dyc_s) @ hc.T
    errs["dw_down"] = rel_f(npy(_take(b.dw_down[e], hh, ff)).astype(np.float64), dWd)
    # dW_gate_up entries: dGU (oracle, all rows of the span) column-quantized x X columns
    jj = np.concatenate([rng.integers(0, F, 8), F + rng.integers(0, F, 8)])
    fcol = jj % F
    dh_cols = _deq(dyq, dys) @ wdc_d[fcol].T            # [span][16]
    Gs, Us = gu_e[:, fcol], gu_e[:, F + fcol]
    gate = jj < F
    vals = np.where(gate[None, :], dh_cols * p_e[:, None] * Us * mlp.dsilu(Gs), dh_cols * p_e[:, None] * mlp.silu(Gs))
    vals[~valid_e] = 0.0
    cq, cs = mx.quantize_rows(vals.T)
    X = np.where(valid_e[:, None], x[np.maximum(perm_src[rows_all], 0)], 0.0)
    xq, xs = mx.quantize_rows(X[:, hh].T)
    dWgu = _deq(cq, cs) @ _deq(xq, xs).T
    errs["dw_gate_up"] = rel_f(npy(_take(b.dw_gate_up[e], jj, hh)).astype(np.float64), dWgu)
    say("[gpu] full-size sampled rel_F", {kk: f"{v:.2e}" for kk, v in errs.items()})
    for key, v in errs.items():
        tol = TOL_REQ if key in ("dx_perm", "dw_gate_up") else TOL
        assert v <= tol, (key, v)


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
