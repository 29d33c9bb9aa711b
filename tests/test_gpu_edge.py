"""Edge cases of the whole path, forward + backward in BF16 and MXFP8, against the oracle.

Uneven routing must run without a per-expert loop ([P2] "Fragmented Expert Kernels": the
grouped call takes per-expert token counts).  The routing is given (caller top-k), so the
groups have exactly the sizes under test:
  * groups of 0, 1, 31, 32, 33, 255, 256, 257 and 513 rows: empty, single-row, around the
    32-row scale block and the 256-row M-tile, several tiles with a ragged tail;
  * H = F = 32, the smallest sizes the layout allows (one scale block along K);
  * one expert receiving every token at E = 8 (seven empty experts, k = 2);
  * a single token (T = 1);
  * the grid's last round as quarter-width work items: 2 experts of 2176 rows each (every
    token on both), H = 4096, so the dX and down GEMMs have 2 x 9 x 16 = 288 tiles on 256
    CUs, and their last 32 tiles (the second expert's last two M-tiles, one of them half
    full) run as 128 items of 256 x 64 in the tail launch.
BF16: y, dx, dW_gate_up, dW_down and d_prob end to end against fp64 on the same bf16
inputs (rel_F 1e-2).  MXFP8: staged, each stage against the oracle fed the GPU's own
quantized operands (rel_F 2e-3; x, dy, weights and the permutation bit-exact; h and dGU
compared after dequantization with their code flips bounded); a bf16-stored stage output
of under 4096 elements (the single token) whose rel_F exceeds 2e-3 is held element by
element to one bf16 rounding instead.  Experts without tokens
get exactly zero weight gradients in both."""
import numpy as np
import pytest
import torch

import synth
from oracle import mlp, mx
from oracle import route as rt
from oracle.metrics import rel_f

pytestmark = pytest.mark.gpu

BF16_TOL = 1e-2
MX_TOL = 2e-3
H_FLIP_MAX = 4e-3
DGU_FLIP_MAX = 2e-3


@pytest.fixture(scope="module")
def m():
    import moe_grouped_expert_amd as mge
    return mge


def _case(name):
    """(x, wgu, wd, dy, E, k, idx, prob, logits): exact bf16 values as fp32 numpy."""
    rng = np.random.default_rng(CASES.index(name) + 900)
    logits = None
    if name == "sizes":
        sizes = [0, 1, 31, 32, 33, 255, 256, 257, 513]
        E, k, H, F = len(sizes), 1, 64, 96
        idx = np.concatenate([np.full(s, e, np.int32) for e, s in enumerate(sizes)])
        idx = rng.permutation(idx)[:, None].astype(np.int32)        # tokens of all experts interleaved
        prob = rng.uniform(0.2, 1.0, idx.shape).astype(np.float32)
    elif name == "h32_f32":
        E, k, H, F, T = 4, 2, 32, 32, 150
        logits = rng.standard_normal((T, E)).astype(np.float32)
        idx = prob = None
    elif name == "one_expert_all_tokens":
        E, k, H, F, T = 8, 2, 64, 64, 300
        idx = np.stack([np.full(T, 3), rng.choice([0, 1, 2, 4, 5, 6, 7], T)], axis=1).astype(np.int32)
        idx[::2] = idx[::2, ::-1]                                    # expert 3 in either slot
        p0 = rng.uniform(0.5, 0.9, T).astype(np.float32)
        prob = np.stack([p0, 1 - p0], axis=1).astype(np.float32)
    elif name == "one_token":
        E, k, H, F, T = 8, 2, 64, 96, 1
        logits = rng.standard_normal((T, E)).astype(np.float32)
        idx = prob = None
    elif name == "tail_split":
        E, k, H, F, T = 2, 2, 4096, 256, 2176
        idx = np.tile(np.array([[0, 1]], np.int32), (T, 1))
        idx[::2] = idx[::2, ::-1]                                    # either expert in slot 0
        prob = rng.uniform(0.2, 0.8, (T, k)).astype(np.float32)
    else:
        raise ValueError(name)
    T = idx.shape[0] if idx is not None else logits.shape[0]
    x = synth.to_bf16_values(rng.standard_normal((T, H)).astype(np.float32))
    wgu = synth.to_bf16_values((rng.standard_normal((E, 2 * F, H)) * 0.05).astype(np.float32))
    wd = synth.to_bf16_values((rng.standard_normal((E, H, F)) * 0.05).astype(np.float32))
    dy = synth.to_bf16_values(rng.standard_normal((T, H)).astype(np.float32))
    return x, wgu, wd, dy, E, k, idx, prob, logits


def _run(m, prec, x, wgu, wd, dy, E, k, idx, prob, logits):
    from tests.gpu_helpers import gpu_bf16
    gx, gwgu, gwd, gdy = gpu_bf16(x), gpu_bf16(wgu), gpu_bf16(wd), gpu_bf16(dy)
    if idx is not None:
        g = m.moe_route_permute(None, gx, k, E=E, align=32, prec=prec, want_col=True,
                                topk_idx=torch.from_numpy(idx).cuda(), topk_prob=torch.from_numpy(prob).cuda())
    else:
        g = m.moe_route_permute(torch.from_numpy(logits).cuda(), gx, k, align=32, prec=prec, want_col=True)
    o = dict(g=g)
    if prec == "mxfp8":
        wq = m.mxfp8_quantize(gwgu, "both")
        dq = m.mxfp8_quantize(gwd, "both")
        f = m.grouped_mlp_fwd(g, wq[0], dq[0], wq[1], dq[1], train=True)
        b = m.grouped_mlp_bwd(gdy, g, f, wq[2], dq[2], wq[3], dq[3], keep_intermediates=True)
        o.update(wq=wq, dq=dq)
    else:
        f = m.grouped_mlp_fwd(g, gwgu, gwd, train=True)
        b = m.grouped_mlp_bwd(gdy, g, f, gwgu, gwd)
    o.update(f=f, b=b, y=m.unpermute_combine(f.y_perm, g.perm_pos), dx=m.unpermute_combine(b.dx_perm, g.perm_pos))
    torch.cuda.synchronize()
    return o


CASES = ["sizes", "h32_f32", "one_expert_all_tokens", "one_token", "tail_split"]


def _needs_256_cus(name):
    if name == "tail_split" and torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the tile arithmetic of this case assumes 256 compute units")


@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
@pytest.mark.parametrize("name", CASES)
def test_edge_fwd_bwd(m, name, prec):
    from tests.gpu_helpers import f64, npy, say
    _needs_256_cus(name)
    x, wgu, wd, dy, E, k, idx, prob, logits = _case(name)
    say("[gpu] edge", name, prec, "T", x.shape[0], "E", E, "k", k, "H", x.shape[1], "F", wd.shape[2])
    o = _run(m, prec, x, wgu, wd, dy, E, k, idx, prob, logits)
    g, f, b = o["g"], o["f"], o["b"]
    if idx is None:
        idx, p = rt.route(logits, k)
        np.testing.assert_array_equal(npy(g.topk_idx), idx)
    else:
        p = prob.astype(np.float64)
    lay = mlp.Layout(npy(g.topk_idx), npy(g.topk_prob).astype(np.float64), E, 32)
    np.testing.assert_array_equal(lay.topk_idx, idx)
    np.testing.assert_array_equal(npy(g.split_sizes), lay.sizes)
    np.testing.assert_array_equal(npy(g.perm_src), lay.perm_src)
    np.testing.assert_array_equal(npy(g.perm_pos), lay.perm_pos)
    if name == "sizes":
        np.testing.assert_array_equal(lay.sizes, [0, 1, 31, 32, 33, 255, 256, 257, 513])
    empty = [e for e in range(E) if lay.sizes[e] == 0]
    for e in empty:
        assert not torch.any(b.dw_gate_up[e]) and not torch.any(b.dw_down[e]), e
    valid = lay.perm_src >= 0
    F = wd.shape[2]
    errs = {}
    if prec == "bf16":
        lay_ref = mlp.Layout(idx, p, E, 32)
        y_ref, saved = mlp.fwd_grouped(x, wgu, wd, lay_ref, keep=True)
        ref = mlp.bwd_grouped(dy, wgu, wd, lay_ref, saved)
        errs = dict(y=rel_f(f64(o["y"]), y_ref), dx=rel_f(f64(o["dx"]), ref["dx"]),
                    dw_gate_up=rel_f(np.stack([f64(t) for t in b.dw_gate_up]), ref["dw_gate_up"]),
                    dw_down=rel_f(np.stack([f64(t) for t in b.dw_down]), ref["dw_down"]),
                    d_prob=rel_f(f64(b.d_prob), ref["d_prob"]))
        say("[gpu] edge rel_F", {kk: f"{v:.2e}" for kk, v in errs.items()})
        for kk, v in errs.items():
            assert v <= BF16_TOL, (kk, v)
        return
    # MXFP8, staged on the GPU's own codes
    wq, dq = o["wq"], o["dq"]
    for e in range(E):
        q, s = mx.quantize_rows(wgu[e])
        np.testing.assert_array_equal(npy(wq[0][e]), q)
        np.testing.assert_array_equal(npy(wq[1][e]), s)
        q, s = mx.quantize_cols(wd[e])
        np.testing.assert_array_equal(npy(dq[2][e]), q)
        np.testing.assert_array_equal(npy(dq[3][e]), s)
    X = lay.gather(x)
    q, s = mx.quantize_rows(X)
    np.testing.assert_array_equal(npy(g.x_perm), q)
    np.testing.assert_array_equal(npy(g.x_perm_scale), s)
    q, s = mx.quantize_cols(X)
    np.testing.assert_array_equal(npy(g.x_col), q)
    np.testing.assert_array_equal(npy(g.x_col_scale), s)
    DY = lay.gather(dy)
    q, s = mx.quantize_rows(DY)
    np.testing.assert_array_equal(npy(b.dy_row), q)
    q, s = mx.quantize_cols(DY)
    np.testing.assert_array_equal(npy(b.dy_col), q)
    lst = lambda t: [npy(u) for u in t]   # noqa: E731
    G, U, h = mlp.mx_gateup_stage(npy(g.x_perm), npy(g.x_perm_scale), lst(wq[0]), lst(wq[1]), lay)
    gu = f64(f.saved_gu)
    errs["G"] = rel_f(gu[valid, :F], G[valid])
    errs["U"] = rel_f(gu[valid, F:], U[valid])
    hq, hs = mx.quantize_rows(h)
    errs["h"] = rel_f(mx.dequantize_rows(npy(f.h), npy(f.h_scale))[valid], mx.dequantize_rows(hq, hs)[valid])
    fl_h = float(np.mean(npy(f.h)[valid] != hq[valid]))
    nrow = int(lay.off[-1])
    hcq, hcs = mx.quantize_cols(h)
    errs["h_col"] = rel_f(mx.dequantize_rows(npy(f.h_col), npy(f.h_col_scale))[:, :nrow],
                          mx.dequantize_rows(hcq, hcs)[:, :nrow])
    Y = mlp.mx_down_stage(npy(f.h), npy(f.h_scale), lst(dq[0]), lst(dq[1]), lay)
    errs["y_perm"] = rel_f(f64(f.y_perm)[valid], Y[valid])
    errs["y"] = rel_f(f64(o["y"]), lay.combine(np.where(valid[:, None], f64(f.y_perm), 0.0)))
    dG, dU, dp_row = mlp.mx_dh_stage(npy(b.dy_row), npy(b.dy_row_scale), lst(dq[2]), lst(dq[3]), gu[:, :F],
                                     gu[:, F:], lay)
    dGU = np.concatenate([dG, dU], axis=1)
    dGU[~valid] = 0.0
    q, s = mx.quantize_rows(dGU)
    errs["dgu_row"] = rel_f(mx.dequantize_rows(npy(b.dgu_row), npy(b.dgu_row_scale))[valid],
                            mx.dequantize_rows(q, s)[valid])
    fl_g = float(np.mean(npy(b.dgu_row)[valid] != q[valid]))
    errs["d_prob"] = rel_f(f64(b.d_prob), lay.to_slots(dp_row))
    dWd = mlp.mx_dw_stage(npy(b.dy_col), npy(b.dy_col_scale), npy(f.h_col), npy(f.h_col_scale), lay)
    errs["dw_down"] = rel_f(np.stack([f64(t) for t in b.dw_down]), dWd)
    dX = mlp.mx_dx_stage(npy(b.dgu_row), npy(b.dgu_row_scale), lst(wq[2]), lst(wq[3]), lay)
    errs["dx_perm"] = rel_f(f64(b.dx_perm)[valid], dX[valid])
    dWgu = mlp.mx_dw_stage(npy(b.dgu_col), npy(b.dgu_col_scale), npy(g.x_col), npy(g.x_col_scale), lay)
    errs["dw_gate_up"] = rel_f(np.stack([f64(t) for t in b.dw_gate_up]), dWgu)
    errs["dx"] = rel_f(f64(o["dx"]), lay.combine(np.where(valid[:, None], f64(b.dx_perm), 0.0)))
    # bf16-stored stage outputs with few elements: (GPU, oracle) pairs for the element bound
    pairs = dict(G=(gu[valid, :F], G[valid]), U=(gu[valid, F:], U[valid]), y_perm=(f64(f.y_perm)[valid], Y[valid]),
                 y=(f64(o["y"]), lay.combine(np.where(valid[:, None], f64(f.y_perm), 0.0))),
                 dx_perm=(f64(b.dx_perm)[valid], dX[valid]),
                 dx=(f64(o["dx"]), lay.combine(np.where(valid[:, None], f64(b.dx_perm), 0.0))))
    small = {kk: v for kk, v in pairs.items() if v[1].size < 4096}
    say("[gpu] edge staged rel_F", {kk: f"{v:.2e}" for kk, v in errs.items()}, f"flips h {fl_h:.1e} dGU {fl_g:.1e}")
    for kk, v in errs.items():
        if v > MX_TOL and kk in small:
            # under 4096 elements the rel_F of one bf16 rounding (about 1.5e-3 on average)
            # spreads past 2e-3; such a stage is held element by element to one rounding
            # (relative 2^-8 at worst) plus the fp32 accumulation (2^-12 relative, 2^-20
            # of the largest magnitude)
            got, ref = small[kk]
            bound = (2.0 ** -8 + 2.0 ** -12) * np.abs(ref) + 2.0 ** -20 * np.abs(ref).max()
            assert np.all(np.abs(got - ref) <= bound), (kk, v, float(np.max(np.abs(got - ref) / (bound + 1e-300))))
            continue
        assert v <= MX_TOL, (kk, v)
    # a single token gives too few codes for a rate: at most one flip there
    n_h, n_g = int(valid.sum()) * F, int(valid.sum()) * 2 * F
    assert fl_h <= max(H_FLIP_MAX, 1.0 / n_h) and fl_g <= max(DGU_FLIP_MAX, 1.0 / n_g), (fl_h, fl_g)


@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
def test_tail_split_rerun_identical(m, prec):
    """Two runs of the case whose dX and down GEMMs end in the quarter-width tail launch give
    the same bits: each output element is one wave's K sum in a fixed order, whichever launch
    computes it."""
    from tests.gpu_helpers import say
    _needs_256_cus("tail_split")
    args = _case("tail_split")
    say("[gpu] edge tail_split rerun", prec)
    a = _run(m, prec, *args)
    b = _run(m, prec, *args)
    v = a["g"].perm_src >= 0            # padding rows of the permuted outputs are not written
    assert torch.equal(a["g"].perm_src, b["g"].perm_src)
    assert torch.equal(a["f"].y_perm[v], b["f"].y_perm[v]) and torch.equal(a["b"].dx_perm[v], b["b"].dx_perm[v])
    assert torch.equal(a["y"], b["y"]) and torch.equal(a["dx"], b["dx"])
    assert all(torch.equal(u, v) for u, v in zip(a["b"].dw_gate_up, b["b"].dw_gate_up))
    assert all(torch.equal(u, v) for u, v in zip(a["b"].dw_down, b["b"].dw_down))
    assert torch.equal(a["b"].d_prob, b["b"].d_prob)
