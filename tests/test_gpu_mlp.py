"""GPU parity of grouped_mlp_fwd / grouped_mlp_bwd / unpermute_combine against the oracle.

BF16 path: end to end against the pure fp64 oracle on the same bf16 inputs,
rel_F <= 1e-2 for y, dx, dW_gate_up, dW_down and d_prob.
MXFP8 path: staged — each stage is compared with the oracle stage fed the GPU's own
quantized inputs to that stage (x, dy and the weights are themselves checked
bit-exact); rel_F <= 2e-3.  Quantized GPU outputs whose fp32 pre-quantization values
differ from fp64 by rounding (h, dGU) are compared after dequantization with the
oracle's quantization of its own fp64 values; the code flip rate is reported.
"""
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
# E4M3 code flips of the quantities the GPU quantizes from its own fp32 values (h in the
# gate-up epilogue, dG and dU in the dh epilogue) against the oracle's quantization of
# its fp64 values of the same stage: about 2x the rates measured on MI355X (h
# 1.4-2.0e-3, dGU 0.8-0.9e-3; the fp32 accumulation of the block-scaled MFMA differs
# from fp64 by about 1e-4 relative, measured by the f32 down stage below)
H_FLIP_MAX = 4e-3
DGU_FLIP_MAX = 2e-3


@pytest.fixture(scope="module")
def m():
    import moe_grouped_expert_amd as mge
    return mge


def deq(c, s):
    return mx.dequantize_rows(c.detach().cpu().numpy(), s.detach().cpu().numpy())


def flip_rate(a, b):
    return float(np.mean(a != b))


# ------------------------------------------------------------------------------ BF16

BF16_CASES = [
    synth.WORKLOADS[0],
    synth.custom(100, T=300, E=3, H=96, F=160, k=2),
    synth.custom(101, T=40, E=1, H=64, F=64, k=1),
    synth.custom(102, T=700, E=6, H=128, F=256, k=3),
    # the limits: 256 experts, top-8, about 9 assignments per expert and some experts empty
    synth.custom(104, T=300, E=256, H=64, F=64, k=8),
]


def run_bf16(m, inp, train=True):
    w = inp.w
    g = m.moe_route_permute(inp.g_logits, inp.g_x, w.k, align=32, prec="bf16", want_col=train)
    f = m.grouped_mlp_fwd(g, inp.g_wgu, inp.g_wd, y_dtype="bf16", train=train)
    y = m.unpermute_combine(f.y_perm, g.perm_pos)
    out = dict(g=g, f=f, y=y)
    if train:
        b = m.grouped_mlp_bwd(inp.g_dy, g, f, inp.g_wgu, inp.g_wd)
        out["b"] = b
        out["dx"] = m.unpermute_combine(b.dx_perm, g.perm_pos)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("w", BF16_CASES, ids=lambda w: w.name)
def test_bf16_fwd_bwd_vs_fp64(m, w):
    from tests.gpu_helpers import Inputs, f64, npy, say
    say("[gpu] bf16 fwd+bwd", w)
    inp = Inputs(w)
    o = run_bf16(m, inp)
    idx, p = rt.route(inp.logits, w.k)
    np.testing.assert_array_equal(npy(o["g"].topk_idx), idx)
    lay = mlp.Layout(idx, p, w.E, 32)
    y_ref, saved = mlp.fwd_grouped(inp.x, inp.wgu, inp.wd, lay, keep=True)
    g_ref = mlp.bwd_grouped(inp.dy, inp.wgu, inp.wd, lay, saved)
    errs = dict(
        y=rel_f(f64(o["y"]), y_ref),
        dx=rel_f(f64(o["dx"]), g_ref["dx"]),
        dw_gate_up=rel_f(np.stack([f64(t) for t in o["b"].dw_gate_up]), g_ref["dw_gate_up"]),
        dw_down=rel_f(np.stack([f64(t) for t in o["b"].dw_down]), g_ref["dw_down"]),
        d_prob=rel_f(f64(o["b"].d_prob), g_ref["d_prob"]),
    )
    say("[gpu] rel_F", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= BF16_TOL, (k, v)


def test_bf16_empty_experts(m):
    from tests.gpu_helpers import Inputs, f64, say
    w = synth.custom(103, T=200, E=5, H=64, F=96, k=2)
    say("[gpu] bf16 empty experts")
    l = synth.logits(w)
    l[:, 0] = -1e30
    l[:, 3] = -1e30
    inp = Inputs(w, logits=l)
    o = run_bf16(m, inp)
    idx, p = rt.route(l, w.k)
    lay = mlp.Layout(idx, p, w.E, 32)
    assert lay.sizes[0] == 0 and lay.sizes[3] == 0
    y_ref, saved = mlp.fwd_grouped(inp.x, inp.wgu, inp.wd, lay, keep=True)
    g_ref = mlp.bwd_grouped(inp.dy, inp.wgu, inp.wd, lay, saved)
    assert rel_f(f64(o["y"]), y_ref) <= BF16_TOL
    for e in (0, 3):
        assert not torch.any(o["b"].dw_gate_up[e]) and not torch.any(o["b"].dw_down[e])
    assert rel_f(np.stack([f64(t) for t in o["b"].dw_down]), g_ref["dw_down"]) <= BF16_TOL


# ------------------------------------------------------------------------------ MXFP8

MX_CASES = [
    synth.custom(200, T=512, E=4, H=256, F=512, k=2, prec="mxfp8"),
    synth.custom(201, T=300, E=5, H=96, F=160, k=2, prec="mxfp8"),
    synth.custom(202, T=1100, E=8, H=512, F=384, k=2, prec="mxfp8"),
    synth.custom(203, T=64, E=1, H=128, F=128, k=1, prec="mxfp8"),
    # many small groups: 64 experts, top-4, about 12 rows each (one partial tile per group)
    synth.custom(205, T=200, E=64, H=64, F=96, k=4, prec="mxfp8"),
    # the limits: 256 experts, top-8, about 9 assignments per expert and some experts empty
    synth.custom(206, T=300, E=256, H=64, F=64, k=8, prec="mxfp8"),
]


def run_mx(m, inp, y_dtype="bf16"):
    w = inp.w
    g = m.moe_route_permute(inp.g_logits, inp.g_x, w.k, align=32, prec="mxfp8", want_col=True)
    wq = m.mxfp8_quantize(inp.g_wgu, "both")
    dq = m.mxfp8_quantize(inp.g_wd, "both")
    f = m.grouped_mlp_fwd(g, wq[0], dq[0], wq[1], dq[1], y_dtype=y_dtype, train=True)
    y = m.unpermute_combine(f.y_perm, g.perm_pos)
    b = m.grouped_mlp_bwd(inp.g_dy, g, f, wq[2], dq[2], wq[3], dq[3], keep_intermediates=True)
    dx = m.unpermute_combine(b.dx_perm, g.perm_pos)
    torch.cuda.synchronize()
    return dict(g=g, wq=wq, dq=dq, f=f, y=y, b=b, dx=dx)


@pytest.mark.parametrize("w", MX_CASES, ids=lambda w: w.name)
def test_mxfp8_staged(m, w):
    from tests.gpu_helpers import Inputs, f64, layout_from_gpu, npy, say
    say("[gpu] mxfp8 staged", w)
    inp = Inputs(w)
    o = run_mx(m, inp)
    g, f, b = o["g"], o["f"], o["b"]
    lay = layout_from_gpu(g, w.E, 32)
    idx, _ = rt.route(inp.logits, w.k)
    np.testing.assert_array_equal(lay.topk_idx, idx)
    valid = npy(g.perm_src) >= 0
    E, F = w.E, w.F
    # weights: bit-exact codes, both orientations
    for e in range(E):
        q, s = mx.quantize_rows(inp.wgu[e])
        np.testing.assert_array_equal(npy(o["wq"][0][e]), q)
        np.testing.assert_array_equal(npy(o["wq"][1][e]), s)
        qc, sc = mx.quantize_cols(inp.wgu[e])
        np.testing.assert_array_equal(npy(o["wq"][2][e]), qc)
        np.testing.assert_array_equal(npy(o["wq"][3][e]), sc)
        q, s = mx.quantize_rows(inp.wd[e])
        np.testing.assert_array_equal(npy(o["dq"][0][e]), q)
        qc, sc = mx.quantize_cols(inp.wd[e])
        np.testing.assert_array_equal(npy(o["dq"][2][e]), qc)
    xq, xs = npy(g.x_perm), npy(g.x_perm_scale)
    q, s = mx.quantize_rows(lay.gather(inp.x))
    np.testing.assert_array_equal(xq, q)
    np.testing.assert_array_equal(xs, s)
    wgu_q = [npy(o["wq"][0][e]) for e in range(E)]
    wgu_s = [npy(o["wq"][1][e]) for e in range(E)]
    wd_q = [npy(o["dq"][0][e]) for e in range(E)]
    wd_s = [npy(o["dq"][1][e]) for e in range(E)]
    errs = {}
    # S2: gate-up + SwiGLU x p (+ quantize h)
    G, U, h = mlp.mx_gateup_stage(xq, xs, wgu_q, wgu_s, lay)
    gu = f64(f.saved_gu)
    errs["G"] = rel_f(gu[valid, :F], G[valid])
    errs["U"] = rel_f(gu[valid, F:], U[valid])
    hq_ref, hs_ref = mx.quantize_rows(h)
    errs["h"] = rel_f(deq(f.h, f.h_scale)[valid], mx.dequantize_rows(hq_ref, hs_ref)[valid])
    flips = flip_rate(npy(f.h)[valid], hq_ref[valid])
    hcq, hcs = mx.quantize_cols(h)
    nrow = int(npy(g.group_offsets)[-1])   # column forms are written up to the last group's end
    errs["h_col"] = rel_f(deq(f.h_col, f.h_col_scale)[:, :nrow], mx.dequantize_rows(hcq, hcs)[:, :nrow])
    # S3: down GEMM on the GPU's own h codes
    Y = mlp.mx_down_stage(npy(f.h), npy(f.h_scale), wd_q, wd_s, lay)
    errs["y_perm"] = rel_f(f64(f.y_perm)[valid], Y[valid])
    # S4: combine
    errs["y"] = rel_f(f64(o["y"]), lay.combine(np.where(valid[:, None], f64(f.y_perm), 0.0)))
    # b1: dy row / column forms bit-exact
    DY = lay.gather(inp.dy)
    q, s = mx.quantize_rows(DY)
    np.testing.assert_array_equal(npy(b.dy_row), q)
    np.testing.assert_array_equal(npy(b.dy_row_scale), s)
    q, s = mx.quantize_cols(DY)
    np.testing.assert_array_equal(npy(b.dy_col), q)
    np.testing.assert_array_equal(npy(b.dy_col_scale), s)
    # b2 + b3: dh GEMM, SwiGLU backward, d_prob
    wdc_q = [npy(o["dq"][2][e]) for e in range(E)]
    wdc_s = [npy(o["dq"][3][e]) for e in range(E)]
    dG, dU, dp_row = mlp.mx_dh_stage(npy(b.dy_row), npy(b.dy_row_scale), wdc_q, wdc_s, gu[:, :F], gu[:, F:], lay)
    dGU = np.concatenate([dG, dU], axis=1)
    dGU[~valid] = 0.0
    q, s = mx.quantize_rows(dGU)
    errs["dgu_row"] = rel_f(deq(b.dgu_row, b.dgu_row_scale)[valid], mx.dequantize_rows(q, s)[valid])
    flips_dgu = flip_rate(npy(b.dgu_row)[valid], q[valid])
    qc, sc = mx.quantize_cols(dGU)
    errs["dgu_col"] = rel_f(deq(b.dgu_col, b.dgu_col_scale)[:, :nrow], mx.dequantize_rows(qc, sc)[:, :nrow])
    errs["d_prob"] = rel_f(f64(b.d_prob), lay.to_slots(dp_row))
    # b4: dW_down on the GPU's column forms
    dWd = mlp.mx_dw_stage(npy(b.dy_col), npy(b.dy_col_scale), npy(f.h_col), npy(f.h_col_scale), lay)
    errs["dw_down"] = rel_f(np.stack([f64(t) for t in b.dw_down]), dWd)
    # b5: dX on the GPU's dGU row form
    wgc_q = [npy(o["wq"][2][e]) for e in range(E)]
    wgc_s = [npy(o["wq"][3][e]) for e in range(E)]
    dX = mlp.mx_dx_stage(npy(b.dgu_row), npy(b.dgu_row_scale), wgc_q, wgc_s, lay)
    errs["dx_perm"] = rel_f(f64(b.dx_perm)[valid], dX[valid])
    # b6: dW_gate_up on the GPU's column forms
    dWgu = mlp.mx_dw_stage(npy(b.dgu_col), npy(b.dgu_col_scale), npy(g.x_col), npy(g.x_col_scale), lay)
    errs["dw_gate_up"] = rel_f(np.stack([f64(t) for t in b.dw_gate_up]), dWgu)
    # b7: combine of dx
    errs["dx"] = rel_f(f64(o["dx"]), lay.combine(np.where(valid[:, None], f64(b.dx_perm), 0.0)))
    say("[gpu] staged rel_F", {k: f"{v:.2e}" for k, v in errs.items()}, f"h flips {flips:.1e} dGU flips {flips_dgu:.1e}")
    for k, v in errs.items():
        assert v <= MX_TOL, (k, v)
    assert flips <= H_FLIP_MAX and flips_dgu <= DGU_FLIP_MAX, (flips, flips_dgu)
    # end to end against the unstaged fp64 MXFP8 pipeline (report; loose bound)
    y_e2e, _ = mlp.mx_fwd_end_to_end(inp.x, inp.wgu, inp.wd, lay)
    e2e = rel_f(f64(o["y"]), y_e2e)
    say("[gpu] end-to-end y rel_F vs fp64 MXFP8 pipeline", f"{e2e:.2e}")
    assert e2e <= 1e-2


def test_mxfp8_deterministic(m):
    from tests.gpu_helpers import Inputs, say
    w = MX_CASES[0]
    say("[gpu] determinism")
    inp = Inputs(w)
    a = run_mx(m, inp)
    b = run_mx(m, inp)
    assert torch.equal(a["y"], b["y"]) and torch.equal(a["dx"], b["dx"])
    assert all(torch.equal(u, v) for u, v in zip(a["b"].dw_gate_up, b["b"].dw_gate_up))
    assert all(torch.equal(u, v) for u, v in zip(a["b"].dw_down, b["b"].dw_down))
    assert torch.equal(a["b"].d_prob, b["b"].d_prob)


def test_mxfp8_empty_experts_zero_grad(m):
    from tests.gpu_helpers import Inputs, say
    w = synth.custom(204, T=400, E=6, H=128, F=192, k=2, prec="mxfp8")
    say("[gpu] mxfp8 empty experts")
    l = synth.logits(w)
    l[:, 1] = -1e30
    l[:, 5] = -1e30
    inp = Inputs(w, logits=l)
    o = run_mx(m, inp)
    for e in (1, 5):
        assert not torch.any(o["b"].dw_gate_up[e]) and not torch.any(o["b"].dw_down[e])
    assert torch.any(o["b"].dw_gate_up[0])


@pytest.mark.parametrize("w", [MX_CASES[0], MX_CASES[2]], ids=lambda w: w.name)
def test_mxfp8_down_stage_f32(m, w):
    """y_perm in fp32 (y_dtype F32): the down GEMM's output without the bf16 rounding,
    against the oracle's block-scaled product on the GPU's own h and W_down codes.  This
    measures the accumulation of the block-scaled MFMA itself (fp32 accumulators,
    K = F); the end-to-end y against the unstaged fp64 MXFP8 pipeline is reported
    beside it (it carries h's code flips and one bf16 rounding, of y)."""
    from tests.gpu_helpers import Inputs, f64, layout_from_gpu, npy, say
    say("[gpu] mxfp8 f32 down stage", w)
    inp = Inputs(w)
    o = run_mx(m, inp, y_dtype="f32")
    g, f = o["g"], o["f"]
    assert f.y_perm.dtype == torch.float32
    lay = layout_from_gpu(g, w.E, 32)
    valid = npy(g.perm_src) >= 0
    wd_q = [npy(o["dq"][0][e]) for e in range(w.E)]
    wd_s = [npy(o["dq"][1][e]) for e in range(w.E)]
    Y = mlp.mx_down_stage(npy(f.h), npy(f.h_scale), wd_q, wd_s, lay)
    err = rel_f(f64(f.y_perm)[valid], Y[valid])
    # gate-up: the product before the epilogue is only visible through h; the h codes'
    # flip rate against the oracle fed the GPU's x and weight codes
    G, U, h = mlp.mx_gateup_stage(npy(g.x_perm), npy(g.x_perm_scale), [npy(t) for t in o["wq"][0]],
                                  [npy(t) for t in o["wq"][1]], lay)
    hq, _ = mx.quantize_rows(h)
    flips = flip_rate(npy(f.h)[valid], hq[valid])
    y_e2e, _ = mlp.mx_fwd_end_to_end(inp.x, inp.wgu, inp.wd, lay)
    e2e = rel_f(f64(o["y"]), y_e2e)
    say(f"[gpu] f32 y_perm stage rel_F {err:.2e}; h flips {flips:.1e}; end-to-end y rel_F {e2e:.2e}")
    assert err <= 5e-4, err
    assert flips <= H_FLIP_MAX
    assert e2e <= 1e-2, e2e   # reported: h's code flips move y by more than the staged bound

