"""GPU parity of the grouped MLP's remaining modes, against the oracle.

* Inference (no saved activations) with group starts that are not padded to 32 rows
  (align 1 and 8): neighbouring experts' rows are adjacent, so a tile's stores past
  its group's last row would overwrite the next group.  Every valid row is checked on
  its own, BF16 end to end against fp64 and MXFP8 stage by stage, with bf16 and f32
  down-projection outputs.
* The backward's accumulate flag: a second call with accumulate adds the same
  gradient again, so dW must be exactly twice the first call's (x + x is exact in
  fp32), and experts without tokens keep whatever their buffers held.
* bf16 weight gradients: the same K loop as the fp32 ones with a rounding epilogue, so
  they must equal the fp32 call's dW rounded to nearest even, bit for bit; accumulate
  with bf16 outputs is rejected.
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
ROW_TOL = 3e-2     # per-row relative error bound (a clobbered row is off by O(1))


@pytest.fixture(scope="module")
def m():
    import moe_grouped_expert_amd as mge
    return mge


def row_rel(a, ref, rows):
    """max over `rows` of |a_r - ref_r| / |ref_r|."""
    num = np.linalg.norm(a[rows] - ref[rows], axis=1)
    den = np.maximum(np.linalg.norm(ref[rows], axis=1), 1e-30)
    return float(np.max(num / den))


@pytest.mark.parametrize("align", [1, 8])
@pytest.mark.parametrize("y_dtype", ["bf16", "f32"])
def test_bf16_inference_unpadded(m, align, y_dtype):
    from tests.gpu_helpers import Inputs, f64, npy, say
    w = synth.custom(110 + align, T=300, E=5, H=96, F=160, k=2)
    say("[gpu] bf16 inference align", align, y_dtype)
    inp = Inputs(w)
    g = m.moe_route_permute(inp.g_logits, inp.g_x, w.k, align=align, prec="bf16")
    f = m.grouped_mlp_fwd(g, inp.g_wgu, inp.g_wd, y_dtype=y_dtype, train=False)
    y = m.unpermute_combine(f.y_perm, g.perm_pos)
    torch.cuda.synchronize()
    idx, p = rt.route(inp.logits, w.k)
    np.testing.assert_array_equal(npy(g.topk_idx), idx)
    lay = mlp.Layout(idx, p, w.E, align)
    np.testing.assert_array_equal(npy(g.group_offsets), lay.off)
    y_ref, saved = mlp.fwd_grouped(inp.x, inp.wgu, inp.wd, lay, keep=True)
    valid = npy(g.perm_src) >= 0
    e_y = rel_f(f64(y), y_ref)
    e_rows = row_rel(f64(f.y_perm), saved["Y"], valid)
    e_h = row_rel(f64(f.h), saved["h"], valid)
    say("[gpu] rel_F y", f"{e_y:.2e}", "max row y_perm", f"{e_rows:.2e}", "max row h", f"{e_h:.2e}")
    assert e_y <= BF16_TOL and e_rows <= ROW_TOL and e_h <= ROW_TOL


@pytest.mark.parametrize("align", [1, 8])
@pytest.mark.parametrize("y_dtype", ["bf16", "f32"])
def test_mxfp8_inference_unpadded(m, align, y_dtype):
    from tests.gpu_helpers import Inputs, f64, layout_from_gpu, npy, say
    w = synth.custom(120 + align, T=500, E=6, H=128, F=192, k=2, prec="mxfp8")
    say("[gpu] mxfp8 inference align", align, y_dtype)
    inp = Inputs(w)
    g = m.moe_route_permute(inp.g_logits, inp.g_x, w.k, align=align, prec="mxfp8")
    wq = m.mxfp8_quantize(inp.g_wgu, "row")
    dq = m.mxfp8_quantize(inp.g_wd, "row")
    f = m.grouped_mlp_fwd(g, wq[0], dq[0], wq[1], dq[1], y_dtype=y_dtype, train=False)
    y = m.unpermute_combine(f.y_perm, g.perm_pos)
    torch.cuda.synchronize()
    lay = layout_from_gpu(g, w.E, align)
    idx, _ = rt.route(inp.logits, w.k)
    np.testing.assert_array_equal(lay.topk_idx, idx)
    valid = npy(g.perm_src) >= 0
    xq, xs = npy(g.x_perm), npy(g.x_perm_scale)
    q, s = mx.quantize_rows(lay.gather(inp.x))
    np.testing.assert_array_equal(xq, q)
    np.testing.assert_array_equal(xs, s)
    E = w.E
    wgu_q = [npy(wq[0][e]) for e in range(E)]
    wgu_s = [npy(wq[1][e]) for e in range(E)]
    wd_q = [npy(dq[0][e]) for e in range(E)]
    wd_s = [npy(dq[1][e]) for e in range(E)]
    _, _, h = mlp.mx_gateup_stage(xq, xs, wgu_q, wgu_s, lay)
    hq_ref, hs_ref = mx.quantize_rows(h)
    h_gpu = mx.dequantize_rows(npy(f.h), npy(f.h_scale))
    h_ref = mx.dequantize_rows(hq_ref, hs_ref)
    Y = mlp.mx_down_stage(npy(f.h), npy(f.h_scale), wd_q, wd_s, lay)
    errs = dict(h=rel_f(h_gpu[valid], h_ref[valid]), y_perm=rel_f(f64(f.y_perm)[valid], Y[valid]),
                y=rel_f(f64(y), lay.combine(np.where(valid[:, None], f64(f.y_perm), 0.0))))
    e_rows = row_rel(f64(f.y_perm), Y, valid)
    e_hrows = row_rel(h_gpu, h_ref, valid)
    say("[gpu] staged rel_F", {k: f"{v:.2e}" for k, v in errs.items()}, "max row y_perm", f"{e_rows:.2e}",
        "max row h", f"{e_hrows:.2e}")
    for k, v in errs.items():
        assert v <= MX_TOL, (k, v)
    assert e_rows <= ROW_TOL and e_hrows <= ROW_TOL


@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
def test_bwd_accumulate(m, prec):
    from tests.gpu_helpers import Inputs, say
    w = synth.custom(130, T=400, E=5, H=128, F=160, k=2, prec=prec)
    say("[gpu] backward accumulate", prec)
    l = synth.logits(w)
    l[:, 2] = -1e30                  # expert 2 gets no tokens
    inp = Inputs(w, logits=l)
    g = m.moe_route_permute(inp.g_logits, inp.g_x, w.k, align=32, prec=prec, want_col=True)
    if prec == "mxfp8":
        wq = m.mxfp8_quantize(inp.g_wgu, "both")
        dq = m.mxfp8_quantize(inp.g_wd, "both")
        f = m.grouped_mlp_fwd(g, wq[0], dq[0], wq[1], dq[1], train=True)
        bw = (wq[2], dq[2], wq[3], dq[3])
    else:
        f = m.grouped_mlp_fwd(g, inp.g_wgu, inp.g_wd, train=True)
        bw = (inp.g_wgu, inp.g_wd)
    b1 = m.grouped_mlp_bwd(inp.g_dy, g, f, *bw)
    first_gu = [t.clone() for t in b1.dw_gate_up]
    first_d = [t.clone() for t in b1.dw_down]
    assert torch.any(first_gu[0]) and not torch.any(first_gu[2])
    # the empty expert's buffers hold a marker that accumulating must leave alone
    b1.dw_gate_up[2].fill_(7.0)
    b1.dw_down[2].fill_(-3.0)
    b2 = m.grouped_mlp_bwd(inp.g_dy, g, f, *bw, accumulate=True, out=b1)
    torch.cuda.synchronize()
    for e in range(w.E):
        if e == 2:
            assert torch.all(b2.dw_gate_up[e] == 7.0) and torch.all(b2.dw_down[e] == -3.0)
        else:
            assert torch.equal(b2.dw_gate_up[e], 2.0 * first_gu[e]), e
            assert torch.equal(b2.dw_down[e], 2.0 * first_d[e]), e


@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
def test_bwd_bf16_dw(m, prec):
    from tests.gpu_helpers import Inputs, say
    w = synth.custom(140, T=400, E=5, H=128, F=160, k=2, prec=prec)
    say("[gpu] backward bf16 dW", prec)
    l = synth.logits(w)
    l[:, 3] = -1e30                  # expert 3 gets no tokens
    inp = Inputs(w, logits=l)
    g = m.moe_route_permute(inp.g_logits, inp.g_x, w.k, align=32, prec=prec, want_col=True)
    if prec == "mxfp8":
        wq = m.mxfp8_quantize(inp.g_wgu, "both")
        dq = m.mxfp8_quantize(inp.g_wd, "both")
        f = m.grouped_mlp_fwd(g, wq[0], dq[0], wq[1], dq[1], train=True)
        bw = (wq[2], dq[2], wq[3], dq[3])
    else:
        f = m.grouped_mlp_fwd(g, inp.g_wgu, inp.g_wd, train=True)
        bw = (inp.g_wgu, inp.g_wd)
    b32 = m.grouped_mlp_bwd(inp.g_dy, g, f, *bw)
    b16 = m.grouped_mlp_bwd(inp.g_dy, g, f, *bw, dw_dtype="bf16")
    torch.cuda.synchronize()
    for e in range(w.E):
        assert b16.dw_gate_up[e].dtype == torch.bfloat16 and b16.dw_down[e].dtype == torch.bfloat16
        assert torch.equal(b16.dw_gate_up[e], b32.dw_gate_up[e].to(torch.bfloat16)), e
        assert torch.equal(b16.dw_down[e], b32.dw_down[e].to(torch.bfloat16)), e
    assert not torch.any(b16.dw_gate_up[3]) and not torch.any(b16.dw_down[3])
    valid = g.perm_src >= 0          # dx_perm defines the valid rows only
    assert torch.equal(b16.dx_perm[valid], b32.dx_perm[valid]) and torch.equal(b16.d_prob, b32.d_prob)
    with pytest.raises(m.MgeError):
        m.grouped_mlp_bwd(inp.g_dy, g, f, *bw, accumulate=True, out=b16, dw_dtype="bf16")
