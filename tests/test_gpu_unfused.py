"""GPU parity of grouped_mlp_fwd_unfused (the forward without the gate-up/SwiGLU fusion)
against the oracle, stage by stage, each stage fed the GPU's own inputs to it:

  1. [G U] bf16 from the grouped gate-up GEMM: against the oracle's GEMM on the GPU's
     x and weight codes (MXFP8) or on the bf16 inputs (BF16);
  2. h bf16 = p * silu(G) * U from the GPU's bf16 G, U (padding rows exactly 0);
  3. MXFP8: the codes and scales of h, bit-exact against the oracle's quantization of
     the GPU's bf16 h (the quantizer's input is exact on both sides);
  4. y_perm: against the oracle's down GEMM on the GPU's h (codes or bf16).
Tolerance rel_F 2e-3 (MXFP8) and 1e-2 (BF16) per stage, each stage holding one bf16
rounding.  At full size (Mixtral shape, MXFP8, 16384 tokens) the same stages on sampled
rows of the largest and the smallest expert, as bench.py times the unfused variant.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import mlp, mx
from oracle.metrics import rel_f

pytestmark = pytest.mark.gpu

CASES = [
    ("mxfp8", synth.custom(1300, T=600, E=4, H=128, F=256, k=2), (), 32),
    ("mxfp8", synth.custom(1301, T=333, E=5, H=96, F=160, k=2), (0, 4), 32),
    ("bf16", synth.custom(1302, T=500, E=3, H=64, F=192, k=2), (1,), 32),
    ("mxfp8", synth.custom(1303, T=421, E=6, H=64, F=96, k=2), (3,), 8),    # groups start at multiples of 8
    ("bf16", synth.custom(1304, T=257, E=3, H=64, F=64, k=1), (), 1),       # unpadded groups
]


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("prec,w,empty,align", CASES,
                         ids=["mx", "mx_empty_ends", "bf16_empty_mid", "mx_align8", "bf16_align1"])
def test_unfused_forward_staged(prec, w, empty, align):
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import Inputs, layout_from_gpu, npy, say

    logits = synth.logits(w)
    for e in empty:
        logits[:, e] = np.float32(-1e30)
    inp = Inputs(w, logits)
    say("[gpu] unfused forward", prec, w.name, "empty", empty)
    mx8 = prec == "mxfp8"
    g = m.moe_route_permute(inp.g_logits, inp.g_x, w.k, align=align, prec=prec)
    if mx8:
        wq = m.mxfp8_quantize(inp.g_wgu, "row")
        dq = m.mxfp8_quantize(inp.g_wd, "row")
        f = m.grouped_mlp_fwd_unfused(g, wq[0], dq[0], wq[1], dq[1], keep_intermediates=True)
        fused = m.grouped_mlp_fwd(g, wq[0], dq[0], wq[1], dq[1])
    else:
        f = m.grouped_mlp_fwd_unfused(g, inp.g_wgu, inp.g_wd, keep_intermediates=True)
        fused = m.grouped_mlp_fwd(g, inp.g_wgu, inp.g_wd)
    torch.cuda.synchronize()
    lay = layout_from_gpu(g, w.E, align)
    np.testing.assert_array_equal(npy(g.group_offsets), lay.off)
    for e in empty:
        assert lay.sizes[e] == 0
    valid = npy(g.perm_src) >= 0
    F = w.F
    tol = 2e-3 if mx8 else 1e-2
    errs = {}
    # 1. [G U]
    if mx8:
        GU = mlp.mx_grouped_nt(npy(g.x_perm), npy(g.x_perm_scale), [npy(q) for q in wq[0]],
                               [npy(s) for s in wq[1]], lay)
    else:
        X = lay.gather(inp.x)
        GU = np.zeros((lay.R, 2 * F))
        for e in range(w.E):
            r = lay.rows(e)
            GU[r] = X[r] @ inp.wgu[e].astype(np.float64).T
    gu = _np(f.gu)
    errs["gu"] = rel_f(gu[valid], GU[valid])
    # 2. h = p * silu(G) * U from the GPU's G, U
    h_gpu = _np(f.h_bf16 if mx8 else f.h)
    p = lay.prob_perm[:, None]
    h_ref = np.where(valid[:, None], p * mlp.silu(gu[:, :F]) * gu[:, F:], 0.0)
    errs["h_bf16"] = rel_f(h_gpu[valid], h_ref[valid])
    assert not np.any(h_gpu[~valid])
    # 3. quantize of h: bit-exact on every row
    if mx8:
        q, s = mx.quantize_rows(h_gpu)
        np.testing.assert_array_equal(npy(f.h), q)
        np.testing.assert_array_equal(npy(f.h_scale), s)
        hd = mx.dequantize_rows(q, s)
        Y = mlp.mx_grouped_nt(q, s, [npy(c) for c in dq[0]], [npy(c) for c in dq[1]], lay)
        flips = float(np.mean(_np(f.h)[valid] != _np(fused.h)[valid]))
    else:
        hd = h_gpu
        Y = np.zeros((lay.R, w.H))
        for e in range(w.E):
            r = lay.rows(e)
            Y[r] = hd[r] @ inp.wd[e].astype(np.float64).T
        flips = float(np.mean(_np(f.h)[valid] != _np(fused.h)[valid]))
    # 4. y_perm
    errs["y_perm"] = rel_f(_np(f.y_perm)[valid], Y[valid])
    d_fused = rel_f(_np(f.y_perm)[valid], _np(fused.y_perm)[valid])
    say("[gpu] unfused", prec, {kk: f"{v:.2e}" for kk, v in errs.items()},
        f"h codes differing from the fused path {flips:.3%}, y_perm rel diff {d_fused:.2e}")
    for key, v in errs.items():
        assert v <= tol, (key, v)


def test_mixtral_unfused_forward_sampled():
    import bench
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import layout_from_gpu, npy, say

    w = synth.WORKLOADS[2]
    dev = torch.device("cuda:0")
    say("[gpu] full-size unfused forward: inputs")
    inp = bench.make_inputs(w, dev)
    step = bench.Step(m, w, inp, train=False, variant="unfused")
    step.keep_intermediates = True
    step()
    torch.cuda.synchronize()
    g, f = step.g, step.f
    lay = layout_from_gpu(g, w.E, 32)
    F = w.F
    rng = np.random.default_rng(7070)
    nonempty = [e for e in range(w.E) if lay.sizes[e] > 0]
    errs = {"gu": [[], []], "h_bf16": [[], []], "y_perm": [[], []]}
    for e in sorted({max(nonempty, key=lambda e: lay.sizes[e]), min(nonempty, key=lambda e: lay.sizes[e])}):
        r = lay.rows(e)
        rows = np.array(sorted({r.start, r.stop - 1} | set(int(v) for v in rng.integers(r.start, r.stop, 4))))
        sel = torch.as_tensor(rows, device=dev, dtype=torch.long)
        xd = mx.dequantize_rows(npy(g.x_perm.index_select(0, sel)), npy(g.x_perm_scale.index_select(0, sel)))
        GU = xd @ mx.dequantize_rows(npy(step.wq[0][e]), npy(step.wq[1][e])).T
        gu = _np(f.gu.index_select(0, sel))
        errs["gu"][0].append(gu)
        errs["gu"][1].append(GU)
        p = npy(g.prob_perm).astype(np.float64)[rows][:, None]
        hb = _np(f.h_bf16.index_select(0, sel))
        errs["h_bf16"][0].append(hb)
        errs["h_bf16"][1].append(p * mlp.silu(gu[:, :F]) * gu[:, F:])
        q, s = mx.quantize_rows(hb)
        np.testing.assert_array_equal(npy(f.h.index_select(0, sel)), q)
        np.testing.assert_array_equal(npy(f.h_scale.index_select(0, sel)), s)
        Y = mx.dequantize_rows(q, s) @ mx.dequantize_rows(npy(step.dq[0][e]), npy(step.dq[1][e])).T
        errs["y_perm"][0].append(_np(f.y_perm.index_select(0, sel)))
        errs["y_perm"][1].append(Y)
    res = {key: rel_f(np.concatenate(a), np.concatenate(b)) for key, (a, b) in errs.items()}
    say("[gpu] full-size unfused", {kk: f"{v:.2e}" for kk, v in res.items()})
    for key, v in res.items():
        assert v <= 2e-3, (key, v)
