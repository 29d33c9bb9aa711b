"""Shared plumbing of the GPU parity tests: build seeded inputs, run the HIP path
through the C ABI, bring results back as numpy."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth
from oracle import mlp
from oracle import route as rt


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def gpu_bf16(a32: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16).to(dev())


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def npy(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


class Inputs:
    """Seeded inputs of one workload, as numpy (exact bf16 values in fp32) and on the GPU."""

    def __init__(self, w: synth.Workload, logits: np.ndarray | None = None):
        self.w = w
        self.logits = synth.logits(w) if logits is None else logits.astype(np.float32)
        self.x = synth.x(w)
        self.wgu = synth.w_gate_up(w)
        self.wd = synth.w_down(w)
        self.dy = synth.dy(w)
        self.g_logits = torch.from_numpy(self.logits).to(dev())
        self.g_x = gpu_bf16(self.x)
        self.g_wgu = gpu_bf16(self.wgu)
        self.g_wd = gpu_bf16(self.wd)
        self.g_dy = gpu_bf16(self.dy)


def layout_from_gpu(route, E: int, align: int) -> mlp.Layout:
    """Oracle layout built from the GPU's routing decision (indices are checked bit-exact
    elsewhere; probabilities are the GPU's fp32 values, an input to the later stages)."""
    return mlp.Layout(npy(route.topk_idx), npy(route.topk_prob).astype(np.float64), E, align)


BF16_TOL = 1e-2      # BF16 path: end to end against fp64 on the same bf16 inputs
MX_TOL = 2e-3        # MXFP8: each stage against the oracle fed the GPU's own quantized operands
H_FLIP_MAX = 4e-3    # code-flip bounds of the epilogue quantizers (fp32 vs fp64 pre-quant values)
DGU_FLIP_MAX = 2e-3


def run_fwd_bwd(m, prec, x, wgu, wd, dy, E, k, idx, prob, logits):
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


def code_flips(gc, gs, rc, rs):
    """GPU codes and scales of a quantized output (blocks of 32 along the last axis) against
    the oracle's codes of the same values: (code flip rate, scale flip rate, every flip valid).

    The GPU quantizes fp32 values that differ from the oracle's fp64 ones by rounding, so a
    value next to a rounding boundary may land on another code (a flip), and a block whose
    amax sits next to a power of two may take the neighbouring scale (a scale flip).  A flip
    is valid when the two dequantized values differ by at most one E4M3 step at their
    magnitude (at the coarser of the two scales) plus 2^-9 of the larger of the block's amax
    and the RMS of the tensor's nonzero values (padding rows are zero on both sides): the
    fp32 pre-quantization error follows the magnitudes the values are computed from (for h,
    about p * 2 * 3e-5 * |U| with G and U of order one, a few times 2^-12 of h's RMS in the
    tails), so an element far below its block's amax, or a block of values near zero, can
    move by more than its own code step.  A scale may differ by more than one step only in
    such a negligible block (amax under 2^-8 of that RMS)."""
    from oracle import mx
    gc, rc = np.asarray(gc), np.asarray(rc)
    gs, rs = np.asarray(gs).astype(np.int32), np.asarray(rs).astype(np.int32)
    ds = gs - rs
    dg, dr = mx.dequantize_rows(gc, gs.astype(np.uint8)), mx.dequantize_rows(rc, rs.astype(np.uint8))
    blk = dr.shape[:-1] + (dr.shape[-1] // 32, 32)
    bmax = np.abs(dr).reshape(blk).max(-1)
    amax = np.repeat(bmax, 32, axis=-1)
    nz = dr[dr != 0]
    rms = float(np.sqrt(np.mean(nz * nz))) if nz.size else 0.0
    scale = np.repeat(np.exp2(np.maximum(gs, rs).astype(np.float64) - 127.0), 32, axis=-1)
    mag = np.maximum(np.abs(dg), np.abs(dr)) / scale
    step = np.exp2(np.floor(np.log2(np.maximum(mag, 2.0 ** -6))) - 3.0) * scale   # subnormal step 2^-9 below 2^-6
    ok = np.abs(dg - dr) <= step + 2.0 ** -9 * np.maximum(amax, rms)
    scale_ok = (np.abs(ds) <= 1) | (bmax <= 2.0 ** -8 * rms)
    valid = bool(np.all(ok) and np.all(scale_ok))
    if not valid:
        bad = np.argwhere(~ok)
        gsx, rsx = np.repeat(gs, 32, axis=-1), np.repeat(rs, 32, axis=-1)
        say("[gpu] invalid flips", len(bad), "of", gc.size, "invalid scale steps:", int(np.sum(~scale_ok)),
            [(tuple(int(v) for v in b), int(gc[tuple(b)]), int(rc[tuple(b)]), int(gsx[tuple(b)]), int(rsx[tuple(b)]),
              float(dg[tuple(b)]), float(dr[tuple(b)]), float(amax[tuple(b)])) for b in bad[:6]])
    return float(np.mean(gc != rc)), float(np.mean(ds != 0)), valid


def flips_within(rate, n, p_max):
    """A flip count over n codes against a bound p_max on the flip probability: at most
    p_max * n plus three standard deviations of a binomial count, plus one (a few hundred
    codes hold too few flips for their rate to settle)."""
    return rate * n <= p_max * n + 3.0 * np.sqrt(p_max * n) + 1.0


def check_fwd_bwd(m, prec, x, wgu, wd, dy, E, k, idx, prob, logits):
    """The whole path (routing or given top-k, permutation, weight quantization, forward,
    backward, combines) on the GPU against the oracle.  BF16: y, dx, dW_gate_up, dW_down and
    d_prob end to end against fp64 on the same bf16 inputs (rel_F 1e-2).  MXFP8: staged, each
    stage against the oracle fed the GPU's own quantized operands (rel_F 2e-3; x, dy, weights
    and the permutation bit-exact; h and dGU compared after dequantization, their code flips
    bounded); a bf16-stored stage output of under 4096 elements whose rel_F exceeds 2e-3 is
    held element by element to one bf16 rounding instead.  The quantized outputs (h in both
    forms, the row form of [dG dU]) must differ from the oracle's codes only by valid flips
    (code_flips), as many as flips_within allows: equal codes dequantize to equal values, so
    their whole difference from the oracle is their flips, each held to one code step, and
    their rel_F (about sqrt(r)/8 at flip rate r) is reported, not bounded again.  d_prob with fewer than 64 values (a few tokens) is a handful of sums whose
    terms may cancel, where a relative error says little; when its rel_F exceeds the bar, each
    value is held to a fraction of the sum of its terms' magnitudes, sum_f |dh silu(G) U|:
    2^-6 in BF16 (the backward uses G and U rounded to bf16, 2^-9 relative each), 2^-10 in
    MXFP8 (fp32 against fp64 arithmetic on the same codes).  Experts without tokens get
    exactly zero weight gradients.  Returns the run's outputs."""
    from oracle import mx
    from oracle.metrics import rel_f
    o = run_fwd_bwd(m, prec, x, wgu, wd, dy, E, k, idx, prob, logits)
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
        say("[gpu] rel_F", {kk: f"{v:.2e}" for kk, v in errs.items()})
        if b.d_prob.numel() < 64 and errs["d_prob"] > BF16_TOL:
            G, U = saved["G"], saved["U"]
            mag = lay_ref.to_slots(np.sum(np.abs(ref["dh"] * (G / (1.0 + np.exp(-G))) * U), axis=1))
            assert np.all(np.abs(f64(b.d_prob) - ref["d_prob"]) <= 2.0 ** -6 * mag), ("d_prob", errs["d_prob"])
            errs.pop("d_prob")
        for kk, v in errs.items():
            assert v <= BF16_TOL, (kk, v)
        return o
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
    fl_h, sfl_h, ok_h = code_flips(npy(f.h)[valid], npy(f.h_scale)[valid], hq[valid], hs[valid])
    nrow = int(lay.off[-1])
    hcq, hcs = mx.quantize_cols(h)
    errs["h_col"] = rel_f(mx.dequantize_rows(npy(f.h_col), npy(f.h_col_scale))[:, :nrow],
                          mx.dequantize_rows(hcq, hcs)[:, :nrow])
    fl_hc, sfl_hc, ok_hc = code_flips(npy(f.h_col)[:, :nrow], npy(f.h_col_scale)[:, :nrow // 32], hcq[:, :nrow],
                                      hcs[:, :nrow // 32])
    fl_hc *= nrow / max(int(valid.sum()), 1)   # a rate over the valid rows (padding rows are zero on both sides)
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
    fl_g, sfl_g, ok_g = code_flips(npy(b.dgu_row)[valid], npy(b.dgu_row_scale)[valid], q[valid], s[valid])
    errs["d_prob"] = rel_f(f64(b.d_prob), lay.to_slots(dp_row))
    if b.d_prob.numel() < 64 and errs["d_prob"] > MX_TOL:
        p_row = npy(g.prob_perm).astype(np.float64)
        mag_row = np.where(valid, np.sum(np.abs(dU * gu[:, F:]), axis=1) / np.where(p_row > 0, p_row, 1.0), 0.0)
        dp_err = np.abs(f64(b.d_prob) - lay.to_slots(dp_row))
        assert np.all(dp_err <= 2.0 ** -10 * lay.to_slots(mag_row)), ("d_prob", errs["d_prob"])
        errs.pop("d_prob")
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
    say("[gpu] staged rel_F", {kk: f"{v:.2e}" for kk, v in errs.items()},
        f"flips h {fl_h:.1e} h_col {fl_hc:.1e} dGU {fl_g:.1e}, scale flips {sfl_h:.1e} {sfl_hc:.1e} {sfl_g:.1e}")
    assert ok_h and ok_hc and ok_g, ("a code or scale that is not a valid flip", ok_h, ok_hc, ok_g)
    flip_rate = dict(h=fl_h, h_col=fl_hc, dgu_row=fl_g)
    for kk, v in errs.items():
        if kk in flip_rate:   # bounded through its flips (code_flips, flips_within)
            continue
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
    # flip counts against their bounds, with the binomial allowance of flips_within
    n_h, n_g = int(valid.sum()) * F, int(valid.sum()) * 2 * F
    assert flips_within(fl_h, n_h, H_FLIP_MAX) and flips_within(fl_g, n_g, DGU_FLIP_MAX), (fl_h, fl_g)
    assert flips_within(fl_hc, n_h, H_FLIP_MAX), fl_hc
    n_hb, n_gb = max(n_h // 32, 1), max(n_g // 32, 1)   # scale flips: the same bounds per block
    assert flips_within(sfl_h, n_hb, H_FLIP_MAX) and flips_within(sfl_hc, n_hb, H_FLIP_MAX), (sfl_h, sfl_hc)
    assert flips_within(sfl_g, n_gb, DGU_FLIP_MAX), sfl_g
    return o
