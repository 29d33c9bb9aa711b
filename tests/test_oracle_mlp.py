"""Pins of the expert-MLP oracle (oracle/mlp.py).

* per-token (O-slow) and grouped (O-grouped) forward agree to 1e-12 on the tiny workload;
* one expert, top-1 (p = 1) reduces to the dense SwiGLU MLP written with whole-matrix numpy;
* the backward passes central finite differences of L = <dy, y> in fp64, for x, the
  weights and the routing probabilities (treated as independent inputs);
* empty experts get exactly zero weight gradients;
* the MXFP8 stages reduce to the exact forward when every operand is representable
  (quantization is then the identity), and the ragged dW stage equals its triple-sum
  definition on a tiny case;
* the MXFP8 SwiGLU-backward stage (mx_dh_stage), fed exactly representable dY and
  W_down column codes, equals the finite-difference-pinned grouped backward's dG, dU
  and d_prob (G of both signs and near 0, p != 1);
* the whole MXFP8 forward (mx_fwd_end_to_end) on representable x and weights equals
  the grouped forward up to the quantization of h, which it applies after the
  probability scaling.
"""
import numpy as np
import pytest

import synth
from oracle import mlp, mx
from oracle import route as rt
from oracle.metrics import rel_f


def tiny(seed=0, T=24, E=3, H=32, F=32, k=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    wgu = rng.standard_normal((E, 2 * F, H)) * 0.3
    wd = rng.standard_normal((E, H, F)) * 0.3
    l = rng.standard_normal((T, E)).astype(np.float32)
    return x, wgu, wd, l


def test_per_token_equals_grouped_c0():
    w = synth.WORKLOADS[0]
    x = synth.x(w)
    wgu = synth.w_gate_up(w)
    wd = synth.w_down(w)
    idx, p = rt.route(synth.logits(w), w.k)
    lay = mlp.Layout(idx, p, w.E, 32)
    y1 = mlp.fwd_per_token(x, wgu, wd, idx, p)
    y2 = mlp.fwd_grouped(x, wgu, wd, lay)
    assert rel_f(y2, y1) <= 1e-12
    assert np.abs(y1).max() > 0


def test_dense_special_case():
    rng = np.random.default_rng(4)
    T, H, F = 40, 32, 64
    x = rng.standard_normal((T, H))
    wg = rng.standard_normal((F, H)) * 0.2
    wu = rng.standard_normal((F, H)) * 0.2
    wd = rng.standard_normal((H, F)) * 0.2
    G = x @ wg.T
    dense = ((G / (1 + np.exp(-G))) * (x @ wu.T)) @ wd.T
    idx = np.zeros((T, 1), np.int32)
    p = np.ones((T, 1))
    lay = mlp.Layout(idx, p, 1, 32)
    y = mlp.fwd_grouped(x, np.concatenate([wg, wu])[None], wd[None], lay)
    np.testing.assert_allclose(y, dense, rtol=1e-12, atol=1e-12)
    y_pt = mlp.fwd_per_token(x, np.concatenate([wg, wu])[None], wd[None], idx, p)
    np.testing.assert_allclose(y_pt, dense, rtol=1e-12, atol=1e-12)


def _loss(x, wgu, wd, idx, p, dy, E):
    lay = mlp.Layout(idx, p, E, 32)
    return float(np.sum(dy * mlp.fwd_grouped(x, wgu, wd, lay)))


def test_backward_finite_differences():
    x, wgu, wd, l = tiny()
    T, H = x.shape
    E = wgu.shape[0]
    idx, p = rt.route(l, 2)
    dy = np.random.default_rng(9).standard_normal((T, H))
    lay = mlp.Layout(idx, p, E, 32)
    _, saved = mlp.fwd_grouped(x, wgu, wd, lay, keep=True)
    g = mlp.bwd_grouped(dy, wgu, wd, lay, saved)
    args = dict(x=x, wgu=wgu, wd=wd, p=p)
    grads = dict(x=g["dx"], wgu=g["dw_gate_up"], wd=g["dw_down"], p=g["d_prob"])

    def L(a):
        return _loss(a["x"], a["wgu"], a["wd"], idx, a["p"], dy, E)

    rng = np.random.default_rng(21)
    for name in args:
        base = args[name]
        scale = np.abs(base).max()
        eps = 1e-6 * scale
        # random directional derivatives
        for _ in range(5):
            d = rng.standard_normal(base.shape)
            ap = dict(args); ap[name] = base + eps * d
            am = dict(args); am[name] = base - eps * d
            fd = (L(ap) - L(am)) / (2 * eps)
            an = float(np.sum(grads[name] * d))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)
        # sampled coordinates
        flat = base.ravel()
        for j in rng.choice(flat.size, size=min(50, flat.size), replace=False):
            bp = flat.copy(); bp[j] += eps
            bm = flat.copy(); bm[j] -= eps
            ap = dict(args); ap[name] = bp.reshape(base.shape)
            am = dict(args); am[name] = bm.reshape(base.shape)
            fd = (L(ap) - L(am)) / (2 * eps)
            an = grads[name].ravel()[j]
            assert abs(fd - an) <= 1e-7 * max(1.0, np.abs(grads[name]).max()), (name, j, fd, an)


def test_empty_experts_zero_grads():
    x, wgu, wd, l = tiny(E=4)
    l[:, 1] = -1e30
    l[:, 3] = -1e30
    idx, p = rt.route(l, 2)
    lay = mlp.Layout(idx, p, 4, 32)
    assert lay.sizes[1] == 0 and lay.sizes[3] == 0
    _, saved = mlp.fwd_grouped(x, wgu, wd, lay, keep=True)
    g = mlp.bwd_grouped(np.ones_like(x), wgu, wd, lay, saved)
    assert not np.any(g["dw_gate_up"][[1, 3]]) and not np.any(g["dw_down"][[1, 3]])
    assert np.any(g["dw_gate_up"][0])


def _representable(rng, shape):
    """Values exactly representable in MXFP8 with scale 2^-8 per block (amax pinned)."""
    codes = rng.integers(0, 0x79, size=shape)   # magnitudes <= 256 so the pinned 1.0 is the amax
    blk = codes.reshape(shape[:-1] + (shape[-1] // 32, 32))
    blk[..., 0] = 0x78                     # 256 * 2^-8 = 1.0 fixes each block's amax
    vals = mx.e4m3_decode(codes.astype(np.uint8)) * np.where(rng.random(shape) < 0.5, -1, 1)
    vals.reshape(blk.shape)[..., 0] = 256.0
    return vals * 2.0 ** -8


def test_mx_stages_reduce_to_exact_when_representable():
    rng = np.random.default_rng(17)
    T, E, H, F, k = 20, 3, 64, 32, 2
    x = _representable(rng, (T, H))
    wgu = _representable(rng, (E, 2 * F, H))
    wd = _representable(rng, (E, H, F))
    l = rng.standard_normal((T, E)).astype(np.float32)
    idx, p = rt.route(l, k)
    lay = mlp.Layout(idx, p, E, 32)
    y, saved = mlp.fwd_grouped(x, wgu, wd, lay, keep=True)
    X = lay.gather(x)
    xq, xs = mx.quantize_rows(X)
    np.testing.assert_array_equal(mx.dequantize_rows(xq, xs), X)
    wq = [mx.quantize_rows(wgu[e]) for e in range(E)]
    G, U, h = mlp.mx_gateup_stage(xq, xs, [a for a, _ in wq], [b for _, b in wq], lay)
    np.testing.assert_allclose(G, saved["G"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(h, saved["h"], rtol=1e-13, atol=1e-15)
    # down stage fed the exact h (quantize h only where representable: use the exact h directly)
    dq = [mx.quantize_rows(wd[e]) for e in range(E)]
    Wd_dec = [mx.dequantize_rows(a, b) for a, b in dq]
    for e in range(E):
        np.testing.assert_array_equal(Wd_dec[e], wd[e])


def test_mx_dw_stage_triple_sum():
    rng = np.random.default_rng(23)
    idx = np.array([[0, 1], [1, 0], [0, 2], [2, 0]], np.int32)
    p = np.full((4, 2), 0.5)
    lay = mlp.Layout(idx, p, 3, 32)
    NA, NB = 3, 2
    A = np.zeros((lay.R, NA))
    B = np.zeros((lay.R, NB))
    for e in range(3):
        r = lay.rows(e)
        A[r] = rng.standard_normal((r.stop - r.start, NA))
        B[r] = rng.standard_normal((r.stop - r.start, NB))
    aq, as_ = mx.quantize_cols(A)
    bq, bs = mx.quantize_cols(B)
    got = mlp.mx_dw_stage(aq, as_, bq, bs, lay)
    Ad = mx.dequantize_rows(aq, as_)
    Bd = mx.dequantize_rows(bq, bs)
    for e in range(3):
        r = lay.rows(e)
        for i in range(NA):
            for j in range(NB):
                ref = sum(Ad[i, m] * Bd[j, m] for m in range(r.start, r.stop))
                assert abs(got[e, i, j] - ref) <= 1e-12 * (1 + abs(ref))


def _col_representable(rng, shape):
    """[..., R, C] values exactly representable in the column form (blocks of 32 rows)."""
    v = _representable(rng, shape[:-2] + (shape[-1], shape[-2]))
    return np.swapaxes(v, -1, -2)


def test_mx_dh_stage_equals_grouped_backward_on_representable_operands():
    rng = np.random.default_rng(31)
    T, E, H, F, k = 64, 4, 64, 96, 2
    x = rng.standard_normal((T, H))
    wgu = rng.standard_normal((E, 2 * F, H)) * 0.3
    wd = _col_representable(rng, (E, H, F))
    dy = _representable(rng, (T, H))
    l = rng.standard_normal((T, E)).astype(np.float32)
    idx, p = rt.route(l, k)
    lay = mlp.Layout(idx, p, E, 32)
    _, saved = mlp.fwd_grouped(x, wgu, wd, lay, keep=True)
    ref = mlp.bwd_grouped(dy, wgu, wd, lay, saved)
    G, U = saved["G"], saved["U"]
    valid = lay.perm_src >= 0
    # the SwiGLU backward is exercised on both branches of silu' and away from p = 1
    assert (G[valid] < -1).any() and (G[valid] > 1).any() and (np.abs(G[valid]) < 0.05).any()
    assert np.all(lay.prob_perm[valid] < 1) and np.ptp(lay.prob_perm[valid]) > 0.3
    dY = lay.gather(dy)
    dyq, dys = mx.quantize_rows(dY)
    np.testing.assert_array_equal(mx.dequantize_rows(dyq, dys), dY)
    wdc = [mx.quantize_cols(wd[e]) for e in range(E)]
    for e in range(E):
        np.testing.assert_array_equal(mx.dequantize_rows(*wdc[e]), wd[e].T)
    dG, dU, dp_row = mlp.mx_dh_stage(dyq, dys, [a for a, _ in wdc], [b for _, b in wdc], G, U, lay)
    np.testing.assert_allclose(dG[valid], ref["dGU"][valid, :F], rtol=1e-12, atol=1e-12 * np.abs(ref["dGU"]).max())
    np.testing.assert_allclose(dU[valid], ref["dGU"][valid, F:], rtol=1e-12, atol=1e-12 * np.abs(ref["dGU"]).max())
    np.testing.assert_allclose(lay.to_slots(dp_row), ref["d_prob"], rtol=1e-12, atol=1e-12 * np.abs(ref["d_prob"]).max())
    # dG and dU differ (a swap of the two would fail above), and both are non-trivial
    assert rel_f(dG[valid], dU[valid]) > 0.5 and np.abs(dG).max() > 0 and np.abs(dU).max() > 0


def test_mx_fwd_end_to_end_equals_grouped_up_to_h_quantization():
    rng = np.random.default_rng(37)
    T, E, H, F, k = 48, 3, 64, 64, 2
    x = _representable(rng, (T, H))
    wgu = _representable(rng, (E, 2 * F, H))
    wd = _representable(rng, (E, H, F))
    l = rng.standard_normal((T, E)).astype(np.float32)
    idx, p = rt.route(l, k)
    lay = mlp.Layout(idx, p, E, 32)
    y_ref, keep = mlp.fwd_grouped(x, wgu, wd, lay, keep=True)
    y, parts = mlp.mx_fwd_end_to_end(x, wgu, wd, lay)
    # x, W_gate_up and W_down are representable: G, U and h = p * silu(G) * U are exact
    for name in ("G", "U", "h"):
        np.testing.assert_allclose(parts[name], keep[name], rtol=1e-13, atol=1e-15)
    # h is quantized along F after the probability scaling, and only h
    hq, hs = mx.quantize_rows(keep["h"])
    np.testing.assert_array_equal(parts["hq"], hq)
    np.testing.assert_array_equal(parts["hs"], hs)
    hd = mx.dequantize_rows(hq, hs)
    Y = np.zeros((lay.R, H))
    for e in range(E):
        r = lay.rows(e)
        Y[r] = hd[r] @ wd[e].T
    np.testing.assert_allclose(y, lay.combine(Y), rtol=1e-12, atol=1e-12 * np.abs(y).max())
    # the h quantization is the only difference from the exact forward: E4M3 keeps 3
    # mantissa bits (relative rounding error <= 2^-4 on normal values)
    err = rel_f(y, y_ref)
    assert 0 < err < 2.0 ** -4
    # the other reading, p * dequantize(quantize(silu(G) * U)), gives a different y on this
    # input, so the check above tells the two apart
    pr = lay.prob_perm[:, None]
    hq2, hs2 = mx.quantize_rows(silu_u := mlp.silu(keep["G"]) * keep["U"])
    Y2 = np.zeros((lay.R, H))
    for e in range(E):
        r = lay.rows(e)
        Y2[r] = (pr[r] * mx.dequantize_rows(hq2, hs2)[r]) @ wd[e].T
    assert rel_f(y, lay.combine(Y2)) > 1e-4 and silu_u.shape == keep["h"].shape

