"""GPU parity of FP8 with one scale per tensor (the format the pages name beside MXFP8)
against the oracle's quantize_tensor, through the C ABI:

  * mge_tensor_scale: the scale byte of the tensor's amax, bit-exact, over sizes with
    vector tails, a base that is not 16-byte aligned, all-zero and extreme tensors, and
    one scale per matrix of a batch;
  * mxfp8_quantize with tensor_scale: row and column codes bit-exact, every block's scale
    the tensor's;
  * moe_route_permute with x_tensor_scale: the permuted x codes bit-exact (padding rows
    zero codes, the tensor's scale);
  * the FP8 forward (unfused chain, h with one scale from its amax) stage by stage: [G U]
    and y_perm within rel_F 2e-3 of the oracle on the GPU's codes, h's scale and codes
    bit-exact from the GPU's bf16 h; at the Mixtral shape on sampled rows, through
    bench.Step's fp8_tensor variant.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import mlp, mx
from oracle.metrics import rel_f

pytestmark = pytest.mark.gpu


def _bf(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to("cuda:0")


def _vals(t):
    return t.float().cpu().numpy().astype(np.float64)


def _npy(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("n,kind", [(1, "normal"), (7, "normal"), (8, "normal"), (1000, "wide"),
                                    (4096 * 37 + 5, "normal"), (1 << 21, "wide"), (4096, "zero"),
                                    (300, "tiny"), (300, "huge"), (2049, "spike")])
def test_tensor_scale_matches_oracle(n, kind):
    import moe_grouped_expert_amd as m

    rng = np.random.default_rng(n)
    if kind == "zero":
        v = np.zeros(n + 3)
    elif kind == "tiny":
        v = rng.standard_normal(n + 3) * 1e-39          # bf16 subnormals: the scale clamps at 0
    elif kind == "huge":
        v = rng.standard_normal(n + 3) * 1e37
    elif kind == "wide":
        v = rng.standard_normal(n + 3) * np.exp2(rng.uniform(-30, 30, n + 3))
    else:
        v = rng.standard_normal(n + 3)
    if kind == "spike":
        v[n + 2] = -1e4                                  # the amax sits in the unaligned tail
    g = _bf(v)
    for off in (0, 3):                                   # base 16-byte aligned, then 6 bytes past
        t = g[off:off + n]
        got = int(m.tensor_scale(t).scale.item())
        _, ref = mx.quantize_tensor(_vals(t))
        assert got == int(ref), (n, kind, off, got, int(ref))


def test_tensor_scale_per_matrix_and_quantize():
    import moe_grouped_expert_amd as m

    rng = np.random.default_rng(77)
    E, R, C = 3, 70, 96
    w = rng.standard_normal((E, R, C)) * np.array([1e-3, 1.0, 300.0])[:, None, None]
    w[1, 5, 7] = 0.0
    g = _bf(w)
    ts = m.tensor_scale(g, per_matrix=True)
    rc, rs, cc, cs = m.mxfp8_quantize(g, "both", tensor_scale=ts.scale)
    torch.cuda.synchronize()
    wv = _vals(g)
    Rp = (R + 31) // 32 * 32
    for e in range(E):
        q, s = mx.quantize_tensor(wv[e])
        assert int(ts.scale[e]) == int(s)
        np.testing.assert_array_equal(_npy(rc[e]), q)
        assert np.all(_npy(rs[e]) == s)
        np.testing.assert_array_equal(_npy(cc[e])[:, :R], q.T)
        assert not _npy(cc[e])[:, R:].any()
        assert np.all(_npy(cs[e]) == s) and _npy(cs[e]).shape == (C, Rp // 32)


@pytest.mark.parametrize("want_col", [False, True])
def test_route_with_x_tensor_scale(want_col):
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import Inputs

    w = synth.custom(1400, T=300, E=4, H=128, F=64, k=2, prec="mxfp8")
    inp = Inputs(w)
    ts = m.tensor_scale(inp.g_x)
    g = m.moe_route_permute(inp.g_logits, inp.g_x, w.k, align=32, prec="mxfp8", want_col=want_col,
                            x_tensor_scale=ts.scale)
    torch.cuda.synchronize()
    q, s = mx.quantize_tensor(inp.x.astype(np.float64))
    src = _npy(g.perm_src)
    valid = src >= 0
    codes = _npy(g.x_perm)
    np.testing.assert_array_equal(codes[valid], q[src[valid]])
    assert not codes[~valid].any()
    assert np.all(_npy(g.x_perm_scale) == s)
    if want_col:
        np.testing.assert_array_equal(_npy(g.x_col)[:, valid], q[src[valid]].T)
        assert not _npy(g.x_col)[:, ~valid].any()
        assert np.all(_npy(g.x_col_scale) == s)


@pytest.mark.parametrize("w,empty", [(synth.custom(1401, T=600, E=4, H=128, F=256, k=2, prec="mxfp8"), ()),
                                     (synth.custom(1402, T=333, E=5, H=96, F=160, k=2, prec="mxfp8"), (2,))],
                         ids=["plain", "empty_mid"])
def test_fp8_tensor_forward_staged(w, empty):
    import bench
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import Inputs, layout_from_gpu, say

    logits = synth.logits(w)
    for e in empty:
        logits[:, e] = np.float32(-1e30)
    inp = Inputs(w, logits)
    st = bench.Step(m, w, dict(logits=inp.g_logits, x=inp.g_x, wgu=inp.g_wgu, wd=inp.g_wd, dy=None), train=False,
                    variant="fp8_tensor")
    st.keep_intermediates = True
    st()
    torch.cuda.synchronize()
    g, f = st.g, st.f
    lay = layout_from_gpu(g, w.E, 32)
    valid = _npy(g.perm_src) >= 0
    F = w.F
    # the operands: x and every expert's weights with one scale each, bit-exact
    qx, sx = mx.quantize_tensor(inp.x.astype(np.float64))
    np.testing.assert_array_equal(_npy(g.x_perm)[valid], qx[_npy(g.perm_src)[valid]])
    for e in range(w.E):
        for wt, qt in ((inp.wgu, st.wq), (inp.wd, st.dq)):
            q, s = mx.quantize_tensor(wt[e].astype(np.float64))
            np.testing.assert_array_equal(_npy(qt[0][e]), q)
            assert np.all(_npy(qt[1][e]) == s)
    errs = {}
    GU = mlp.mx_grouped_nt(_npy(g.x_perm), _npy(g.x_perm_scale), [_npy(c) for c in st.wq[0]],
                           [_npy(c) for c in st.wq[1]], lay)
    gu = _vals(f.gu)
    errs["gu"] = rel_f(gu[valid], GU[valid])
    hb = _vals(f.h_bf16)
    href = lay.prob_perm[:, None] * mlp.silu(gu[:, :F]) * gu[:, F:]
    errs["h_bf16"] = rel_f(hb[valid], href[valid])
    assert not hb[~valid].any()
    q, s = mx.quantize_tensor(hb)
    assert int(f.h_tensor_scale.item()) == int(s)
    np.testing.assert_array_equal(_npy(f.h), q)
    assert np.all(_npy(f.h_scale) == s)
    Y = mlp.mx_grouped_nt(q, _npy(f.h_scale), [_npy(c) for c in st.dq[0]], [_npy(c) for c in st.dq[1]], lay)
    errs["y_perm"] = rel_f(_vals(f.y_perm)[valid], Y[valid])
    y = lay.combine(_vals(f.y_perm))
    errs["y"] = rel_f(_vals(st.y), y)
    say("[gpu] fp8 per-tensor forward", w.name, {k: f"{v:.2e}" for k, v in errs.items()},
        "scales x/h", int(sx), int(s))
    for key, v in errs.items():
        assert v <= 2e-3, (key, v)


def test_mixtral_fp8_tensor_forward_sampled():
    import bench
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import layout_from_gpu, say

    w = synth.WORKLOADS[2]
    dev = torch.device("cuda:0")
    say("[gpu] full-size fp8 per-tensor forward: inputs")
    inp = bench.make_inputs(w, dev)
    st = bench.Step(m, w, inp, train=False, variant="fp8_tensor")
    st.keep_intermediates = True
    st()
    torch.cuda.synchronize()
    g, f = st.g, st.f
    lay = layout_from_gpu(g, w.E, 32)
    F = w.F
    # scales of x and of every expert's weights against the oracle (amax over the whole tensor)
    assert int(st.ts["x"].scale.item()) == int(mx.block_scale_exponent(float(inp["x"].abs().max())) + 127)
    for e in range(w.E):
        assert int(st.ts["wgu"].scale[e]) == int(mx.block_scale_exponent(float(inp["wgu"][e].abs().max())) + 127)
        assert int(st.ts["wd"].scale[e]) == int(mx.block_scale_exponent(float(inp["wd"][e].abs().max())) + 127)
    assert int(f.h_tensor_scale.item()) == int(mx.block_scale_exponent(float(f.h_bf16.abs().max())) + 127)
    rng = np.random.default_rng(7171)
    nonempty = [e for e in range(w.E) if lay.sizes[e] > 0]
    acc = {"gu": [[], []], "y_perm": [[], []]}
    hs = int(f.h_tensor_scale.item())
    for e in sorted({max(nonempty, key=lambda e: lay.sizes[e]), min(nonempty, key=lambda e: lay.sizes[e])}):
        r = lay.rows(e)
        rows = np.array(sorted({r.start, r.stop - 1} | set(int(v) for v in rng.integers(r.start, r.stop, 4))))
        sel = torch.as_tensor(rows, device=dev, dtype=torch.long)
        xd = mx.dequantize_rows(_npy(g.x_perm.index_select(0, sel)), _npy(g.x_perm_scale.index_select(0, sel)))
        GU = xd @ mx.dequantize_rows(_npy(st.wq[0][e]), _npy(st.wq[1][e])).T
        acc["gu"][0].append(_vals(f.gu.index_select(0, sel)))
        acc["gu"][1].append(GU)
        hb = _vals(f.h_bf16.index_select(0, sel))
        codes = mx.e4m3_encode(hb * 2.0 ** -(hs - 127))
        np.testing.assert_array_equal(_npy(f.h.index_select(0, sel)), codes)
        Y = mx.dequantize_tensor(codes, np.uint8(hs)) @ mx.dequantize_rows(_npy(st.dq[0][e]), _npy(st.dq[1][e])).T
        acc["y_perm"][0].append(_vals(f.y_perm.index_select(0, sel)))
        acc["y_perm"][1].append(Y)
    res = {k: rel_f(np.concatenate(a), np.concatenate(b)) for k, (a, b) in acc.items()}
    say("[gpu] full-size fp8 per-tensor", {k: f"{v:.2e}" for k, v in res.items()})
    for key, v in res.items():
        assert v <= 2e-3, (key, v)


def test_tensor_scale_strided_batch_through_the_abi():
    """batch_stride > n: each tensor is the first n elements of its stride (the rest, which
    holds the largest values here, must not count)."""
    import ctypes as C

    import moe_grouped_expert_amd._binding as B

    rng = np.random.default_rng(91)
    batch, stride, n = 3, 100, 60
    v = rng.standard_normal((batch, stride)) * np.array([1e-3, 1.0, 7.0])[:, None]
    v[:, n:] = 1e6
    g = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to("cuda:0")
    out = torch.zeros(batch, dtype=torch.uint8, device="cuda:0")
    ws = torch.empty(max(int(B.lib().mge_tensor_scale_workspace_bytes(batch, n)), 256), dtype=torch.uint8,
                     device="cuda:0")
    a = B.TensorScaleArgs()
    a.struct_size = C.sizeof(B.TensorScaleArgs)
    a.batch, a.n, a.batch_stride = batch, n, stride
    a.in_, a.scale, a.workspace, a.workspace_bytes = g.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel()
    assert B.lib().mge_tensor_scale(C.byref(a), None) == 0
    torch.cuda.synchronize()
    vals = g.float().cpu().numpy().astype(np.float64)
    for b in range(batch):
        assert int(out[b]) == int(mx.quantize_tensor(vals[b, :n])[1])


def test_quantize_segments_of_an_empty_tensor():
    """R = 0 with segments: every output row is padding (codes and scales 0)."""
    import moe_grouped_expert_amd as m

    g = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda:0")
    seg = torch.zeros(3, dtype=torch.int32, device="cuda:0")
    rc, rs, cc, cs = m.mxfp8_quantize(g, "both", seg_offsets=seg)
    torch.cuda.synchronize()
    assert rc.shape == (m.perm_rows(0, 1, 2, 32), 64)
    assert not rc.any() and not rs.any() and not cc.any() and not cs.any()


@pytest.mark.parametrize("w,empty", [(synth.custom(1403, T=500, E=4, H=128, F=192, k=2, prec="mxfp8"), ()),
                                     (synth.custom(1404, T=300, E=5, H=96, F=128, k=2, prec="mxfp8"), (0, 3))],
                         ids=["plain", "empty_first_mid"])
def test_fp8_tensor_training_staged(w, empty):
    """The FP8 training step with one scale per tensor (bench.Step's fp8_tensor variant,
    fwd + bwd) stage by stage: every quantized operand's scale and codes bit-exact against
    the oracle's quantize_tensor of the values the GPU quantized (x, dy, the weights in
    both forms; h and [dG dU] from the GPU's own bf16 values, both forms); every product
    within rel_F 2e-3 of the oracle fed the GPU's codes ([G U], y_perm, [dG dU] from the
    GPU's dY codes and saved G, U, d_prob, dW_down, dX, dW_gate_up); empty experts get
    zero weight gradients."""
    import bench
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import Inputs, layout_from_gpu, say

    logits = synth.logits(w)
    for e in empty:
        logits[:, e] = np.float32(-1e30)
    inp = Inputs(w, logits)
    st = bench.Step(m, w, dict(logits=inp.g_logits, x=inp.g_x, wgu=inp.g_wgu, wd=inp.g_wd, dy=inp.g_dy), train=True,
                    variant="fp8_tensor")
    st.keep_intermediates = True
    st()
    torch.cuda.synchronize()
    g, f, b = st.g, st.f, st.b
    lay = layout_from_gpu(g, w.E, 32)
    src = _npy(g.perm_src)
    valid = src >= 0
    F, E = w.F, w.E
    lst = lambda t: [_npy(u) for u in t]   # noqa: E731
    # x: one scale, row and column forms
    qx, sx = mx.quantize_tensor(inp.x.astype(np.float64))
    np.testing.assert_array_equal(_npy(g.x_perm)[valid], qx[src[valid]])
    np.testing.assert_array_equal(_npy(g.x_col)[:, valid], qx[src[valid]].T)
    assert not _npy(g.x_col)[:, ~valid].any() and np.all(_npy(g.x_col_scale) == sx)
    # weights: one scale per matrix, both forms
    for e in range(E):
        for wt, qt in ((inp.wgu, st.wq), (inp.wd, st.dq)):
            q, s = mx.quantize_tensor(wt[e].astype(np.float64))
            np.testing.assert_array_equal(_npy(qt[0][e]), q)
            np.testing.assert_array_equal(_npy(qt[2][e])[:, :q.shape[0]], q.T)
            assert np.all(_npy(qt[1][e]) == s) and np.all(_npy(qt[3][e]) == s)
    errs = {}
    # forward: [G U] (the saved G, U), h in bf16, h's one scale in both forms, y_perm, y
    GU = mlp.mx_grouped_nt(_npy(g.x_perm), _npy(g.x_perm_scale), lst(st.wq[0]), lst(st.wq[1]), lay)
    gu = _vals(f.saved_gu)
    assert f.gu is f.saved_gu
    errs["gu"] = rel_f(gu[valid], GU[valid])
    hb = _vals(f.h_bf16)
    errs["h_bf16"] = rel_f(hb[valid], (lay.prob_perm[:, None] * mlp.silu(gu[:, :F]) * gu[:, F:])[valid])
    assert not hb[~valid].any()
    qh, sh = mx.quantize_tensor(hb)
    assert int(f.h_tensor_scale.item()) == int(sh)
    np.testing.assert_array_equal(_npy(f.h), qh)
    np.testing.assert_array_equal(_npy(f.h_col), qh.T)
    assert np.all(_npy(f.h_scale) == sh) and np.all(_npy(f.h_col_scale) == sh)
    Y = mlp.mx_grouped_nt(qh, _npy(f.h_scale), lst(st.dq[0]), lst(st.dq[1]), lay)
    errs["y_perm"] = rel_f(_vals(f.y_perm)[valid], Y[valid])
    errs["y"] = rel_f(_vals(st.y), lay.combine(np.where(valid[:, None], _vals(f.y_perm), 0.0)))
    # backward: dy's one scale (row and column forms of the permuted dY)
    qd, sd = mx.quantize_tensor(inp.dy.astype(np.float64))
    assert int(b.dy_tensor_scale.item()) == int(sd)
    np.testing.assert_array_equal(_npy(b.dy_row)[valid], qd[src[valid]])
    assert not _npy(b.dy_row)[~valid].any() and np.all(_npy(b.dy_row_scale) == sd)
    np.testing.assert_array_equal(_npy(b.dy_col)[:, valid], qd[src[valid]].T)
    assert np.all(_npy(b.dy_col_scale) == sd)
    # the SwiGLU backward in bf16 from the GPU's dY codes, W_down column codes and saved G, U
    dG, dU, dp_row = mlp.mx_dh_stage(_npy(b.dy_row), _npy(b.dy_row_scale), lst(st.dq[2]), lst(st.dq[3]),
                                     gu[:, :F], gu[:, F:], lay)
    dgb = _vals(b.dgu_bf16)
    errs["dgu_bf16"] = rel_f(dgb[valid], np.concatenate([dG, dU], axis=1)[valid])
    assert not dgb[~valid].any()
    errs["d_prob"] = rel_f(_vals(b.d_prob), lay.to_slots(dp_row))
    # [dG dU]'s one scale from the GPU's bf16 values, both forms
    qg, sg = mx.quantize_tensor(dgb)
    assert int(b.dgu_tensor_scale.item()) == int(sg)
    np.testing.assert_array_equal(_npy(b.dgu_row), qg)
    np.testing.assert_array_equal(_npy(b.dgu_col), qg.T)
    assert np.all(_npy(b.dgu_row_scale) == sg) and np.all(_npy(b.dgu_col_scale) == sg)
    # the GEMMs on the GPU's codes
    dWd = mlp.mx_dw_stage(_npy(b.dy_col), _npy(b.dy_col_scale), _npy(f.h_col), _npy(f.h_col_scale), lay)
    errs["dw_down"] = rel_f(np.stack([_vals(t) for t in b.dw_down]), dWd)
    dX = mlp.mx_dx_stage(_npy(b.dgu_row), _npy(b.dgu_row_scale), lst(st.wq[2]), lst(st.wq[3]), lay)
    errs["dx_perm"] = rel_f(_vals(b.dx_perm)[valid], dX[valid])
    dWgu = mlp.mx_dw_stage(_npy(b.dgu_col), _npy(b.dgu_col_scale), _npy(g.x_col), _npy(g.x_col_scale), lay)
    errs["dw_gate_up"] = rel_f(np.stack([_vals(t) for t in b.dw_gate_up]), dWgu)
    errs["dx"] = rel_f(_vals(st.dx), lay.combine(np.where(valid[:, None], _vals(b.dx_perm), 0.0)))
    for e in empty:
        assert not torch.any(b.dw_gate_up[e]) and not torch.any(b.dw_down[e])
    say("[gpu] fp8 per-tensor training", w.name, {k: f"{v:.2e}" for k, v in errs.items()},
        "scales x/h/dy/dgu", int(sx), int(sh), int(sd), int(sg))
    for key, v in errs.items():
        assert v <= 2e-3, (key, v)


def test_mixtral_fp8_tensor_training_sampled():
    """The Mixtral-shaped training step (8192 tokens) with one scale per tensor, as bench.py
    times its fp8_tensor variant: every scale against the oracle's rule on the tensor the
    GPU quantized (x, dy and the weights from the inputs; h and [dG dU] from the GPU's bf16
    values), codes bit-exact on sampled rows, and on sampled rows of two experts [G U], h,
    y_perm, [dG dU] (from the GPU's dY codes and saved G, U), d_prob and dX (from the GPU's
    [dG dU] codes) within rel_F 2e-3; dW entries over an expert's token span from the
    GPU's column codes."""
    import bench
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import layout_from_gpu, say

    w = synth.WORKLOADS[4]
    dev = torch.device("cuda:0")
    say("[gpu] full-size fp8 per-tensor training: inputs")
    inp = bench.make_inputs(w, dev)
    st = bench.Step(m, w, inp, train=True, variant="fp8_tensor")
    st.keep_intermediates = True
    st()
    torch.cuda.synchronize()
    g, f, b = st.g, st.f, st.b
    lay = layout_from_gpu(g, w.E, 32)
    F, H, E = w.F, w.H, w.E
    F2 = 2 * F
    sc = lambda t: int(mx.block_scale_exponent(float(t.abs().max())) + 127)   # noqa: E731
    assert int(st.ts["x"].scale.item()) == sc(inp["x"])
    assert int(b.dy_tensor_scale.item()) == sc(inp["dy"])
    for e in range(E):
        assert int(st.ts["wgu"].scale[e]) == sc(inp["wgu"][e]) and int(st.ts["wd"].scale[e]) == sc(inp["wd"][e])
    hs, ds = int(f.h_tensor_scale.item()), int(b.dgu_tensor_scale.item())
    assert hs == sc(f.h_bf16) and ds == sc(b.dgu_bf16)
    src = _npy(g.perm_src)
    prob = _npy(g.prob_perm).astype(np.float64)
    pp_all = _npy(g.perm_pos)
    slot = {int(pp_all[t, i]): (t, i) for t in range(w.T) for i in range(w.k)}
    dpg = _npy(b.d_prob)
    rng = np.random.default_rng(7272)
    acc = {key: [[], []] for key in ("gu", "h", "y_perm", "dgu", "d_prob", "dx_perm", "dw_down", "dw_gate_up")}

    def add(key, got, ref):
        acc[key][0].append(np.asarray(got, np.float64).ravel())
        acc[key][1].append(np.asarray(ref, np.float64).ravel())

    def take(t, idx, dim=0):
        return t.index_select(dim, torch.as_tensor(idx, device=dev, dtype=torch.long))

    sx, sdy = int(st.ts["x"].scale.item()), int(b.dy_tensor_scale.item())
    for e in (0, E - 1):
        r = lay.rows(e)
        rows = np.array(sorted({r.start, r.stop - 1} | set(int(v) for v in rng.integers(r.start, r.stop, 4))))
        toks = src[rows]
        # codes of x, dy and h, dGU on the sampled rows: the tensor's one scale
        np.testing.assert_array_equal(_npy(take(g.x_perm, rows)), mx.e4m3_encode(_vals(take(inp["x"], toks)) * 2.0 ** -(sx - 127)))
        np.testing.assert_array_equal(_npy(take(b.dy_row, rows)), mx.e4m3_encode(_vals(take(inp["dy"], toks)) * 2.0 ** -(sdy - 127)))
        hb = _vals(take(f.h_bf16, rows))
        np.testing.assert_array_equal(_npy(take(f.h, rows)), mx.e4m3_encode(hb * 2.0 ** -(hs - 127)))
        gb = _vals(take(b.dgu_bf16, rows))
        np.testing.assert_array_equal(_npy(take(b.dgu_row, rows)), mx.e4m3_encode(gb * 2.0 ** -(ds - 127)))
        # forward products on the GPU's codes
        xd = mx.dequantize_rows(_npy(take(g.x_perm, rows)), _npy(take(g.x_perm_scale, rows)))
        GU = xd @ mx.dequantize_rows(_npy(st.wq[0][e]), _npy(st.wq[1][e])).T
        gu = _vals(take(f.saved_gu, rows))
        add("gu", gu, GU)
        add("h", hb, prob[rows][:, None] * mlp.silu(gu[:, :F]) * gu[:, F:])
        Y = mx.dequantize_tensor(_npy(take(f.h, rows)), np.uint8(hs)) @ mx.dequantize_rows(_npy(st.dq[0][e]), _npy(st.dq[1][e])).T
        add("y_perm", _vals(take(f.y_perm, rows)), Y)
        # backward: dh from the GPU's dY codes and W_down column codes, SwiGLU backward on the saved G, U
        dh = mx.dequantize_tensor(_npy(take(b.dy_row, rows)), np.uint8(sdy)) @ mx.dequantize_rows(_npy(st.dq[2][e]), _npy(st.dq[3][e])).T
        p = prob[rows][:, None]
        G, U = gu[:, :F], gu[:, F:]
        add("dgu", gb, np.concatenate([dh * p * U * mlp.dsilu(G), dh * p * mlp.silu(G)], axis=1))
        add("d_prob", [float(dpg[slot[int(rr)]]) for rr in rows], np.sum(dh * mlp.silu(G) * U, axis=1))
        hc = np.unique(np.concatenate([[0, H - 1], rng.integers(0, H, 30)]))
        wgc = mx.dequantize_rows(_npy(take(st.wq[2][e], hc)), _npy(take(st.wq[3][e], hc)))
        add("dx_perm", _vals(take(take(b.dx_perm, rows), hc, 1)),
            mx.dequantize_tensor(_npy(take(b.dgu_row, rows)), np.uint8(ds)) @ wgc.T)
        # weight gradients over the expert's token span from the GPU's column codes
        span = lay.kspan(e)
        sb = slice(span.start // 32, span.stop // 32)
        hh = np.unique(rng.integers(0, H, 8))
        ff = np.unique(rng.integers(0, F, 8))
        dyc = mx.dequantize_rows(_npy(take(b.dy_col, hh)[:, span]), _npy(take(b.dy_col_scale, hh)[:, sb]))
        hcd = mx.dequantize_rows(_npy(take(f.h_col, ff)[:, span]), _npy(take(f.h_col_scale, ff)[:, sb]))
        add("dw_down", _npy(take(take(b.dw_down[e], hh), ff, 1)), dyc @ hcd.T)
        jj = np.unique(np.concatenate([rng.integers(0, F, 4), F + rng.integers(0, F, 4)]))
        gcd = mx.dequantize_rows(_npy(take(b.dgu_col, jj)[:, span]), _npy(take(b.dgu_col_scale, jj)[:, sb]))
        xcd = mx.dequantize_rows(_npy(take(g.x_col, hh)[:, span]), _npy(take(g.x_col_scale, hh)[:, sb]))
        add("dw_gate_up", _npy(take(take(b.dw_gate_up[e], jj), hh, 1)), gcd @ xcd.T)
    res = {k: rel_f(np.concatenate(a), np.concatenate(r_)) for k, (a, r_) in acc.items()}
    say("[gpu] full-size fp8 per-tensor training", {k: f"{v:.2e}" for k, v in res.items()},
        "scales x/h/dy/dgu", sx, hs, sdy, ds)
    for key, v in res.items():
        assert v <= 2e-3, (key, v)
