"""Bit-exact pins of the quantizers inside the fused GEMM epilogues (MXFP8; BF16 roundings too).

The SwiGLU x prob epilogue of the gate-up GEMM quantizes h = p * silu(G) * U from fp32
registers, and the SwiGLU-backward epilogue of the dh GEMM quantizes dG, dU the same way;
in general their fp32 values differ from the oracle's fp64 ones by rounding, so the usual
tests compare those codes after dequantization.  Here the inputs make every one of those
values exact in fp32, so the oracle's quantization must give the same codes and scales
bit for bit, in both forms:
  * one expert, top-1: p = 1 exactly (softmax over one logit);
  * x and W_gate positive integers 1..4 (exact in E4M3 under any block scale the
    quantizer picks for them), W_up, W_down, dy integers in -4..4: every GEMM sum is an
    integer below 2^24, exact in fp32;
  * G >= H = 64, so 1 + e^-G rounds to 1 in fp32: silu(G) = G and silu'(G) = 1 exactly,
    h = G * U, dG = dh * U, dU = dh * G, all integers below 2^24.
A mistake in a lane exchange, an amax reduction, a scale or a byte transpose of either
epilogue changes codes here.  d_prob sums 64 products beyond 2^24 and is compared to
rel_F 1e-6.
"""
import numpy as np
import pytest
import torch

from oracle import mlp, mx
from oracle.metrics import rel_f

pytestmark = pytest.mark.gpu


def _int_bf16(rng, shape, lo, hi):
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return v, torch.from_numpy(v).to(torch.bfloat16).to("cuda:0")


@pytest.mark.parametrize("T,H,F", [(96, 64, 96), (300, 64, 64)])
def test_fused_epilogue_quantizers_bit_exact(T, H, F):
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import layout_from_gpu, npy, say

    rng = np.random.default_rng(T + F)
    say("[gpu] exact epilogue codes", T, H, F)
    x, gx = _int_bf16(rng, (T, H), 1, 4)
    wg, _ = _int_bf16(rng, (1, F, H), 1, 4)
    wu, _ = _int_bf16(rng, (1, F, H), -4, 4)
    wgu = np.concatenate([wg, wu], axis=1)
    gwgu = torch.from_numpy(wgu).to(torch.bfloat16).to("cuda:0")
    wd, gwd = _int_bf16(rng, (1, H, F), -4, 4)
    dy, gdy = _int_bf16(rng, (T, H), -4, 4)
    logits = torch.zeros((T, 1), dtype=torch.float32, device="cuda:0")
    g = m.moe_route_permute(logits, gx, 1, align=32, prec="mxfp8", want_col=True)
    wq = m.mxfp8_quantize(gwgu, "both")
    dq = m.mxfp8_quantize(gwd, "both")
    f = m.grouped_mlp_fwd(g, wq[0], dq[0], wq[1], dq[1], train=True)
    b = m.grouped_mlp_bwd(gdy, g, f, wq[2], dq[2], wq[3], dq[3], keep_intermediates=True)
    torch.cuda.synchronize()
    assert torch.all(g.topk_prob == 1.0)
    lay = layout_from_gpu(g, 1, 32)
    valid = npy(g.perm_src) >= 0
    nrow = int(npy(g.group_offsets)[-1])
    # the operands are exact: codes times power-of-two scales reproduce the integers
    xq, xs = npy(g.x_perm), npy(g.x_perm_scale)
    np.testing.assert_array_equal(mx.dequantize_rows(xq, xs)[valid], x[npy(g.perm_src)[valid]])
    np.testing.assert_array_equal(mx.dequantize_rows(npy(wq[0][0]), npy(wq[1][0])), wgu[0])
    # forward epilogue: G, U (bf16), h codes in both forms
    G, U, h = mlp.mx_gateup_stage(xq, xs, [npy(wq[0][0])], [npy(wq[1][0])], lay)
    assert G[valid].min() >= H and np.abs(h).max() < 2 ** 24
    np.testing.assert_array_equal(G, np.rint(G))
    gu = f.saved_gu.float().cpu().numpy().astype(np.float64)
    ref_g = torch.from_numpy(G[valid]).to(torch.bfloat16).double().numpy()
    ref_u = torch.from_numpy(U[valid]).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(gu[valid, :F], ref_g)
    np.testing.assert_array_equal(gu[valid, F:], ref_u)
    q, s = mx.quantize_rows(h)
    np.testing.assert_array_equal(npy(f.h)[valid], q[valid])
    np.testing.assert_array_equal(npy(f.h_scale)[valid], s[valid])
    qc, sc = mx.quantize_cols(h)
    np.testing.assert_array_equal(npy(f.h_col)[:, :nrow], qc[:, :nrow])
    np.testing.assert_array_equal(npy(f.h_col_scale)[:, :nrow // 32], sc[:, :nrow // 32])
    # backward epilogue: dG, dU codes in both forms, from the GPU's exact G, U
    dG, dU, dp_row = mlp.mx_dh_stage(npy(b.dy_row), npy(b.dy_row_scale), [npy(dq[2][0])], [npy(dq[3][0])],
                                     gu[:, :F], gu[:, F:], lay)
    dGU = np.where(valid[:, None], np.concatenate([dG, dU], axis=1), 0.0)
    assert np.abs(dGU).max() < 2 ** 24
    np.testing.assert_array_equal(dGU, np.rint(dGU))
    q, s = mx.quantize_rows(dGU)
    np.testing.assert_array_equal(npy(b.dgu_row)[valid], q[valid])
    np.testing.assert_array_equal(npy(b.dgu_row_scale)[valid], s[valid])
    qc, sc = mx.quantize_cols(dGU)
    np.testing.assert_array_equal(npy(b.dgu_col)[:, :nrow], qc[:, :nrow])
    np.testing.assert_array_equal(npy(b.dgu_col_scale)[:, :nrow // 32], sc[:, :nrow // 32])
    err = rel_f(b.d_prob.double().cpu().numpy(), lay.to_slots(dp_row))
    say("[gpu] exact epilogue codes: all bit-exact; d_prob rel_F", f"{err:.1e}")
    assert err <= 1e-6


def test_fused_epilogues_bf16_bit_exact():
    """The BF16 path on the same exact-valued inputs: h, its transpose, G, U, dG and dU
    leave as bf16 roundings (RNE) of exact values, so they equal the oracle's bit for bit."""
    import moe_grouped_expert_amd as m
    from tests.gpu_helpers import layout_from_gpu, npy, say

    T, H, F = 200, 64, 96
    rng = np.random.default_rng(77)
    say("[gpu] exact epilogue bf16", T, H, F)
    x, gx = _int_bf16(rng, (T, H), 1, 4)
    wg, _ = _int_bf16(rng, (1, F, H), 1, 4)
    wu, _ = _int_bf16(rng, (1, F, H), -4, 4)
    wgu = np.concatenate([wg, wu], axis=1)
    gwgu = torch.from_numpy(wgu).to(torch.bfloat16).to("cuda:0")
    wd, gwd = _int_bf16(rng, (1, H, F), -4, 4)
    dy, gdy = _int_bf16(rng, (T, H), -4, 4)
    logits = torch.zeros((T, 1), dtype=torch.float32, device="cuda:0")
    g = m.moe_route_permute(logits, gx, 1, align=32, prec="bf16", want_col=True)
    f = m.grouped_mlp_fwd(g, gwgu, gwd, train=True)
    b = m.grouped_mlp_bwd(gdy, g, f, gwgu, gwd, keep_intermediates=True)
    torch.cuda.synchronize()
    lay = layout_from_gpu(g, 1, 32)
    valid = npy(g.perm_src) >= 0
    nrow = int(npy(g.group_offsets)[-1])

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).double().numpy()

    def gpu(t):
        return t.double().cpu().numpy()

    _, sv = mlp.fwd_grouped(x, wgu, wd, lay, keep=True)      # the oracle's grouped forward (p = 1)
    G, U, h = sv["G"], sv["U"], sv["h"]
    GU = np.concatenate([G, U], axis=1)
    assert G[valid].min() >= H and np.abs(h).max() < 2 ** 24
    np.testing.assert_array_equal(h, np.where(valid[:, None], G * U, 0.0))   # silu(G) = G exactly
    np.testing.assert_array_equal(gpu(f.saved_gu)[valid], bf(GU)[valid])
    np.testing.assert_array_equal(gpu(f.h)[valid], bf(h)[valid])
    np.testing.assert_array_equal(gpu(f.h_col)[:, :nrow], bf(h.T)[:, :nrow])
    # backward from the GPU's bf16 G, U: dh = dY W_down, dG = dh U, dU = dh G (the backward's
    # definition with p = 1 and silu'(G) = silu(G) / G = 1 on these inputs)
    gsv = gpu(f.saved_gu)
    assert np.all(mlp.dsilu(gsv[valid, :F]) == 1.0) and np.all(mlp.silu(gsv[valid, :F]) == gsv[valid, :F])
    dh = lay.gather(dy) @ wd[0].astype(np.float64)
    dGU = np.where(valid[:, None], np.concatenate([dh * gsv[:, F:], dh * gsv[:, :F]], axis=1), 0.0)
    assert np.abs(dGU).max() < 2 ** 24
    np.testing.assert_array_equal(gpu(b.dgu_row)[valid], bf(dGU)[valid])
    np.testing.assert_array_equal(gpu(b.dgu_col)[:, :nrow], bf(dGU.T)[:, :nrow])
    say("[gpu] exact epilogue bf16: all bit-exact")
