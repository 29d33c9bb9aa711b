"""The routed SwiGLU expert MLP, forward and backward, in fp64 — oracle, test infrastructure only.

Per token t with selected experts S_t and probabilities p_t ([P1] intro and
"Grouped experts instead of a Python loop"; [P4] paragraph on the Sequential
fusion, which places the probability-scaled SwiGLU between the two grouped linears):

    y_t = sum_i  W_down[e] ( p_ti * silu(W_gate[e] x_t) * (W_up[e] x_t) ),   e = S_t[i]

with silu(z) = z / (1 + exp(-z)) (the SwiGLU of Shazeer, "GLU Variants Improve
Transformer", 2020: silu(gate) times up; the pages do not define it).  W_gate_up[e]
stacks W_gate (rows 0..F-1) over W_up (rows F..2F-1).

Two tiers:
  * ``fwd_per_token`` walks tokens and their experts one by one (the per-expert
    formulation the pages contrast grouped execution with);
  * ``fwd_grouped`` / ``bwd_grouped`` gather each expert's tokens, as the grouped
    call does, and use one fp64 matmul per expert and projection.

The backward is the gradient of L = <dy, y> with respect to x, W_gate_up, W_down and
p (the pages only say that the fused forward comes with a fused backward):
    dY = gather(dy), dh = dY W_down, dp = sum_f dh * silu(G) * U,
    dU = dh * p * silu(G), dG = dh * p * U * sig(G) * (1 + G (1 - sig(G))),
    dW_down = dY^T h, dW_gate_up = [dG dU]^T X, dX = [dG dU] W_gate_up, dx = combine(dX).

MXFP8 stage functions (``mx_*``) evaluate one GEMM stage on given quantized operands
(block-scaled product, exact decode) so that each GPU stage can be compared with an
oracle fed the same quantized inputs.
"""
from __future__ import annotations

import numpy as np

from . import mx
from . import route as rt


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def dsilu(z):
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


# ----------------------------------------------------------------------------- O-slow

def fwd_per_token(x, w_gate_up, w_down, topk_idx, topk_prob):
    """Per-token, per-expert evaluation of y (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    E, F2, _ = w_gate_up.shape
    F = F2 // 2
    y = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        for i in range(topk_idx.shape[1]):
            e = int(topk_idx[t, i])
            wg = np.asarray(w_gate_up[e, :F], dtype=np.float64)
            wu = np.asarray(w_gate_up[e, F:], dtype=np.float64)
            wd = np.asarray(w_down[e], dtype=np.float64)
            h = float(topk_prob[t, i]) * silu(wg @ x[t]) * (wu @ x[t])
            y[t] += wd @ h
    return y


# ----------------------------------------------------------------------------- O-grouped

class Layout:
    """Permuted layout of one routing decision (rows grouped by expert)."""

    def __init__(self, topk_idx, topk_prob, E: int, align: int = 32):
        self.topk_idx = np.asarray(topk_idx)
        self.topk_prob = np.asarray(topk_prob, dtype=np.float64)
        self.T, self.k = self.topk_idx.shape
        self.E = E
        self.align = align
        self.sizes = rt.split_sizes(self.topk_idx, E)
        self.off = rt.group_offsets(self.sizes, align)
        self.perm_src, self.perm_pos = rt.permutation(self.topk_idx, E, align)
        self.R = len(self.perm_src)
        self.prob_perm = rt.prob_permuted(self.topk_prob, self.perm_pos, self.R)

    def rows(self, e: int) -> slice:
        return slice(int(self.off[e]), int(self.off[e]) + int(self.sizes[e]))

    def kspan(self, e: int) -> slice:
        """Rows of group e including its zero padding up to a multiple of 32."""
        m = int(self.sizes[e])
        return slice(int(self.off[e]), int(self.off[e]) + (m + 31) // 32 * 32)

    def gather(self, a):
        """Permuted copy of a [T][C]; padding rows are zero."""
        a = np.asarray(a, dtype=np.float64)
        out = np.zeros((self.R, a.shape[1]), dtype=np.float64)
        v = self.perm_src >= 0
        out[v] = a[self.perm_src[v]]
        return out

    def combine(self, a_perm):
        """out[t] = sum_i a_perm[perm_pos[t, i]] in slot order i = 0..k-1."""
        a_perm = np.asarray(a_perm, dtype=np.float64)
        out = np.zeros((self.T, a_perm.shape[1]), dtype=np.float64)
        for i in range(self.k):
            out += a_perm[self.perm_pos[:, i]]
        return out

    def to_slots(self, per_row):
        """[R] per-row values -> [T][k] per assignment."""
        return np.asarray(per_row)[self.perm_pos]


def fwd_grouped(x, w_gate_up, w_down, lay: Layout, keep=False):
    """Grouped forward: returns y [T][H] (and the intermediates if keep)."""
    E, F2, H = w_gate_up.shape
    F = F2 // 2
    X = lay.gather(x)
    G = np.zeros((lay.R, F))
    U = np.zeros((lay.R, F))
    h = np.zeros((lay.R, F))
    Y = np.zeros((lay.R, H))
    for e in range(E):
        r = lay.rows(e)
        if r.stop == r.start:
            continue
        GU = X[r] @ np.asarray(w_gate_up[e], dtype=np.float64).T
        G[r], U[r] = GU[:, :F], GU[:, F:]
        h[r] = lay.prob_perm[r][:, None] * silu(G[r]) * U[r]
        Y[r] = h[r] @ np.asarray(w_down[e], dtype=np.float64).T
    y = lay.combine(Y)
    if keep:
        return y, dict(X=X, G=G, U=U, h=h, Y=Y)
    return y


def bwd_grouped(dy, w_gate_up, w_down, lay: Layout, saved):
    """Grouped backward of L = <dy, y>. Returns dict dx, dw_gate_up, dw_down, d_prob, dX
    and the permuted intermediates dh ([R][F]) and dGU = [dG dU] ([R][2F])."""
    E, F2, H = w_gate_up.shape
    F = F2 // 2
    X, G, U, h = saved["X"], saved["G"], saved["U"], saved["h"]
    dY = lay.gather(dy)
    dX = np.zeros((lay.R, H))
    dp_row = np.zeros(lay.R)
    dh_all = np.zeros((lay.R, F))
    dGU_all = np.zeros((lay.R, F2))
    dw_gu = np.zeros((E, F2, H))
    dw_d = np.zeros((E, H, F))
    for e in range(E):
        r = lay.rows(e)
        if r.stop == r.start:
            continue
        wd = np.asarray(w_down[e], dtype=np.float64)
        wgu = np.asarray(w_gate_up[e], dtype=np.float64)
        p = lay.prob_perm[r][:, None]
        dh = dY[r] @ wd
        s = silu(G[r])
        dp_row[r] = np.sum(dh * s * U[r], axis=1)
        dU = dh * p * s
        dG = dh * p * U[r] * dsilu(G[r])
        dGU = np.concatenate([dG, dU], axis=1)
        dh_all[r] = dh
        dGU_all[r] = dGU
        dw_d[e] = dY[r].T @ h[r]
        dw_gu[e] = dGU.T @ X[r]
        dX[r] = dGU @ wgu
    return dict(dx=lay.combine(dX), dw_gate_up=dw_gu, dw_down=dw_d, d_prob=lay.to_slots(dp_row), dX=dX,
                dh=dh_all, dGU=dGU_all)


# ----------------------------------------------------------------------------- MXFP8 stages

def mx_grouped_nt(qa, sa, qb_list, sb_list, lay: Layout):
    """Ragged-M block-scaled GEMM: out[rows_e] = dec(A[rows_e]) dec(B_e)^T per expert."""
    N = qb_list[0].shape[0]
    out = np.zeros((lay.R, N))
    for e in range(lay.E):
        r = lay.rows(e)
        if r.stop == r.start:
            continue
        out[r] = mx.mx_matmul_nt(qa[r], sa[r], qb_list[e], sb_list[e])
    return out


def mx_gateup_stage(xq, xs, wgu_q, wgu_s, lay: Layout):
    """a5+a6 on quantized operands: returns G, U and h = p*silu(G)*U (fp64, [R][F])."""
    GU = mx_grouped_nt(xq, xs, wgu_q, wgu_s, lay)
    F = GU.shape[1] // 2
    G, U = GU[:, :F], GU[:, F:]
    h = lay.prob_perm[:, None] * silu(G) * U
    valid = np.zeros(lay.R, bool)
    for e in range(lay.E):
        valid[lay.rows(e)] = True
    h[~valid] = 0.0
    return G, U, h


def mx_down_stage(hq, hs, wd_q, wd_s, lay: Layout):
    """a7 on quantized operands: y_perm = dec(h_q) dec(W_down)^T per expert."""
    return mx_grouped_nt(hq, hs, wd_q, wd_s, lay)


def mx_dh_stage(dyq, dys, wd_colq, wd_cols, G, U, lay: Layout):
    """b2 on quantized operands: dh = dec(dY) dec(W_down col)^T, then SwiGLU backward.

    G and U are the saved values the GPU stored.  Returns dG, dU ([R][F]) and the
    per-row d_prob (before mapping to [T][k]).
    """
    dh = mx_grouped_nt(dyq, dys, wd_colq, wd_cols, lay)
    G = np.asarray(G, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    p = lay.prob_perm[:, None]
    s = silu(G)
    dp_row = np.sum(dh * s * U, axis=1)
    dU = dh * p * s
    dG = dh * p * U * dsilu(G)
    return dG, dU, dp_row


def mx_dw_stage(a_colq, a_cols, b_colq, b_cols, lay: Layout):
    """b4 / b6 on quantized column forms: dW[e] = dec(A col)[:, span_e] dec(B col)[:, span_e]^T.

    Column forms are [N][R] K-contiguous along tokens with blocks of 32 rows that
    start at each group's first row; the span of group e includes its zero padding.
    """
    NA = a_colq.shape[0]
    NB = b_colq.shape[0]
    out = np.zeros((lay.E, NA, NB))
    for e in range(lay.E):
        s = lay.kspan(e)
        if s.stop == s.start:
            continue
        b0, b1 = s.start // 32, s.stop // 32
        out[e] = mx.mx_matmul_nt(a_colq[:, s], a_cols[:, b0:b1], b_colq[:, s], b_cols[:, b0:b1])
    return out


def mx_dx_stage(dguq, dgus, wgu_colq, wgu_cols, lay: Layout):
    """b5 on quantized operands: dX = dec(dGU) dec(W_gate_up col)^T per expert."""
    return mx_grouped_nt(dguq, dgus, wgu_colq, wgu_cols, lay)


def mx_fwd_end_to_end(x, w_gate_up, w_down, lay: Layout):
    """Whole MXFP8 forward in fp64 with the quantization points of the MXFP8 path.

    x rows along H, W_gate_up rows along H, h (after the probability scaling) rows
    along F, W_down rows along F; everything else exact.  Returns y and parts.
    """
    E = w_gate_up.shape[0]
    X = lay.gather(x)
    xq, xs = mx.quantize_rows(X)
    wq = [mx.quantize_rows(w_gate_up[e]) for e in range(E)]
    dq = [mx.quantize_rows(w_down[e]) for e in range(E)]
    G, U, h = mx_gateup_stage(xq, xs, [a for a, _ in wq], [b for _, b in wq], lay)
    hq, hs = mx.quantize_rows(h)
    Y = mx_down_stage(hq, hs, [a for a, _ in dq], [b for _, b in dq], lay)
    return lay.combine(Y), dict(xq=xq, xs=xs, G=G, U=U, h=h, hq=hq, hs=hs, Y=Y)
