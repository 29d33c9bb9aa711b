"""Top-k routing and the token permutation by expert — oracle, test infrastructure only.

Per the pages, each token is sent to a small number of experts ([P1] intro), and the
grouped call collects every expert's tokens and is told how many each expert has
through a separate ``split_sizes`` argument ([P1] "Grouped experts instead of a
Python loop"; [P4] paragraph on GroupedLinear); the SwiGLU output is
scaled by the routing probability ([P4] paragraph on the Sequential fusion).

Readings where the pages are silent:
  * selection: the k largest fp32 logits, ordered by (logit descending, expert
    index ascending) — ties go to the lower index, -0.0 equals +0.0;
  * probabilities: softmax over all E logits renormalised over the k selected,
    which in exact arithmetic is the softmax over the k selected logits alone;
  * permuted layout: experts in index order, each group starting at a multiple of
    ``align`` rows; inside a group the assignments (t, i) keep their
    lexicographic order (a stable counting sort); rows that no assignment fills
    are padding (perm_src = -1);
  * total rows of the permuted buffers: T*k + E*(align-1), rounded up to 32.
"""
from __future__ import annotations

import numpy as np


def perm_rows(T: int, k: int, E: int, align: int) -> int:
    n = T * k + E * (align - 1)
    return (n + 31) // 32 * 32


def route(logits, k: int):
    """Returns topk_idx int32 [T][k] and topk_prob fp64 [T][k]."""
    l = np.asarray(logits, dtype=np.float64)
    T, E = l.shape
    idx = np.zeros((T, k), dtype=np.int32)
    prob = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        # order experts by (logit desc, index asc): sort key pairs explicitly
        order = sorted(range(E), key=lambda e: (-l[t, e], e))
        sel = order[:k]
        idx[t] = sel
        z = l[t, sel]
        m = z.max()
        ez = np.exp(z - m)
        prob[t] = ez / ez.sum()
    return idx, prob


def split_sizes(topk_idx, E: int) -> np.ndarray:
    """split_sizes[e] = number of (token, slot) assignments routed to expert e."""
    s = np.zeros(E, dtype=np.int64)
    for e in np.asarray(topk_idx).ravel():
        s[e] += 1
    return s.astype(np.int32)


def group_offsets(sizes, align: int) -> np.ndarray:
    """Exclusive prefix sum of the sizes rounded up to ``align``: int32 [E+1]."""
    off = [0]
    for m in sizes:
        off.append(off[-1] + (int(m) + align - 1) // align * align)
    return np.array(off, dtype=np.int32)


def permutation(topk_idx, E: int, align: int):
    """Stable counting sort of the assignments by expert.

    Returns perm_src int32 [R] (token of each permuted row, -1 for padding) and
    perm_pos int32 [T][k] (permuted row of assignment (t, i)), with R = perm_rows.
    """
    topk_idx = np.asarray(topk_idx)
    T, k = topk_idx.shape
    sizes = split_sizes(topk_idx, E)
    off = group_offsets(sizes, align)
    R = perm_rows(T, k, E, align)
    perm_src = np.full(R, -1, dtype=np.int32)
    perm_pos = np.zeros((T, k), dtype=np.int32)
    fill = [int(off[e]) for e in range(E)]
    for t in range(T):
        for i in range(k):
            e = int(topk_idx[t, i])
            row = fill[e]
            fill[e] += 1
            perm_src[row] = t
            perm_pos[t, i] = row
    return perm_src, perm_pos


def prob_permuted(topk_prob, perm_pos, R: int) -> np.ndarray:
    """prob_perm[row] = p of the assignment stored in that row (0 on padding)."""
    pp = np.zeros(R, dtype=np.float64)
    T, k = perm_pos.shape
    for t in range(T):
        for i in range(k):
            pp[perm_pos[t, i]] = topk_prob[t, i]
    return pp


def router_bwd(topk_idx, topk_prob, d_prob, E: int) -> np.ndarray:
    """Gradient of the routing probabilities with respect to the router logits.

    The probabilities of a token's k slots are the softmax of the selected logits
    z_i = l[idx_i] (the reading of [P1] intro / [P4] GroupedLinear used by ``route``),
    so the chain rule through that softmax gives, with s = sum_j p_j * d_p_j,
        d_z_i = p_i * (d_p_i - s),
    and each d_z_i is added to the logit it was gathered from: d_l[t][idx_i] += d_z_i.
    Logits that no slot selected get 0: the renormalised probabilities do not depend on
    them.  Indices outside [0, E) contribute nothing.  Returns fp64 [T][E].
    """
    idx = np.asarray(topk_idx)
    p = np.asarray(topk_prob, dtype=np.float64)
    dp = np.asarray(d_prob, dtype=np.float64)
    T, k = idx.shape
    out = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        s = sum(p[t, j] * dp[t, j] for j in range(k))
        for i in range(k):
            e = int(idx[t, i])
            if 0 <= e < E:
                out[t, e] += p[t, i] * (dp[t, i] - s)
    return out
