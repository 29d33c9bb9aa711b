"""MXFP8 (E4M3 elements + E8M0 block scales) in fp64 — oracle, test infrastructure only.

What the pages fix: 8-bit elements, with a run of 32 neighbouring elements sharing
one scale ([P1] "Memory and quantization overhead"; [P4] paragraph on FP8/MXFP8).  The element format (E4M3), the scale format (E8M0, a power of two)
and the scale-selection rule come from the OCP MX v1.0 specification [OCP]:

  * E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits.  Normal values
    (1 + m/8) * 2^(E-7) for E in 1..15; subnormals m * 2^-9; E=15,m=7 is NaN,
    so the largest finite magnitude is 448.  There are no infinities.
  * E8M0: an unsigned biased exponent s, value 2^(s-127); 255 is NaN.
  * shared exponent of a block:  e = floor(log2(amax)) - emax_elem, emax_elem = 8
    for E4M3, clamped to the E8M0 range; an all-zero block takes the smallest
    scale.  Elements are v / 2^e converted to E4M3 with round-to-nearest-even,
    saturating magnitudes beyond 448 to 448 (the conversion the spec allows
    when clamping is chosen).

FP8 with one scale per tensor (quantize_tensor) applies the same rule with the
whole tensor as the block.

Readings where the pages are silent (listed in the design notes): floor rule
with saturation (not the ceil/no-clip rule); -0 encodes as 0x80; partial
blocks are zero-padded.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
EMAX_ELEM = 8          # floor(log2(448))
SCALE_BIAS = 127
BLOCK = 32


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 byte codes -> fp64 values (exact).  0x7F/0xFF (NaN) decode to nan."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(E == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(E.astype(np.float64) - 7.0))
    mag = np.where(((c & 0x7F) == 0x7F), np.nan, mag)
    return sign * mag


def e4m3_encode(w) -> np.ndarray:
    """fp64 values -> E4M3 codes, round-to-nearest-even with saturation at 448.

    Written from the format definition: find the binade of |w| (not below the
    subnormal binade 2^-6), the spacing there is 2^(binade-3); round |w| to a
    multiple of that spacing with ties to even; the code is then
    8*(binade+7) + (multiple - 8), which also covers subnormals (binade -6) and
    carries into the next binade when the rounded multiple reaches 16.
    """
    w = np.asarray(w, dtype=np.float64)
    neg = np.signbit(w)
    a = np.abs(w)
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(a)               # a = mant * 2**ex, mant in [0.5, 1)
    binade = np.maximum(ex - 1, -6)       # floor(log2 a), not below the subnormal binade
    q = np.exp2(binade.astype(np.float64) - 3.0)
    r = np.rint(a / q)                    # numpy rint: ties to even
    code = (8 * (binade + 7) + r.astype(np.int64) - 8)
    code = np.where(a == 0.0, 0, code)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = code.astype(np.int64) | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def e8m0_decode(s) -> np.ndarray:
    s = np.asarray(s).astype(np.float64)
    return np.exp2(s - SCALE_BIAS)


def block_scale_exponent(amax) -> np.ndarray:
    """Unbiased shared exponent e of a block with the given amax (floor rule, clamped)."""
    amax = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(amax)
    fl = np.where(amax > 0, ex - 1, -10_000)   # floor(log2 0) := -inf
    return np.clip(fl - EMAX_ELEM, -127, 127).astype(np.int64)


def quantize_rows(v) -> tuple[np.ndarray, np.ndarray]:
    """Quantize along the last axis in blocks of 32 consecutive values.

    v: [..., C] (fp64-representable values). Returns codes uint8 [..., C_pad] and
    scales uint8 [..., C_pad/32] with C_pad = ceil(C/32)*32; a partial last block
    is padded with zeros.
    """
    v = np.asarray(v, dtype=np.float64)
    C = v.shape[-1]
    Cp = (C + BLOCK - 1) // BLOCK * BLOCK
    if Cp != C:
        pad = [(0, 0)] * (v.ndim - 1) + [(0, Cp - C)]
        v = np.pad(v, pad)
    blk = v.reshape(v.shape[:-1] + (Cp // BLOCK, BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    e = block_scale_exponent(amax)
    w = blk * np.exp2(-e.astype(np.float64))[..., None]
    codes = e4m3_encode(w).reshape(v.shape[:-1] + (Cp,))
    scales = (e + SCALE_BIAS).astype(np.uint8)
    return codes, scales


def quantize_cols(v) -> tuple[np.ndarray, np.ndarray]:
    """Column orientation of a [..., R, C] matrix: blocks of 32 consecutive rows.

    Stored transposed (K-contiguous): codes [..., C, R_pad], scales
    [..., C, R_pad/32].  By definition this is quantize_rows of the transpose.
    """
    v = np.asarray(v, dtype=np.float64)
    return quantize_rows(np.swapaxes(v, -1, -2))


def pad_segments(v, seg_offsets) -> np.ndarray:
    """Rows of v [R][C] regrouped so that segment s (rows seg_offsets[s] .. seg_offsets[s+1])
    starts at a multiple of 32: segment s lands at sum_{j<s} ceil(len_j / 32) * 32 and the
    rows up to the next segment are zero.  Returns [sum of padded lengths][C]."""
    v = np.asarray(v, dtype=np.float64)
    off = np.asarray(seg_offsets, dtype=np.int64)
    parts = []
    for s in range(len(off) - 1):
        seg = v[off[s]:off[s + 1]]
        n = len(seg)
        pad = (n + BLOCK - 1) // BLOCK * BLOCK - n
        parts.append(np.concatenate([seg, np.zeros((pad, v.shape[1]))]) if pad else seg)
    return np.concatenate(parts) if parts else np.zeros((0, v.shape[1]))


def quantize_cols_segmented(v, seg_offsets) -> tuple[np.ndarray, np.ndarray]:
    """Column form whose 32-row blocks restart at every segment start (the per-expert token
    blocks of the weight gradients, [P4] paragraph on GroupedLinear: each expert's tokens
    form their own group): quantize_cols of pad_segments(v), so no block mixes two
    segments."""
    return quantize_cols(pad_segments(v, seg_offsets))


def quantize_tensor(v) -> tuple[np.ndarray, np.uint8]:
    """FP8 with one scale for the whole tensor: E4M3 codes (same shape as v) and one
    E8M0 scale byte.

    The pages name FP8 beside MXFP8, both 8-bit, MXFP8 adding a scale per block of 32
    ([P1] "Memory and quantization overhead"; [P4] paragraph on FP8/MXFP8); they do not
    say how the FP8 scale is chosen.  Reading: the MX rule above with the whole tensor as
    the block ("current" scaling from the tensor's own amax, a power-of-two scale):
    e = floor(log2 amax) - 8 clamped to [-127, 127] (all-zero: -127), codes =
    RNE(v / 2^e) onto E4M3 with saturation at 448.
    """
    v = np.asarray(v, dtype=np.float64)
    amax = float(np.max(np.abs(v))) if v.size else 0.0
    e = int(block_scale_exponent(amax))
    codes = e4m3_encode(v * np.exp2(-float(e)))
    return codes, np.uint8(e + SCALE_BIAS)


def dequantize_tensor(codes, scale) -> np.ndarray:
    """Inverse of quantize_tensor's encoding: element value * 2^(scale-127)."""
    return e4m3_decode(codes) * float(e8m0_decode(scale))


def dequantize_rows(codes, scales) -> np.ndarray:
    """Inverse of quantize_rows' encoding: element value * 2^(s-127)."""
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    C = codes.shape[-1]
    vals = e4m3_decode(codes).reshape(codes.shape[:-1] + (C // BLOCK, BLOCK))
    return (vals * e8m0_decode(scales)[..., None]).reshape(codes.shape)


def mx_matmul_nt(qa, sa, qb, sb) -> np.ndarray:
    """C[m,n] = sum_b 2^(ea[m,b]+eb[n,b]) * sum_j dec(qa[m,32b+j]) * dec(qb[n,32b+j]).

    Both operands are K-contiguous (row forms along K).  Decoded values are exact in
    fp64, so this is the block-scaled product up to fp64 summation rounding.
    """
    A = dequantize_rows(qa, sa)
    B = dequantize_rows(qb, sb)
    return A @ B.T
