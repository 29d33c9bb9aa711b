"""Pins of the MXFP8 oracle (oracle/mx.py) against the format definition.

* hand-derived E4M3 code points and worked blocks (tests/golden, OCP MX v1.0);
* exhaustive brute force: every finite bfloat16 pattern, placed in blocks whose
  amax sweeps the whole scale range, checked against a nearest-of-grid search
  (np.searchsorted over the 127 non-negative finite E4M3 values) with the
  even-code tie-break;
* invariants: scales are powers of two, amax/2^e in [256, 512) when the scale
  is not clamped, exact values round-trip, quantization is idempotent;
* the block-scaled product reduces to np.matmul when all scales are 1 and is
  linear in each block's scale.
"""
import os

import numpy as np
import pytest

from oracle import mx

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _grid():
    codes = np.arange(0x7F, dtype=np.uint8)          # 0x00..0x7E, non-negative finite
    vals = mx.e4m3_decode(codes)
    assert np.all(np.diff(vals) > 0)
    return codes, vals


def nearest_code(w):
    """Independent brute force: nearest E4M3 value, ties to the even code, saturating."""
    codes, vals = _grid()
    w = np.asarray(w, dtype=np.float64)
    a = np.abs(w)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    dlo = np.abs(a - vals[lo])
    dhi = np.abs(vals[hi] - a)
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(codes[lo] % 2 == 0, lo, hi)))
    pick = np.where(a >= vals[-1], len(vals) - 1, pick)
    c = codes[pick].astype(np.int64)
    return (c | np.where(np.signbit(w), 0x80, 0)).astype(np.uint8)


def all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)].astype(np.float64)


def test_golden_code_points():
    for line in open(os.path.join(GOLD, "e4m3_points.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        c, v = line.split()
        c = int(c, 16)
        got = mx.e4m3_decode(np.array([c], np.uint8))[0]
        assert got == float(v) and np.signbit(got) == np.signbit(float(v)), (hex(c), got, v)
        assert mx.e4m3_encode(np.array([float(v)]))[0] == c, hex(c)


def _runs(tokens, conv):
    out = []
    for tok in tokens:
        v, n = tok.split("*")
        out += [conv(v)] * int(n)
    return out


def test_golden_blocks():
    n = 0
    for line in open(os.path.join(GOLD, "mx_blocks.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        blk, sc, cd = [s.strip() for s in line.split(";")]
        vals = np.array(_runs(blk.split()[1:], float))
        scale = int(sc.split()[1])
        codes = np.array(_runs(cd.split()[1:], lambda s: int(s, 16)), np.uint8)
        assert vals.shape == (32,) and codes.shape == (32,)
        q, s = mx.quantize_rows(vals[None, :])
        assert int(s[0, 0]) == scale, line
        np.testing.assert_array_equal(q[0], codes, err_msg=line)
        n += 1
    assert n >= 7


def test_encode_exhaustive_bf16_vs_nearest_grid():
    v = all_finite_bf16()
    np.testing.assert_array_equal(mx.e4m3_encode(v), nearest_code(v))


def test_encode_midpoints_and_neighbours():
    _, vals = _grid()
    mids = (vals[:-1] + vals[1:]) / 2
    eps = np.spacing(mids)
    w = np.concatenate([mids, mids + eps, mids - eps, -mids, vals, -vals, [448.0, 449.0, 464.0, 1e6, 2.0 ** -11]])
    np.testing.assert_array_equal(mx.e4m3_encode(w), nearest_code(w))


def test_block_sweep_all_scales_exhaustive():
    """Blocks whose amax fixes e over [-127, 127]; the other values sweep all bf16 <= amax."""
    allv = all_finite_bf16()
    allv = allv[allv != 0]
    mags = np.unique(np.abs(allv))
    # amax = 1.5 * 2^(t + 8) gives floor(log2 amax) - 8 = t; the extra entries sit in
    # the clamped range (bf16 normals below 2^-119 and bf16 subnormals)
    amaxes = [1.5 * 2.0 ** (t + 8) for t in range(-127, 120)] + [2.0 ** -120, 2.0 ** -126, 2.0 ** -130, 2.0 ** -133]
    for amax in amaxes:
        target_e = amax
        others = mags[mags <= amax]
        if others.size == 0:
            continue
        sign = np.where(np.arange(others.size) % 2 == 0, 1.0, -1.0)
        others = others * sign
        nb = (others.size + 30) // 31
        pad = np.zeros(nb * 31)
        pad[: others.size] = others
        blocks = np.concatenate([np.full((nb, 1), amax), pad.reshape(nb, 31)], axis=1)
        q, s = mx.quantize_rows(blocks)
        e = s.astype(np.int64) - 127
        exp_e = max(int(np.floor(np.log2(amax))) - 8, -127)
        assert np.all(e == exp_e), target_e
        w = blocks * 2.0 ** (-exp_e)
        np.testing.assert_array_equal(q, nearest_code(w))
        if exp_e > -127:
            r = amax / 2.0 ** exp_e
            assert 256 <= r < 512


def test_scale_is_power_of_two_and_clamped():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-140, 120, size=(64, 1)))
    q, s = mx.quantize_rows(v)
    sc = mx.e8m0_decode(s)
    m, ex = np.frexp(sc)
    assert np.all(m == 0.5)
    assert s.min() >= 0 and s.max() <= 254


def test_exact_values_roundtrip():
    rng = np.random.default_rng(7)
    _, vals = _grid()
    for e in (-127, -20, -8, 0, 5, 100):
        codes = rng.integers(0, 0x7F, size=(16, 32))
        codes[:, 0] = rng.integers(0x78, 0x7F, size=16)   # block amax/2^e in [256, 448]
        signs = np.where(rng.random((16, 32)) < 0.5, -1.0, 1.0)
        v = signs * vals[codes] * 2.0 ** e
        q, s = mx.quantize_rows(v)
        assert np.all(s.astype(int) - 127 == e)
        np.testing.assert_array_equal(mx.dequantize_rows(q, s), v)


def test_idempotent():
    rng = np.random.default_rng(11)
    v = rng.standard_normal((32, 128)) * 3.7
    q, s = mx.quantize_rows(v)
    q2, s2 = mx.quantize_rows(mx.dequantize_rows(q, s))
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(s, s2)


def test_partial_block_padding_and_cols():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((40, 70))
    q, s = mx.quantize_rows(v)
    assert q.shape == (40, 96) and s.shape == (40, 3)
    assert np.all(q[:, 70:] == 0)
    qc, sc = mx.quantize_cols(v)
    assert qc.shape == (70, 64) and sc.shape == (70, 2)
    qt, st = mx.quantize_rows(v.T)
    np.testing.assert_array_equal(qc, qt)
    # a column block holds 32 consecutive rows of one column
    blk = v[0:32, 5]
    qb, sb = mx.quantize_rows(blk[None, :])
    np.testing.assert_array_equal(qc[5, :32], qb[0])
    assert sc[5, 0] == sb[0, 0]


def test_mx_matmul_unit_scales_is_matmul():
    rng = np.random.default_rng(13)
    qa = rng.integers(0, 256, size=(8, 64)).astype(np.uint8)
    qb = rng.integers(0, 256, size=(5, 64)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0
    qb[(qb & 0x7F) == 0x7F] = 0
    sa = np.full((8, 2), 127, np.uint8)
    sb = np.full((5, 2), 127, np.uint8)
    ref = np.matmul(mx.e4m3_decode(qa), mx.e4m3_decode(qb).T)
    np.testing.assert_allclose(mx.mx_matmul_nt(qa, sa, qb, sb), ref, rtol=1e-14, atol=1e-300)
    # doubling one block's scale doubles exactly that block's contribution
    sa2 = sa.copy()
    sa2[3, 1] = 128
    part = np.matmul(mx.e4m3_decode(qa[3, 32:]), mx.e4m3_decode(qb[:, 32:]).T)
    got = mx.mx_matmul_nt(qa, sa2, qb, sb)
    np.testing.assert_allclose(got[3], ref[3] + part, rtol=1e-14)
    np.testing.assert_allclose(np.delete(got, 3, 0), np.delete(ref, 3, 0), rtol=1e-14)


# ------------------------------------------------------------------------------ FP8, one scale per tensor

def test_tensor_quantize_equals_block_quantize_when_blocks_share_the_amax():
    """Special case that reduces to the pinned block quantizer: every 32-block holds the
    tensor's amax, so each block's scale is the tensor's and the codes coincide."""
    rng = np.random.default_rng(31)
    for amax in (448.0, 3.0, 2.0 ** -20, 1e30):
        v = rng.uniform(-amax, amax, size=(12, 96))
        v[:, ::32] = amax * np.where(rng.random((12, 3)) < 0.5, -1.0, 1.0)
        q, s = mx.quantize_tensor(v)
        qb, sb = mx.quantize_rows(v)
        assert np.all(sb == s)
        np.testing.assert_array_equal(q, qb)


def test_tensor_quantize_brute_force_and_underflow():
    """Every code is the nearest E4M3 value of v / 2^e (ties to even, saturating), with e
    fixed by the tensor amax; values far below the amax go subnormal or to zero, which a
    block scale would have rescued."""
    rng = np.random.default_rng(32)
    mag = np.exp2(rng.uniform(-40, 8, size=4000))
    v = mag * np.where(rng.random(4000) < 0.5, -1.0, 1.0)
    q, s = mx.quantize_tensor(v)
    e = int(s) - 127
    amax = np.max(np.abs(v))
    assert 256.0 <= amax * 2.0 ** -e < 512.0
    np.testing.assert_array_equal(q, nearest_code(v * 2.0 ** -e))
    small = np.abs(v) < 2.0 ** (e - 10)        # below half the smallest subnormal
    assert small.any() and np.all((q[small] & 0x7F) == 0)


def test_tensor_quantize_zero_exact_and_idempotent():
    q, s = mx.quantize_tensor(np.zeros((4, 64)))
    assert s == 0 and not q.any()
    # exactly representable values (E4M3 x 2^e with the tensor's amax in [256, 448] x 2^e) round-trip
    rng = np.random.default_rng(33)
    codes = rng.integers(0, 0x7F, size=(8, 64)).astype(np.uint8) | np.where(rng.random((8, 64)) < 0.5, 0x80, 0).astype(np.uint8)
    codes[0, 0] = 0x7E                          # 448: the amax, scale 2^-3 below
    v = mx.e4m3_decode(codes) * 2.0 ** -3
    q, s = mx.quantize_tensor(v)
    assert s == 127 - 3
    np.testing.assert_array_equal(mx.dequantize_tensor(q, s), v)
    q2, s2 = mx.quantize_tensor(mx.dequantize_tensor(q, s))
    np.testing.assert_array_equal(q2, q)
    assert s2 == s


# ------------------------------------------------------------------------------ segmented column form

def test_segmented_cols_blocks_restart_at_segments():
    rng = np.random.default_rng(41)
    v = rng.standard_normal((100, 64)) * np.exp2(rng.integers(-8, 8, size=(100, 1)))
    off = [0, 7, 7, 40, 72, 100]                 # an empty segment, lengths 7, 33, 32, 28
    q, s = mx.quantize_cols_segmented(v, off)
    lens = np.diff(off)
    padded = (lens + 31) // 32 * 32
    assert q.shape == (64, padded.sum()) and s.shape == (64, padded.sum() // 32)
    start = np.concatenate([[0], np.cumsum(padded)])
    for k in range(len(lens)):
        if lens[k] == 0:
            continue
        # each segment alone, zero-padded to 32 rows: the same codes and scales
        qk, sk = mx.quantize_cols(v[off[k]:off[k + 1]])
        np.testing.assert_array_equal(q[:, start[k]:start[k] + qk.shape[1]], qk)
        np.testing.assert_array_equal(s[:, start[k] // 32:start[k] // 32 + sk.shape[1]], sk)


def test_segmented_cols_aligned_segments_equal_plain_cols():
    rng = np.random.default_rng(42)
    v = rng.standard_normal((96, 32))
    q, s = mx.quantize_cols_segmented(v, [0, 32, 96])
    qp, sp = mx.quantize_cols(v)
    np.testing.assert_array_equal(q, qp)
    np.testing.assert_array_equal(s, sp)
