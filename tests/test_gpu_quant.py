"""GPU parity of mxfp8_quantize (through the C ABI) against the oracle: bit-exact codes
and scales, row and column orientation, exhaustive over every finite bfloat16 pattern
placed in blocks whose amax sweeps the whole scale range, plus ragged shapes."""
import numpy as np
import pytest
import torch

from oracle import mx

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import moe_grouped_expert_amd as mge
    from tests.gpu_helpers import say
    say("[gpu] quantize tests on", torch.cuda.get_device_name(0))
    return mge


def sweep_blocks():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    mags = np.unique(np.abs(f[np.isfinite(f) & (f != 0)])).astype(np.float64)
    rows = []
    amaxes = [1.5 * 2.0 ** (t + 8) for t in range(-127, 120)] + [2.0 ** -120, 2.0 ** -126, 2.0 ** -130, 2.0 ** -133]
    for amax in amaxes:
        others = mags[mags <= amax]
        if others.size == 0:
            continue
        others = others * np.where(np.arange(others.size) % 2 == 0, 1.0, -1.0)
        nb = (others.size + 30) // 31
        pad = np.zeros(nb * 31)
        pad[: others.size] = others
        rows.append(np.concatenate([np.full((nb, 1), amax), pad.reshape(nb, 31)], axis=1))
    blk = np.concatenate(rows)                 # [nblocks][32], each row one block
    nb = blk.shape[0] // 256 * 256           # rows of 8 blocks, a multiple of 32 rows
    return blk[:nb].reshape(nb // 8, 256).astype(np.float32)


def test_quantize_exhaustive_bitexact(m):
    from tests.gpu_helpers import gpu_bf16, npy, say
    v = sweep_blocks()
    say("[gpu] exhaustive quantize, shape", v.shape)
    g = gpu_bf16(v)
    rc, rs, _, _ = m.mxfp8_quantize(g, "row")
    q, s = mx.quantize_rows(v.astype(np.float64))
    np.testing.assert_array_equal(npy(rs), s)
    np.testing.assert_array_equal(npy(rc), q)
    # column orientation of the transpose is the row quantization of the original
    gt = g.t().contiguous()
    _, _, cc, cs = m.mxfp8_quantize(gt, "col")
    np.testing.assert_array_equal(npy(cs), s)
    np.testing.assert_array_equal(npy(cc), q)
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape", [(3, 100, 96), (1, 7, 32), (2, 64, 128), (1, 130, 4160), (4, 33, 288)])
def test_quantize_shapes_row_col(m, shape):
    from tests.gpu_helpers import gpu_bf16, npy, say
    say("[gpu] quantize shape", shape)
    rng = np.random.default_rng(sum(shape))
    v = (rng.standard_normal(shape) * np.exp2(rng.integers(-20, 20, size=shape[:-1] + (1,)))).astype(np.float32)
    g = gpu_bf16(v)
    rc, rs, cc, cs = m.mxfp8_quantize(g, "both")
    vb = g.float().cpu().numpy().astype(np.float64)
    q, s = mx.quantize_rows(vb)
    np.testing.assert_array_equal(npy(rc), q)
    np.testing.assert_array_equal(npy(rs), s)
    qc, sc = mx.quantize_cols(vb)
    np.testing.assert_array_equal(npy(cc), qc)
    np.testing.assert_array_equal(npy(cs), sc)


@pytest.mark.parametrize("offsets", [[0, 7, 7, 40, 72, 100], [0, 100], [0, 0, 32, 64, 100, 100], [0, 1, 2, 3, 100]])
def test_quantize_segments_matches_oracle(offsets):
    """Segments along R placed at 32-row multiples: row and column codes and scales
    bit-exact against the oracle's zero-padded segments (empty segments, lengths below,
    at and above 32, a segment at either end)."""
    import moe_grouped_expert_amd as m

    rng = np.random.default_rng(len(offsets) * 100 + offsets[1])
    R, C, B = 100, 96, 2
    v = rng.standard_normal((B, R, C)) * np.exp2(rng.integers(-6, 6, size=(B, R, 1)))
    g = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to("cuda:0")
    seg = torch.tensor(offsets, dtype=torch.int32, device="cuda:0")
    rc, rs, cc, cs = m.mxfp8_quantize(g, "both", seg_offsets=seg)
    torch.cuda.synchronize()
    Rs = m.perm_rows(R, 1, len(offsets) - 1, 32)
    assert rc.shape == (B, Rs, C) and cc.shape == (B, C, Rs)
    vals = g.float().cpu().numpy().astype(np.float64)
    for b in range(B):
        padded = mx.pad_segments(vals[b], offsets)
        full = np.zeros((Rs, C))
        full[:len(padded)] = padded
        q, s = mx.quantize_rows(full)
        np.testing.assert_array_equal(rc[b].cpu().numpy(), q)
        np.testing.assert_array_equal(rs[b].cpu().numpy(), s)
        qc, sc = mx.quantize_cols_segmented(vals[b], offsets)
        n = qc.shape[1]
        np.testing.assert_array_equal(cc[b].cpu().numpy()[:, :n], qc)
        np.testing.assert_array_equal(cs[b].cpu().numpy()[:, :n // 32], sc)
        assert not cc[b].cpu().numpy()[:, n:].any() and not cs[b].cpu().numpy()[:, n // 32:].any()
