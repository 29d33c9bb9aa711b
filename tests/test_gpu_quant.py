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
