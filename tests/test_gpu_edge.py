"""Edge cases of the whole path, forward + backward in BF16 and MXFP8, against the oracle.

Uneven routing must run without a per-expert loop ([P2] "Fragmented Expert Kernels": the
grouped call takes per-expert token counts).  The routing is given (caller top-k), so the
groups have exactly the sizes under test:
  * groups of 0, 1, 31, 32, 33, 255, 256, 257 and 513 rows: empty, single-row, around the
    32-row scale block and the 256-row M-tile, several tiles with a ragged tail;
  * H = F = 32, the smallest sizes the layout allows (one scale block along K);
  * one expert receiving every token at E = 8 (seven empty experts, k = 2);
  * a single token (T = 1);
  * the grid's last round as quarter-width work items: 2 experts of 2176 rows each (every
    token on both), H = 4096, so the dX and down GEMMs have 2 x 9 x 16 = 288 tiles on 256
    CUs, and their last 32 tiles (the second expert's last two M-tiles, one of them half
    full) run as 128 items of 256 x 64 in the tail launch.
BF16: y, dx, dW_gate_up, dW_down and d_prob end to end against fp64 on the same bf16
inputs (rel_F 1e-2).  MXFP8: staged, each stage against the oracle fed the GPU's own
quantized operands (rel_F 2e-3; x, dy, weights and the permutation bit-exact; h and dGU
compared after dequantization with their code flips bounded); a bf16-stored stage output
of under 4096 elements (the single token) whose rel_F exceeds 2e-3 is held element by
element to one bf16 rounding instead.  Experts without tokens
get exactly zero weight gradients in both."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import moe_grouped_expert_amd as mge
    return mge


def _case(name):
    """(x, wgu, wd, dy, E, k, idx, prob, logits): exact bf16 values as fp32 numpy."""
    rng = np.random.default_rng(CASES.index(name) + 900)
    logits = None
    if name == "sizes":
        sizes = [0, 1, 31, 32, 33, 255, 256, 257, 513]
        E, k, H, F = len(sizes), 1, 64, 96
        idx = np.concatenate([np.full(s, e, np.int32) for e, s in enumerate(sizes)])
        idx = rng.permutation(idx)[:, None].astype(np.int32)        # tokens of all experts interleaved
        prob = rng.uniform(0.2, 1.0, idx.shape).astype(np.float32)
    elif name == "h32_f32":
        E, k, H, F, T = 4, 2, 32, 32, 150
        logits = rng.standard_normal((T, E)).astype(np.float32)
        idx = prob = None
    elif name == "one_expert_all_tokens":
        E, k, H, F, T = 8, 2, 64, 64, 300
        idx = np.stack([np.full(T, 3), rng.choice([0, 1, 2, 4, 5, 6, 7], T)], axis=1).astype(np.int32)
        idx[::2] = idx[::2, ::-1]                                    # expert 3 in either slot
        p0 = rng.uniform(0.5, 0.9, T).astype(np.float32)
        prob = np.stack([p0, 1 - p0], axis=1).astype(np.float32)
    elif name == "one_token":
        E, k, H, F, T = 8, 2, 64, 96, 1
        logits = rng.standard_normal((T, E)).astype(np.float32)
        idx = prob = None
    elif name == "tail_split":
        E, k, H, F, T = 2, 2, 4096, 256, 2176
        idx = np.tile(np.array([[0, 1]], np.int32), (T, 1))
        idx[::2] = idx[::2, ::-1]                                    # either expert in slot 0
        prob = rng.uniform(0.2, 0.8, (T, k)).astype(np.float32)
    else:
        raise ValueError(name)
    T = idx.shape[0] if idx is not None else logits.shape[0]
    x = synth.to_bf16_values(rng.standard_normal((T, H)).astype(np.float32))
    wgu = synth.to_bf16_values((rng.standard_normal((E, 2 * F, H)) * 0.05).astype(np.float32))
    wd = synth.to_bf16_values((rng.standard_normal((E, H, F)) * 0.05).astype(np.float32))
    dy = synth.to_bf16_values(rng.standard_normal((T, H)).astype(np.float32))
    return x, wgu, wd, dy, E, k, idx, prob, logits


CASES = ["sizes", "h32_f32", "one_expert_all_tokens", "one_token", "tail_split"]


def _needs_256_cus(name):
    if name == "tail_split" and torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the tile arithmetic of this case assumes 256 compute units")


@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
@pytest.mark.parametrize("name", CASES)
def test_edge_fwd_bwd(m, name, prec):
    from tests.gpu_helpers import check_fwd_bwd, npy, say
    _needs_256_cus(name)
    x, wgu, wd, dy, E, k, idx, prob, logits = _case(name)
    say("[gpu] edge", name, prec, "T", x.shape[0], "E", E, "k", k, "H", x.shape[1], "F", wd.shape[2])
    o = check_fwd_bwd(m, prec, x, wgu, wd, dy, E, k, idx, prob, logits)
    if name == "sizes":
        np.testing.assert_array_equal(npy(o["g"].split_sizes), [0, 1, 31, 32, 33, 255, 256, 257, 513])

@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
def test_tail_split_rerun_identical(m, prec):
    """Two runs of the case whose dX and down GEMMs end in the quarter-width tail launch give
    the same bits: each output element is one wave's K sum in a fixed order, whichever launch
    computes it."""
    from tests.gpu_helpers import run_fwd_bwd, say
    _needs_256_cus("tail_split")
    args = _case("tail_split")
    say("[gpu] edge tail_split rerun", prec)
    a = run_fwd_bwd(m, prec, *args)
    b = run_fwd_bwd(m, prec, *args)
    v = a["g"].perm_src >= 0            # padding rows of the permuted outputs are not written
    assert torch.equal(a["g"].perm_src, b["g"].perm_src)
    assert torch.equal(a["f"].y_perm[v], b["f"].y_perm[v]) and torch.equal(a["b"].dx_perm[v], b["b"].dx_perm[v])
    assert torch.equal(a["y"], b["y"]) and torch.equal(a["dx"], b["dx"])
    assert all(torch.equal(u, v) for u, v in zip(a["b"].dw_gate_up, b["b"].dw_gate_up))
    assert all(torch.equal(u, v) for u, v in zip(a["b"].dw_down, b["b"].dw_down))
    assert torch.equal(a["b"].d_prob, b["b"].d_prob)
