"""A seeded sweep of random configurations through the whole path, forward + backward in
BF16 and MXFP8, against the oracle at the edge-case bars (tests/gpu_helpers.check_fwd_bwd):
BF16 end to end within rel_F 1e-2 of fp64, MXFP8 staged within 2e-3 on the GPU's own codes
with bit-exact routing, permutation and operand codes.

The configurations are drawn once from a fixed seed: expert counts 1 to 256, top-k up to
min(E, 8), H and F any multiple of 32 up to 384, 1 to 1500 tokens, and four kinds of routing
(router logits; logits with a skew bias that leaves some experts empty; caller-given
distinct experts; caller-given experts that may repeat within a token, whose repeated slots
each take a row of their own)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

ROUTINGS = ("logits", "skew", "given", "given_repeat")


def _configs(n=16, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 3, 5, 8, 16, 33, 64, 128, 256]))
        k = int(rng.integers(1, min(E, 8) + 1))
        H = 32 * int(rng.integers(1, 13))
        F = 32 * int(rng.integers(1, 13))
        T = int(np.exp(rng.uniform(0.0, np.log(1500.0))))
        routing = ROUTINGS[i % len(ROUTINGS)]
        out.append((i, E, k, H, F, max(T, 1), routing))
    return out


CONFIGS = _configs()


def _inputs(i, E, k, H, F, T, routing):
    """(x, wgu, wd, dy, E, k, idx, prob, logits) of one configuration: exact bf16 values as fp32."""
    rng = np.random.default_rng(7000 + i)
    logits = idx = prob = None
    if routing in ("logits", "skew"):
        logits = rng.standard_normal((T, E)).astype(np.float32)
        if routing == "skew" and E > k:
            # a Zipf-like tilt, and up to a quarter of the experts (never more than E - k) empty
            logits += (-1.5 * np.log1p(rng.permutation(E))).astype(np.float32)[None, :]
            n_empty = min(E // 4, E - k)
            if n_empty > 0:
                logits[:, rng.choice(E, n_empty, replace=False)] = -1e30
    else:
        if routing == "given":
            idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        else:
            idx = rng.integers(0, E, (T, k)).astype(np.int32)
        prob = rng.uniform(0.05, 1.0, (T, k)).astype(np.float32)
    x = synth.to_bf16_values(rng.standard_normal((T, H)).astype(np.float32))
    wgu = synth.to_bf16_values((rng.standard_normal((E, 2 * F, H)) / np.sqrt(H)).astype(np.float32))
    wd = synth.to_bf16_values((rng.standard_normal((E, H, F)) / np.sqrt(F)).astype(np.float32))
    dy = synth.to_bf16_values(rng.standard_normal((T, H)).astype(np.float32))
    return x, wgu, wd, dy, E, k, idx, prob, logits


@pytest.fixture(scope="module")
def m():
    import moe_grouped_expert_amd as mge
    return mge


@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: f"c{c[0]}-E{c[1]}-k{c[2]}-H{c[3]}-F{c[4]}-T{c[5]}-{c[6]}")
def test_random_fwd_bwd(m, cfg, prec):
    from tests.gpu_helpers import check_fwd_bwd, say
    say("[gpu] random", prec, cfg)
    check_fwd_bwd(m, prec, *_inputs(*cfg))
