"""Writes synth/c3_router_bias.json: the per-expert router bias of the skewed workload.

The skewed workload (8 experts, 32768 tokens, top-2) wants expert token counts that
follow a Zipf law with s = 1.2 over six experts, and two experts with no tokens.
Experts 2 and 5 get a bias of -1e30 so they never enter the top-2; Zipf ranks 1..6
go to experts [3, 0, 6, 1, 7, 4].  The remaining biases come from a fixed-point
iteration b_e += 0.5 * (ln target_e - ln observed_e) on the workload's own seeded
logits, routed by the CPU oracle, until every share is within 2 % of its target.

Run:  python -m synth.calibrate_c3_bias
"""
from __future__ import annotations

import json
import os

import numpy as np

import synth
from oracle import route as rt

RANK_TO_EXPERT = [3, 0, 6, 1, 7, 4]
EMPTY = [2, 5]
ZIPF_S = 1.2


def main():
    w = synth.WORKLOADS[3]
    ranks = np.arange(1, 7, dtype=np.float64)
    share = ranks ** -ZIPF_S
    share /= share.sum()
    target = np.zeros(w.E)
    for r, e in enumerate(RANK_TO_EXPERT):
        target[e] = share[r]
    bias = np.zeros(w.E)
    bias[EMPTY] = -1e30
    for it in range(200):
        l = synth.logits(w, bias=bias.astype(np.float32))
        idx, _ = rt.route(l, w.k)
        obs = rt.split_sizes(idx, w.E) / float(w.T * w.k)
        live = [e for e in range(w.E) if e not in EMPTY]
        err = max(abs(obs[e] / target[e] - 1.0) for e in live)
        print(f"iter {it}: max rel share error {err:.4f}", flush=True)
        if err < 0.02:
            break
        for e in live:
            bias[e] += 0.5 * (np.log(target[e]) - np.log(max(obs[e], 1e-9)))
    sizes = rt.split_sizes(idx, w.E)
    out = dict(
        workload=w.name, zipf_s=ZIPF_S, rank_to_expert=RANK_TO_EXPERT, empty_experts=EMPTY,
        bias=[float(np.float32(b)) for b in bias], target_share=[float(t) for t in target],
        achieved_split_sizes=[int(s) for s in sizes],
    )
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c3_router_bias.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
