"""Seeded synthetic inputs for the grouped expert MLP workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no routing, no quantization, no GEMM).  Both the CPU oracle
tests and the GPU path take their inputs from here.

Recipe (one stream per tensor so tensors are independent of each other):
  numpy Generator(PCG64(SeedSequence([cfg_id, tensor_id]))), samples drawn in
  fp32, then rounded to bfloat16 with round-to-nearest-even (torch's conversion).
  tensor ids: logits=0, x=1, w_gate=2, w_up=3, w_down=4, dy=5.
  logits ~ N(0,1) fp32 [T][E] (+ a per-expert bias for the skewed workload)
  x ~ N(0,1) [T][H];  W_gate, W_up ~ N(0, 0.02^2) [E][F][H] stacked into
  W_gate_up [E][2F][H] (gate rows first);  W_down ~ N(0, 0.02^2) [E][H][F];
  dy ~ N(0,1) [T][H].
For the large Mixtral-shaped workloads the big tensors can also be drawn on the
GPU with torch's seeded generator (same distributions, different stream); the
logits always come from numpy so the routing, and hence split_sizes, is fixed.
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

TID_LOGITS, TID_X, TID_WGATE, TID_WUP, TID_WDOWN, TID_DY = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    """One expert-layer workload: sizes, precision and which passes run."""
    cfg_id: int
    name: str
    T: int
    E: int
    H: int
    F: int
    k: int
    prec: str            # "bf16" or "mxfp8"
    backward: bool
    skew: bool = False
    weight_std: float = 0.02
    extra: dict = field(default_factory=dict)

    @property
    def M(self) -> int:
        return self.T * self.k

    @property
    def ep(self) -> int:
        """Expert-parallel degree of a one-rank share (1: the whole layer on one GPU)."""
        return int(self.extra.get("ep", 1))

    @property
    def T_route(self) -> int:
        """Tokens the router sees: T per rank times the expert-parallel degree."""
        return self.T * self.ep

    def flops_fwd(self) -> float:
        # gate-up 4*M*H*F, down 2*M*H*F
        return 6.0 * self.M * self.H * self.F

    def flops_bwd(self) -> float:
        # dh 2MHF, dW_down 2MHF, dX 4MHF, dW_gate_up 4MHF
        return 12.0 * self.M * self.H * self.F


WORKLOADS = {
    0: Workload(0, "tiny_bf16_fwd_bwd", T=256, E=4, H=64, F=128, k=2, prec="bf16", backward=True),
    1: Workload(1, "mixtral_bf16_fwd", T=16384, E=8, H=4096, F=14336, k=2, prec="bf16", backward=False),
    2: Workload(2, "mixtral_mxfp8_fwd", T=16384, E=8, H=4096, F=14336, k=2, prec="mxfp8", backward=False),
    3: Workload(3, "mixtral_mxfp8_fwd_zipf_skew", T=32768, E=8, H=4096, F=14336, k=2, prec="mxfp8",
                backward=False, skew=True),
    4: Workload(4, "mixtral_mxfp8_train_step", T=8192, E=8, H=4096, F=14336, k=2, prec="mxfp8", backward=True),
    # One rank's share under expert parallelism: ep ranks of T tokens each are routed over
    # the 8 experts; rank 0 holds experts 0 .. 8/ep - 1 and receives their assignments.
    5: Workload(5, "mixtral_mxfp8_fwd_ep8_rank_share", T=16384, E=8, H=4096, F=14336, k=2, prec="mxfp8",
                backward=False, extra={"ep": 8}),
    6: Workload(6, "mixtral_mxfp8_fwd_ep4_rank_share", T=16384, E=8, H=4096, F=14336, k=2, prec="mxfp8",
                backward=False, extra={"ep": 4}),
    7: Workload(7, "mixtral_mxfp8_train_step_ep8_rank_share", T=8192, E=8, H=4096, F=14336, k=2, prec="mxfp8",
                backward=True, extra={"ep": 8}),
    # The training step's GEMMs as dense ones: one expert, top-1, the same 16384 rows, so
    # every M-tile shares one weight matrix (the shape of a plain dense FP8 GEMM).
    8: Workload(8, "mxfp8_train_step_one_expert", T=16384, E=1, H=4096, F=14336, k=1, prec="mxfp8", backward=True),
}


def rng(cfg_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, tensor_id])))


def to_bf16_values(a32: np.ndarray) -> np.ndarray:
    """Round fp32 samples to bfloat16 (RNE, via torch) and return them as fp32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def skew_bias(E: int) -> np.ndarray:
    """Per-expert router bias of the skewed workload (calibrated offline)."""
    with open(os.path.join(_HERE, "c3_router_bias.json")) as f:
        d = json.load(f)
    b = np.array(d["bias"], dtype=np.float32)
    assert b.shape == (E,)
    return b


def logits(w: Workload, bias: np.ndarray | None = None) -> np.ndarray:
    """Router logits fp32 [T_route][E]; the skewed workload adds its per-expert bias."""
    z = rng(w.cfg_id, TID_LOGITS).standard_normal((w.T_route, w.E), dtype=np.float32)
    if w.skew:
        b = skew_bias(w.E) if bias is None else bias.astype(np.float32)
        z = (z + b[None, :]).astype(np.float32)
    return z


def x(w: Workload) -> np.ndarray:
    return to_bf16_values(rng(w.cfg_id, TID_X).standard_normal((w.T, w.H), dtype=np.float32))


def dy(w: Workload) -> np.ndarray:
    return to_bf16_values(rng(w.cfg_id, TID_DY).standard_normal((w.T, w.H), dtype=np.float32))


def w_gate_up(w: Workload) -> np.ndarray:
    """[E][2F][H]: rows 0..F-1 are the gate projection, rows F..2F-1 the up projection."""
    g = rng(w.cfg_id, TID_WGATE).standard_normal((w.E, w.F, w.H), dtype=np.float32) * np.float32(w.weight_std)
    u = rng(w.cfg_id, TID_WUP).standard_normal((w.E, w.F, w.H), dtype=np.float32) * np.float32(w.weight_std)
    return to_bf16_values(np.concatenate([g, u], axis=1))


def w_down(w: Workload) -> np.ndarray:
    d = rng(w.cfg_id, TID_WDOWN).standard_normal((w.E, w.H, w.F), dtype=np.float32) * np.float32(w.weight_std)
    return to_bf16_values(d)


def custom(cfg_id: int, T: int, E: int, H: int, F: int, k: int, prec: str = "bf16",
           backward: bool = True, weight_std: float = 0.02) -> Workload:
    """Ad-hoc workload (edge-case tests); cfg_id seeds the streams."""
    return Workload(cfg_id, f"custom_{cfg_id}", T=T, E=E, H=H, F=F, k=k, prec=prec, backward=backward,
                    weight_std=weight_std)


def torch_normal_bf16(shape, std: float, seed: int, device):
    """Large tensors drawn on the device with torch's seeded generator, rounded to bfloat16."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, std, generator=g)
    return t.to(torch.bfloat16)
