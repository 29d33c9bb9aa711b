"""Shared plumbing of the GPU parity tests: build seeded inputs, run the HIP path
through the C ABI, bring results back as numpy."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth
from oracle import mlp
from oracle import route as rt


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def gpu_bf16(a32: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16).to(dev())


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def npy(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


class Inputs:
    """Seeded inputs of one workload, as numpy (exact bf16 values in fp32) and on the GPU."""

    def __init__(self, w: synth.Workload, logits: np.ndarray | None = None):
        self.w = w
        self.logits = synth.logits(w) if logits is None else logits.astype(np.float32)
        self.x = synth.x(w)
        self.wgu = synth.w_gate_up(w)
        self.wd = synth.w_down(w)
        self.dy = synth.dy(w)
        self.g_logits = torch.from_numpy(self.logits).to(dev())
        self.g_x = gpu_bf16(self.x)
        self.g_wgu = gpu_bf16(self.wgu)
        self.g_wd = gpu_bf16(self.wd)
        self.g_dy = gpu_bf16(self.dy)


def layout_from_gpu(route, E: int, align: int) -> mlp.Layout:
    """Oracle layout built from the GPU's routing decision (indices are checked bit-exact
    elsewhere; probabilities are the GPU's fp32 values, an input to the later stages)."""
    return mlp.Layout(npy(route.topk_idx), npy(route.topk_prob).astype(np.float64), E, align)
