#!/usr/bin/env python3
"""Throughput of the grouped expert MLP hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input, every
stage in the library's HIP kernels through the C ABI:
  moe_route_permute (top-k routing, split_sizes, stable permutation, x gathered and
  MXFP8-quantized row- and column-wise) -> mxfp8_quantize of the 16-bit master
  weights (row and column forms, as every training step re-quantizes them) ->
  grouped_mlp_fwd (gate-up GEMM + SwiGLU x prob + quantize-h epilogue, down GEMM) ->
  unpermute_combine -> grouped_mlp_bwd (dy permute + quantize, dh GEMM + SwiGLU
  backward, d_prob, dW_down, dX, dW_gate_up) -> unpermute_combine of dx ->
  moe_router_bwd (d_logits from d_prob).

Default workload: the Mixtral-8x7B-shaped expert layer (8 experts, hidden 4096,
ffn 14336, top-2) training step in MXFP8 with 16-bit master weights, 8192 tokens.
Inputs are seeded synthetic tensors, resident in HBM before timing starts.

Prints ONE JSON line.  `value` is algorithmic TFLOP/s of the step (6*M*H*F forward +
12*M*H*F backward, M = tokens * top-k; no padding, no recompute); tokens/s beside it.
`ms_per_step` comes from a pass of K steps with no per-kernel events; `roofline` is for
the kernel with the largest share of the step time, from HIP events recorded around
each kernel launch on its own stream during a second pass of K steps (whose own time
is `profiled_ms_per_step`).  `cpu_baseline` is the fp64 CPU oracle timed on a bounded sample of the same
workload (rank 0, one GPU only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "grouped-MLP fwd/bwd TFLOP/s + tokens/s, Mixtral-8x7B expert layer, MXFP8"

# Published dense MFMA peaks of the MI355X (TFLOP/s) and its HBM3E bandwidth (GB/s).
PEAK_TFLOPS = {"mxfp8": 5000.0, "bf16": 2500.0}
PEAK_HBM_GBS = 8000.0

WORKLOADS = {
    # name: (synth workload id, training step?)
    "train_mxfp8": (4, True),
    "fwd_bf16": (1, False),
    "fwd_mxfp8": (2, False),
    "fwd_mxfp8_skew": (3, False),
    "tiny_bf16": (0, True),    # 4 experts, hidden 64, ffn 128, 256 tokens: latency-bound
    # one rank's share of an expert-parallel layer (its local experts, its received rows)
    "fwd_mxfp8_ep8": (5, False),
    "fwd_mxfp8_ep4": (6, False),
    "train_mxfp8_ep8": (7, True),
    # the same step on one expert (top-1, 16384 rows): the GEMMs as dense ones
    "train_mxfp8_dense": (8, True),
}

# How the forward runs: one grouped launch per projection over every expert with the
# SwiGLU x prob (+ quantize) fused into the gate-up epilogue ("grouped", the method);
# one launch per expert and projection with the same kernels ("expert_loop", the
# per-expert loop the grouped call replaces); or grouped launches without the fusion,
# [G U] through HBM in bf16, a standalone SwiGLU x prob and a standalone quantize of h
# ("unfused", what the fused operation replaces); or the unfused chain in FP8 with one
# scale per tensor instead of one per block of 32 ("fp8_tensor": x, each expert's
# weights and h each take one power-of-two scale from their amax; the GEMMs are the
# block-scaled ones with every block of a tensor on the same scale).
VARIANTS = ("grouped", "expert_loop", "unfused", "fp8_tensor")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------ inputs

def make_inputs(w, dev):
    """Seeded inputs: routing logits from numpy (fixes split_sizes), the large tensors
    drawn on the device with torch's seeded generator, same distributions."""
    import torch

    import synth
    logits = torch.from_numpy(synth.logits(w)).to(dev)
    x = synth.torch_normal_bf16((w.T, w.H), 1.0, 1000 * w.cfg_id + synth.TID_X, dev)
    wg = synth.torch_normal_bf16((w.E, w.F, w.H), w.weight_std, 1000 * w.cfg_id + synth.TID_WGATE, dev)
    wu = synth.torch_normal_bf16((w.E, w.F, w.H), w.weight_std, 1000 * w.cfg_id + synth.TID_WUP, dev)
    wgu = torch.cat([wg, wu], dim=1).contiguous()
    del wg, wu
    wd = synth.torch_normal_bf16((w.E, w.H, w.F), w.weight_std, 1000 * w.cfg_id + synth.TID_WDOWN, dev)
    dy = synth.torch_normal_bf16((w.T, w.H), 1.0, 1000 * w.cfg_id + synth.TID_DY, dev) if w.backward else None
    return dict(logits=logits, x=x, wgu=wgu, wd=wd, dy=dy)


def make_ep_share_inputs(m, w, dev):
    """Inputs of rank 0 of an expert-parallel layer with w.ep ranks of w.T tokens each.

    The w.ep * w.T tokens are routed over all E experts with the library's router (set-up,
    outside the timed steps); rank 0 holds experts 0 .. E/ep - 1 and receives every
    assignment routed to them, in the order (source token, slot), with its expert index
    (local = global here) and its routing probability: what an all-to-all-v of the
    dispatching ranks' permuted rows delivers.  The received rows of x (and of dy for the
    training step) are drawn fresh, N(0, 1) like the tokens they stand for.  Returns the
    inputs and the rank's local problem as a workload: T = rows received, k = 1."""
    import dataclasses

    import torch

    import synth
    e_loc = w.E // w.ep
    logits = torch.from_numpy(synth.logits(w)).to(dev)
    g = m.moe_route_permute(logits, None, w.k, align=32)
    mask = g.topk_idx < e_loc
    idx = g.topk_idx[mask].to(torch.int32).reshape(-1, 1).contiguous()
    prob = g.topk_prob[mask].to(torch.float32).reshape(-1, 1).contiguous()
    n = int(idx.shape[0])
    wl = dataclasses.replace(w, T=n, E=e_loc, k=1, extra={})
    x = synth.torch_normal_bf16((n, w.H), 1.0, 1000 * w.cfg_id + synth.TID_X, dev)
    wg = synth.torch_normal_bf16((e_loc, w.F, w.H), w.weight_std, 1000 * w.cfg_id + synth.TID_WGATE, dev)
    wu = synth.torch_normal_bf16((e_loc, w.F, w.H), w.weight_std, 1000 * w.cfg_id + synth.TID_WUP, dev)
    wgu = torch.cat([wg, wu], dim=1).contiguous()
    del wg, wu
    wd = synth.torch_normal_bf16((e_loc, w.H, w.F), w.weight_std, 1000 * w.cfg_id + synth.TID_WDOWN, dev)
    dy = synth.torch_normal_bf16((n, w.H), 1.0, 1000 * w.cfg_id + synth.TID_DY, dev) if w.backward else None
    return dict(logits=None, idx=idx, prob=prob, x=x, wgu=wgu, wd=wd, dy=dy), wl


# ------------------------------------------------------------------------------ step

class Step:
    """The hot path with every output buffer allocated once (allocation stays outside
    the timed region; the library itself never allocates).

    With inputs from make_ep_share_inputs the step is one expert-parallel rank's: the
    received rows are permuted by their given local expert and probability (k = 1), and
    the router's backward stays with the dispatching ranks.  variant "expert_loop" runs
    the forward as one single-group grouped_mlp_fwd per expert, "unfused" as
    grouped_mlp_fwd_unfused (both inference only).  keep_intermediates keeps the unfused
    call's [G U] and bf16 h, and the backward's dY and dGU codes, in buffers of their own
    instead of the workspace (the same kernels; the parity tests read them)."""

    def __init__(self, m, w, inp, train, variant="grouped", dw_dtype="f32"):
        self.m, self.w, self.inp, self.train = m, w, inp, train
        self.variant = variant
        self.dw_dtype = dw_dtype
        self.keep_intermediates = False
        self.prec = w.prec
        self.given = inp.get("idx") is not None
        self.g = None
        self.wq = self.dq = None
        self.f = self.b = None
        self.y = self.dx = self.dl = None
        self.groups = None
        self.ts = {}

    def _fwd_expert_loop(self):
        """E launches of each projection: expert e's group alone, as a one-expert call
        whose sizes and offsets are the e-th entries of the device arrays (nothing is
        read back to the host) over the shared permuted buffers (T = R rows, k = 1,
        align = 1, so the call's row count is R)."""
        import dataclasses

        m, g = self.m, self.g
        if self.groups is None:
            self.groups = [dataclasses.replace(g, E=1, T=g.R, k=1, align=1, split_sizes=g.split_sizes[e:e + 1],
                                               group_offsets=g.group_offsets[e:e + 2]) for e in range(g.E)]
        mx = self.prec == "mxfp8"
        for e, ge in enumerate(self.groups):
            if mx:
                self.f = m.grouped_mlp_fwd(ge, self.wq[0][e:e + 1], self.dq[0][e:e + 1], self.wq[1][e:e + 1],
                                           self.dq[1][e:e + 1], out=self.f)
            else:
                self.f = m.grouped_mlp_fwd(ge, self.inp["wgu"][e:e + 1], self.inp["wd"][e:e + 1], out=self.f)
        return self.f

    def _fp8_tensor(self):
        """FP8 with one scale per tensor: the scale of x, of each expert's W_gate_up and
        W_down, and of h (inside the unfused forward) from their amax, every block of a
        tensor quantized with it.  Training also quantizes the weights' column forms with
        their scale, saves [G U] and h's column form, and runs the backward with one scale
        for dY and one for [dG dU]."""
        m, w, inp, ts = self.m, self.w, self.inp, self.ts
        ts["x"] = m.tensor_scale(inp["x"], out=ts.get("x"))
        self.g = m.moe_route_permute(inp["logits"], inp["x"], w.k, align=32, prec="mxfp8", want_col=self.train,
                                     out=self.g, x_tensor_scale=ts["x"].scale)
        ts["wgu"] = m.tensor_scale(inp["wgu"], per_matrix=True, out=ts.get("wgu"))
        ts["wd"] = m.tensor_scale(inp["wd"], per_matrix=True, out=ts.get("wd"))
        orient = "both" if self.train else "row"
        self.wq = m.mxfp8_quantize(inp["wgu"], orient, out=self.wq, tensor_scale=ts["wgu"].scale)
        self.dq = m.mxfp8_quantize(inp["wd"], orient, out=self.dq, tensor_scale=ts["wd"].scale)
        self.f = m.grouped_mlp_fwd_unfused(self.g, self.wq[0], self.dq[0], self.wq[1], self.dq[1], h_per_tensor=True,
                                           keep_intermediates=self.keep_intermediates, train=self.train, out=self.f)
        self.y = m.unpermute_combine(self.f.y_perm, self.g.perm_pos, out=self.y)
        if self.train:
            self.b = m.grouped_mlp_bwd(inp["dy"], self.g, self.f, self.wq[2], self.dq[2], self.wq[3], self.dq[3],
                                       keep_intermediates=self.keep_intermediates, out=self.b, dw_dtype=self.dw_dtype,
                                       per_tensor=True)
            self.dx = m.unpermute_combine(self.b.dx_perm, self.g.perm_pos, out=self.dx)
            self.dl = m.moe_router_bwd(self.g.topk_idx, self.g.topk_prob, self.b.d_prob, w.E, out=self.dl)

    def __call__(self):
        m, w, inp = self.m, self.w, self.inp
        mx = self.prec == "mxfp8"
        if self.variant == "fp8_tensor":
            self._fp8_tensor()
            return
        if self.given:
            self.g = m.moe_route_permute(None, inp["x"], 1, E=w.E, align=32, prec=self.prec, want_col=self.train,
                                         topk_idx=inp["idx"], topk_prob=inp["prob"], out=self.g)
        else:
            self.g = m.moe_route_permute(inp["logits"], inp["x"], w.k, align=32, prec=self.prec,
                                         want_col=self.train, out=self.g)
        if mx:
            orient = "both" if self.train else "row"
            self.wq = m.mxfp8_quantize(inp["wgu"], orient, out=self.wq)
            self.dq = m.mxfp8_quantize(inp["wd"], orient, out=self.dq)
        if self.variant == "expert_loop":
            self._fwd_expert_loop()
        elif self.variant == "unfused":
            if mx:
                self.f = m.grouped_mlp_fwd_unfused(self.g, self.wq[0], self.dq[0], self.wq[1], self.dq[1],
                                                   keep_intermediates=self.keep_intermediates, out=self.f)
            else:
                self.f = m.grouped_mlp_fwd_unfused(self.g, inp["wgu"], inp["wd"],
                                                   keep_intermediates=self.keep_intermediates, out=self.f)
        elif mx:
            self.f = m.grouped_mlp_fwd(self.g, self.wq[0], self.dq[0], self.wq[1], self.dq[1], train=self.train,
                                       out=self.f)
        else:
            self.f = m.grouped_mlp_fwd(self.g, inp["wgu"], inp["wd"], train=self.train, out=self.f)
        self.y = m.unpermute_combine(self.f.y_perm, self.g.perm_pos, out=self.y)
        if self.train:
            if mx:
                self.b = m.grouped_mlp_bwd(inp["dy"], self.g, self.f, self.wq[2], self.dq[2], self.wq[3], self.dq[3],
                                           keep_intermediates=self.keep_intermediates, out=self.b,
                                           dw_dtype=self.dw_dtype)
            else:
                self.b = m.grouped_mlp_bwd(inp["dy"], self.g, self.f, inp["wgu"], inp["wd"],
                                           keep_intermediates=self.keep_intermediates, out=self.b,
                                           dw_dtype=self.dw_dtype)
            self.dx = m.unpermute_combine(self.b.dx_perm, self.g.perm_pos, out=self.dx)
            if not self.given:
                self.dl = m.moe_router_bwd(self.g.topk_idx, self.g.topk_prob, self.b.d_prob, w.E, out=self.dl)


# ------------------------------------------------------------------------------ per-kernel work

def kernel_work(name, w, R, launches_per_step=1.0):
    """Algorithmic work of one launch of a library kernel: ("flop", n) or ("byte", n).

    GEMMs: the method's flops on the M = T*k real rows (no padding rows), shared by the
    step's launches of that GEMM (one grouped launch, or one per expert in the expert
    loop).  HBM-bound kernels: bytes that must cross HBM once (inputs read, outputs
    written) per launch."""
    M, H, F, T, k, E = w.M, w.H, w.F, w.T, w.k, w.E
    mhf = float(M) * H * F
    gemm = {"gemm_gateup_swiglu": 4 * mhf, "gemm_gateup_store": 4 * mhf, "gemm_down": 2 * mhf, "gemm_dh": 2 * mhf,
            "gemm_dx": 4 * mhf, "gemm_dw_down": 2 * mhf, "gemm_dw_gateup": 4 * mhf}
    for key, v in gemm.items():
        if name.startswith(key + "_"):
            return "flop", v / max(launches_per_step, 1.0)
    mxb = 1.0 + 1.0 / 32.0            # bytes per MXFP8 element (code + scale share)
    if name == "permute_quant_mx":
        # x or dy gathered (bf16 read once per token) -> row and (training) column forms
        forms = 2 if w.backward else 1
        return "byte", 2.0 * T * H + forms * mxb * M * H + 4.0 * R
    if name == "permute_bf16":
        return "byte", 2.0 * T * H + (2 if w.backward else 1) * 2.0 * M * H + 4.0 * R
    if name == "quant_mx":
        # the step's two weight quantizations (W_gate_up: 2FH, W_down: HF per expert),
        # averaged per launch: bf16 read, row and (training) column forms written
        forms = 2 if w.backward else 1
        return "byte", 1.5 * E * H * F * (2.0 + forms * mxb)
    if name == "transpose_bf16":
        # BF16 backward: each expert's W_down [H][F] and W_gate_up [2F][H] transposed
        # (2 B read + 2 B written per element), two launches per expert: 6*H*F B on average
        return "byte", 6.0 * H * F
    if name == "swiglu_prob":
        # unfused forward: [G U] bf16 read, h bf16 written, p read (valid rows)
        return "byte", 6.0 * M * F + 4.0 * M
    if name == "quant_h_mx":
        # unfused forward: the bf16 h read, its row form (and, training, column form) written
        return "byte", M * F * (2.0 + (2 if w.backward else 1) * mxb)
    if name == "quant_dgu_mx":
        # FP8 with one scale per tensor: the bf16 [dG dU] read, both forms written
        return "byte", M * 2.0 * F * (2.0 + 2 * mxb)
    if name == "combine":
        return "byte", 2.0 * k * T * H + 2.0 * T * H + 4.0 * T * k
    if name == "router_bwd":
        # indices, probabilities and d_prob read once, d_logits written
        return "byte", 12.0 * T * k + 4.0 * T * E
    if name in ("route_topk", "route_scatter"):
        return "byte", 4.0 * T * E + 8.0 * T * k if name == "route_topk" else 4.0 * T * k * 4
    return None


def summarize_kernels(records, steps, w, R, prec):
    """Aggregates the per-launch event timings into per-kernel statistics."""
    agg = {}
    for name, ms in records:
        if ms < 0:
            continue
        a = agg.setdefault(name, dict(launches=0, total_ms=0.0))
        a["launches"] += 1
        a["total_ms"] += ms
    total = sum(a["total_ms"] for a in agg.values())
    out = {}
    for name, a in sorted(agg.items(), key=lambda kv: -kv[1]["total_ms"]):
        avg = a["total_ms"] / a["launches"]
        d = dict(launches_per_step=a["launches"] / steps, avg_ms=round(avg, 5),
                 share=round(a["total_ms"] / total, 4) if total > 0 else None)
        wk = kernel_work(name, w, R, a["launches"] / steps)
        if wk is not None:
            kind, n = wk
            if kind == "flop":
                tf = n / (avg * 1e-3) / 1e12
                d.update(tflops=round(tf, 1), frac_of_peak=round(tf / PEAK_TFLOPS[prec], 4))
            else:
                gbs = n / (avg * 1e-3) / 1e9
                d.update(gbs=round(gbs, 1), frac_of_hbm=round(gbs / PEAK_HBM_GBS, 4))
        out[name] = d
    return out, total / steps


# ------------------------------------------------------------------------------ traffic (rocprofv3 counters)

# Sources that build a kernel family: the GEMM kernels are made from these files, from
# the grouped-GEMM part of mge_internal.hpp (GemmParams) and from the launch constants of
# api.cpp (raster bands); every other kernel is checked against all sources.
GEMM_SOURCES = ("gemm_impl.hpp", "gemm_mx.hip", "gemm_bf16.hip", "gemm_host.cpp", "mge_common.hpp")
GEMM_PARAMS_MARK = "// ------------------------------------------------------------ grouped GEMM"


def _code_text(text):
    """C/C++ source bytes without comments, trailing blanks and empty lines: what the
    compiler sees, so that counters stay attached to a kernel across comment edits."""
    out, in_block = [], False
    for line in text.decode("utf-8", "replace").split("\n"):
        code, i, n = [], 0, len(line)
        while i < n:
            if in_block:
                j = line.find("*/", i)
                if j < 0:
                    break
                in_block, i = False, j + 2
                continue
            c = line[i]
            if c in "\"'":                      # string or character literal, copied whole
                j = i + 1
                while j < n and line[j] != c:
                    j += 2 if line[j] == "\\" else 1
                code.append(line[i:j + 1])
                i = j + 1
                continue
            if line.startswith("//", i):
                break
            if line.startswith("/*", i):
                in_block, i = True, i + 2
                continue
            code.append(c)
            i += 1
        kept = "".join(code).rstrip()
        if kept.strip():
            out.append(kept)
    return "\n".join(out).encode()


def kernel_source_digest(family="all"):
    """Digest of the code of a kernel family ("gemm" or "all"), comments left out:
    counter-derived traffic is only reported while the kernels are the ones the counters
    were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_grouped_expert_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if not f.endswith((".hip", ".hpp", ".cpp", ".h")):
            continue
        with open(os.path.join(csrc, f), "rb") as fh:
            text = fh.read()
        if family == "gemm":
            if f == "mge_internal.hpp":
                text = text[text.index(GEMM_PARAMS_MARK.encode()):]
            elif f == "api.cpp":
                # the launch settings the host passes the GEMMs (raster bands and the like)
                text = b"\n".join(l for l in text.split(b"\n") if l.startswith(b"constexpr int k"))
            elif f not in GEMM_SOURCES:
                continue
        h.update(f.encode() + b"\0" + _code_text(text))
    return h.hexdigest()[:16]


def _digest_family(kernel):
    return "gemm" if kernel.startswith("gemm_") else "all"


COPY_CAL_BYTES = 1 << 30   # the plain device-to-device copy the counters are calibrated on


def calibrate_copy():
    """A plain 1 GiB device-to-device copy (three launches): under rocprofv3 --pmc its
    FETCH_SIZE / WRITE_SIZE readings give the factor from counter units to HBM bytes."""
    import torch

    src = torch.ones(COPY_CAL_BYTES, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_CAL_BYTES, "launches": 3}))


def _short_kernel(name):
    """'mge::gemm_dx_mx(mge::GemmParams)' -> 'gemm_dx_mx'; 'void mge::k<true>(...)' -> 'k<true>'."""
    if name.startswith("void "):
        name = name[5:]
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):   # the parameter list starts at the first '(' outside <...>
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    name = name[:cut]
    return name[5:] if name.startswith("mge::") else name


def _counter_values(path):
    import csv

    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def summarize_counters(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, workload):
    """profiles/traffic.json from four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE, in
    KiB per dispatch, over one training step and over the 1 GiB copy): per library kernel,
    the mean per dispatch of each counter scaled by copy_bytes / (copy's reading)."""
    def cal(path):
        vals = [v for n, vs in _counter_values(path).items() if "copyBuffer" in n or "copy" in n.lower() for v in vs]
        return COPY_CAL_BYTES / (max(vals) * 1024.0)

    f_scale, w_scale = cal(cal_fetch_csv), cal(cal_write_csv)
    fetch, write = _counter_values(fetch_csv), _counter_values(write_csv)
    kernels = {}
    for name, fv in fetch.items():
        if "mge::" not in name or name not in write:
            continue
        wv = write[name]
        fb = sum(fv) / len(fv) * 1024.0 * f_scale
        wb = sum(wv) / len(wv) * 1024.0 * w_scale
        kernels[_short_kernel(name)] = {"dispatches": len(fv), "fetch_bytes": round(fb), "write_bytes": round(wb),
                                        "hbm_bytes_per_launch": round(fb + wb)}
    out = {"source_digest": kernel_source_digest(),
           "source_digests": {fam: kernel_source_digest(fam) for fam in ("all", "gemm")},
           "calibration": {"copy_bytes": COPY_CAL_BYTES, "fetch_factor": round(f_scale, 5),
                           "write_factor": round(w_scale, 5)},
           "kernels": {workload: kernels}}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(f"wrote {path}: {len(kernels)} kernels, fetch x{f_scale:.4f}, write x{w_scale:.4f}")


def traffic_for(kernel, workload):
    """HBM bytes per launch of `kernel` from profiles/traffic.json (FETCH_SIZE + WRITE_SIZE
    per dispatch, scaled by the copy-kernel calibration), or None when absent or stale."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    fam = _digest_family(kernel)
    if d.get("source_digests", {}).get(fam) != kernel_source_digest(fam):
        return None
    e = d.get("kernels", {}).get(workload, {}).get(kernel)
    return None if e is None else e.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------------------ CPU baseline

def cpu_baseline(w, max_rows=None, f_cols=None):
    """The fp64 CPU oracle, as it stands, on a bounded sample of the workload.

    Sample: expert 0 of the workload, the first `max_rows` assignments routed to it
    (None: all of them, the expert's whole group; their tokens and routing probabilities
    from the oracle's own routing of the workload's logits), the full hidden size and
    the first `f_cols` of the expert's ffn columns (gate, up and down weights restricted
    to them), through the whole
    MXFP8 training step (or forward) as the oracle defines it (BF16 workloads: the grouped
    definition on the bf16 values): quantize the weights
    (row and column forms), permute and quantize x, gate-up GEMM + SwiGLU x prob,
    quantize h, down GEMM, combine; backward: dy permute/quantize, dh + SwiGLU
    backward, d_prob, dW_down, dX, dW_gate_up.  Rate = the sample's algorithmic flops
    (the same 6 + 12 flops per assignment, hidden and ffn column) / wall time."""
    import numpy as np

    import synth
    from oracle import mlp, mx
    from oracle import route as rt

    cores = len(os.sched_getaffinity(0))
    if max_rows is None:
        l = synth.logits(w)                                          # every token: expert 0's whole group
    else:
        l = synth.logits(w)[:max(4096, 2 * max_rows * w.E // w.k)]   # enough tokens to find max_rows for expert 0
    idx, p = rt.route(l, w.k)
    hit = np.argwhere(idx == 0)[:max_rows]
    toks, slots = hit[:, 0], hit[:, 1]
    n = len(toks)
    fs = w.F if f_cols is None else min(f_cols, w.F)
    std = np.float32(w.weight_std)
    # expert 0's weights from the workload's numpy streams (the first rows of each stream
    # are expert 0), restricted to the sampled ffn columns
    wg0 = synth.to_bf16_values(synth.rng(w.cfg_id, synth.TID_WGATE).standard_normal((fs, w.H), dtype=np.float32) * std)
    wu0 = synth.to_bf16_values(synth.rng(w.cfg_id, synth.TID_WUP).standard_normal((fs, w.H), dtype=np.float32) * std)
    wd0 = synth.to_bf16_values(
        synth.rng(w.cfg_id, synth.TID_WDOWN).standard_normal((w.H, w.F), dtype=np.float32)[:, :fs] * std)
    wgu0 = np.concatenate([wg0, wu0], axis=0)
    xs = synth.x(w)[toks]
    dys = synth.dy(w)[toks] if w.backward else None
    t0 = time.perf_counter()
    lay = mlp.Layout(np.zeros((n, 1), np.int32), p[toks, slots][:, None], 1, 32)
    if w.prec == "bf16":
        # the BF16 path: the grouped definition on the bf16 values, no quantization
        y, saved = mlp.fwd_grouped(xs, wgu0[None], wd0[None], lay, keep=True)
        flops = 6.0 * n * w.H * fs
        if w.backward:
            mlp.bwd_grouped(dys, wgu0[None], wd0[None], lay, saved)
            flops += 12.0 * n * w.H * fs
        dt = time.perf_counter() - t0
        tok = n / w.k * fs / w.F
        out = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
               "sample": (f"expert 0 of the {w.name} workload: its first {n} routed assignments, full H={w.H}, "
                          f"ffn columns 0..{fs - 1} of F={w.F}; whole BF16 "
                          f"{'training step (fwd+bwd)' if w.backward else 'forward'}; fp64 numpy, {dt:.2f} s wall"),
               "seconds": round(dt, 3), "tokens_per_s": round(tok / dt, 4), "extrapolated": True,
               "extrapolated_step_seconds": round((w.flops_fwd() + (w.flops_bwd() if w.backward else 0.0)) / (flops / dt), 2)}
        if w.T * w.H * w.F <= 1 << 24:
            # small workloads: the per-token tier too, the whole forward token by token
            x_all, l_all = synth.x(w), synth.logits(w)
            i_all, p_all = rt.route(l_all, w.k)
            t1 = time.perf_counter()
            mlp.fwd_per_token(x_all, synth.w_gate_up(w), synth.w_down(w), i_all, p_all)
            out["per_token_forward_seconds"] = round(time.perf_counter() - t1, 4)
        return out
    wq = mx.quantize_rows(wgu0)
    dq = mx.quantize_rows(wd0)
    X = lay.gather(xs)
    xq, xsc = mx.quantize_rows(X)
    G, U, h = mlp.mx_gateup_stage(xq, xsc, [wq[0]], [wq[1]], lay)
    hq, hs = mx.quantize_rows(h)
    Y = mlp.mx_down_stage(hq, hs, [dq[0]], [dq[1]], lay)
    lay.combine(Y)
    flops = 6.0 * n * w.H * fs
    if w.backward:
        wqc = mx.quantize_cols(wgu0)
        dqc = mx.quantize_cols(wd0)
        xc = mx.quantize_cols(X)
        hc = mx.quantize_cols(h)
        DY = lay.gather(dys)
        dyq, dysc = mx.quantize_rows(DY)
        dyc = mx.quantize_cols(DY)
        dG, dU, dp = mlp.mx_dh_stage(dyq, dysc, [dqc[0]], [dqc[1]], G, U, lay)
        dGU = np.concatenate([dG, dU], axis=1)
        gq, gs = mx.quantize_rows(dGU)
        gc = mx.quantize_cols(dGU)
        mlp.mx_dw_stage(dyc[0], dyc[1], hc[0], hc[1], lay)
        dX = mlp.mx_dx_stage(gq, gs, [wqc[0]], [wqc[1]], lay)
        mlp.mx_dw_stage(gc[0], gc[1], xc[0], xc[1], lay)
        lay.combine(dX)
        flops += 12.0 * n * w.H * fs
    dt = time.perf_counter() - t0
    # token-equivalents: assignments / k, scaled by the fraction of the ffn width done
    tok = n / w.k * fs / w.F
    rate = flops / dt
    whole = w.flops_fwd() + (w.flops_bwd() if w.backward else 0.0)
    group = "its whole group of" if max_rows is None else "its first"
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": (f"expert 0 of the {w.name} workload: {group} {n} routed assignments, full H={w.H}, "
                       f"ffn columns 0..{fs - 1} of F={w.F}; whole MXFP8 "
                       f"{'training step (fwd+bwd)' if w.backward else 'forward'} incl. that weight slice's "
                       f"quantization; fp64 numpy, {dt:.1f} s wall; the work per assignment and per ffn column "
                       f"is uniform, so the whole step extrapolates linearly (extrapolated_step_seconds)"),
            "seconds": round(dt, 2), "tokens_per_s": round(tok / dt, 4),
            "extrapolated": True, "extrapolated_step_seconds": round(whole / rate, 1)}


# ------------------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="train_mxfp8", choices=sorted(WORKLOADS))
    ap.add_argument("--variant", default="grouped", choices=VARIANTS,
                    help="grouped projections (default) or the per-expert launch loop (forward workloads)")
    ap.add_argument("--dw-dtype", default="f32", choices=("f32", "bf16"),
                    help="weight-gradient output of the training step (default fp32)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured in a HIP graph (the per-kernel breakdown still comes "
                         "from an eager profiled pass; the eager time is reported beside it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=None,
                    help="assignments in the CPU oracle sample (default: expert 0's whole group for MXFP8, 4096 for BF16)")
    ap.add_argument("--cpu-fcols", type=int, default=None,
                    help="ffn columns in the CPU oracle sample (default: F/2 for MXFP8, all for BF16)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only the 1 GiB copy the traffic counters are calibrated on")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="write profiles/traffic.json from rocprofv3 counter_collection.csv files (no GPU)")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.workload)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import moe_grouped_expert_amd as m
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    m.lib()   # raises when the HIP library is not built: there is no other path
    dev = torch.device("cuda:0")
    wid, train = WORKLOADS[args.workload]
    w = synth.WORKLOADS[wid]
    if args.variant == "fp8_tensor" and (wid not in (2, 3, 4)):
        print("the fp8_tensor variant runs the MXFP8 workloads (fwd_mxfp8, fwd_mxfp8_skew, train_mxfp8)",
              file=sys.stderr)
        sys.exit(2)
    if args.variant in ("expert_loop", "unfused") and train:
        print(f"the {args.variant} variant runs forward workloads only", file=sys.stderr)
        sys.exit(2)
    log(f"[bench] workload {w.name}: T={w.T} E={w.E} H={w.H} F={w.F} k={w.k} prec={w.prec} train={train} "
        f"ep={w.ep} variant={args.variant}")
    wg = w   # the workload as named; w becomes the problem this GPU runs
    if w.ep > 1:
        inp, w = make_ep_share_inputs(m, w, dev)
        log(f"[bench] rank 0 of {wg.ep}: experts 0..{w.E - 1}, {w.T} received rows")
    else:
        inp = make_inputs(w, dev)
    torch.cuda.synchronize()
    step = Step(m, w, inp, train, args.variant, args.dw_dtype)
    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")
    R = step.g.R
    sizes = step.g.split_sizes.cpu().tolist()

    stream = torch.cuda.current_stream(dev)
    graph = None
    if args.graph:
        # the step only launches kernels on the current stream (no allocation, memset, copy
        # or host synchronization inside the library's calls), so it can be captured whole;
        # a warm-up on a side stream (default priority) first, as torch's capture expects
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        log("[bench] step captured in a HIP graph")

    def timed_pass(profile, replay=False):
        """K steps bracketed by synchronizations; one event before, after and between
        consecutive steps (no extra synchronization).  With profile, the library also
        records an event pair around every kernel launch (per-kernel times); with replay,
        each step is a replay of the captured graph."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        if profile:
            m.profile_start()
        ev[0].record(stream)
        for i in range(args.steps):
            if replay:
                graph.replay()
            else:
                step()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        recs = m.profile_stop() if profile else None
        return ev[0].elapsed_time(ev[-1]) / args.steps, sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)), recs

    # the headline: a pass with no per-kernel events (graph replays with --graph); then a
    # profiled eager pass of the same steps for the per-kernel breakdown and the roofline
    # of the dominant kernel
    ms, per_step, _ = timed_pass(False, replay=graph is not None)
    log(f"[bench] {args.steps} timed steps{' (graph replays)' if graph is not None else ''}: {ms:.3f} ms/step")
    ms_eager = timed_pass(False)[0] if graph is not None else None
    ms_prof, _, records = timed_pass(True)
    log(f"[bench] {args.steps} profiled steps (an event pair per kernel): {ms_prof:.3f} ms/step")

    flops = w.flops_fwd() + (w.flops_bwd() if train else 0.0)
    tflops = flops / (ms * 1e-3) / 1e12
    tok_s = w.T / (ms * 1e-3)
    kernels, kern_ms = summarize_kernels(records, args.steps, w, R, w.prec)
    dom = next(iter(kernels))
    dk = kernels[dom]
    wk = kernel_work(dom, w, R, dk["launches_per_step"])
    if wk and wk[0] == "flop":
        ach = wk[1] / (dk["avg_ms"] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_TFLOPS[w.prec],
                "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS[w.prec], 4),
                "traffic": traffic_for(dom, args.workload) if args.variant == "grouped" else None, "avg_launch_ms": dk["avg_ms"],
                "algorithmic_flop_per_launch": wk[1]}
    else:
        nb = wk[1] if wk else None
        ach = nb / (dk["avg_ms"] * 1e-3) / 1e9 if nb else None
        roof = {"kernel": dom, "bound": "hbm", "achieved": ach and round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": ach and round(ach / PEAK_HBM_GBS, 4),
                "traffic": traffic_for(dom, args.workload) if args.variant == "grouped" else None, "avg_launch_ms": dk["avg_ms"]}
    gemm_ms = sum(v["avg_ms"] * v["launches_per_step"] for k, v in kernels.items() if k.startswith("gemm_"))
    # the grouped-MLP calls alone (grouped_mlp_fwd, _unfused, grouped_mlp_bwd): every launch but the routing,
    # the x permute, the weight quantization, the combines and the router backward
    # (the one-scale-per-tensor amax passes count with the quantization, outside)
    outside = ("route_", "router_bwd", "combine", "quant_mx", "permute_", "tensor_", "seg_map")
    mlp_ms = sum(v["avg_ms"] * v["launches_per_step"] for k, v in kernels.items() if not k.startswith(outside))
    if train:   # the dy permute-quantize belongs to grouped_mlp_bwd: one of the step's two permute launches
        mlp_ms += sum(v["avg_ms"] * v["launches_per_step"] for k, v in kernels.items() if k.startswith("permute_")) / 2
    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8" if args.variant == "fp8_tensor" else w.prec,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "E": w.E, "H": w.H, "F": w.F, "k": w.k, "prec": w.prec,
                   "passes": "fwd+bwd" if train else "fwd", "align": 32, "split_sizes": sizes,
                   "parallelism": "single GPU", "variant": args.variant,
                   **({"graph": True} if graph is not None else {}),
                   **({"dw_dtype": args.dw_dtype} if train else {})},
        "tokens_per_s": round(tok_s, 1),
        "algorithmic_tflop_per_step": round(flops / 1e12, 4),
        "gemm_only": {"ms_per_step": round(gemm_ms, 4),
                      "tflops": round(flops / (gemm_ms * 1e-3) / 1e12, 1) if gemm_ms > 0 else None},
        "grouped_mlp_calls": {"ms_per_step": round(mlp_ms, 4),
                              "tflops": round(flops / (mlp_ms * 1e-3) / 1e12, 1) if mlp_ms > 0 else None},
        "kernel_ms_per_step": round(kern_ms, 4),
        **({"eager_ms_per_step": round(ms_eager, 4)} if ms_eager is not None else {}),
        "profiled_ms_per_step": round(ms_prof, 4),
        "step_ms": {"median": round(per_step[len(per_step) // 2], 4), "min": round(per_step[0], 4),
                    "max": round(per_step[-1], 4)},
        "device": {"name": torch.cuda.get_device_name(dev),
                   "compute_units": torch.cuda.get_device_properties(dev).multi_processor_count},
        "roofline": roof,
        "kernels": kernels,
    }
    if wg.ep > 1:
        out["config"].update(ep_rank_share={"ep": wg.ep, "tokens_per_rank": wg.T, "experts": wg.E,
                                            "top_k": wg.k, "local_experts": w.E, "rows_received": w.T})
        out["rows_per_s"] = out.pop("tokens_per_s")   # received rows (assignments), k = 1 locally
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        # MXFP8: expert 0's whole group over half of the ffn columns (about 12 s of fp64 numpy
        # on 16 host cores; the weight-slice quantization and the GEMMs both scale with the
        # columns, so the mix of the two is that of the whole step); an expert holding more
        # than 4096 rows on average (the one-expert workload) is sampled by its first 2048
        big_group = wg.T * wg.k > 4096 * wg.E
        rows = args.cpu_rows if args.cpu_rows is not None else (4096 if wg.prec == "bf16" else (2048 if big_group else None))
        fcols = args.cpu_fcols if args.cpu_fcols is not None else (None if wg.prec == "bf16" else max(32, wg.F // 2))
        out["cpu_baseline"] = cpu_baseline(wg, rows, fcols)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
