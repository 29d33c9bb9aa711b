"""ctypes binding of libmge.so (include/mge.h), with the same call names.

Argument marshalling only: tensors are allocated with torch (device memory and the
current stream are torch's), every step of the computation runs in the library's HIP
kernels.  If the library is not built the first call raises — there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmge.so")

MGE_OK, MGE_ERR_INVALID_ARG, MGE_ERR_UNSUPPORTED, MGE_ERR_WORKSPACE, MGE_ERR_HIP, MGE_ERR_DEVICE_CHECK = range(6)
PREC = {"bf16": 0, "mxfp8": 1}
DTYPE = {"bf16": 0, "f32": 1}
ORIENT_ROW, ORIENT_COL = 1, 2
ROUTE_WANT_COL, ROUTE_PROB_GIVEN = 1, 2

vp = C.c_void_p
i32 = C.c_int32
u32 = C.c_uint32
i64 = C.c_int64


class RouteArgs(C.Structure):
    _fields_ = [("struct_size", u32), ("T", i32), ("E", i32), ("k", i32), ("H", i32), ("align", i32),
                ("prec", i32), ("flags", u32),
                ("logits", vp), ("x", vp), ("topk_idx", vp), ("topk_prob", vp), ("split_sizes", vp),
                ("group_offsets", vp), ("perm_src", vp), ("perm_pos", vp), ("prob_perm", vp),
                ("x_perm", vp), ("x_perm_scale", vp), ("x_col", vp), ("x_col_scale", vp),
                ("workspace", vp), ("workspace_bytes", C.c_size_t), ("x_tensor_scale", vp)]


class QuantArgs(C.Structure):
    _fields_ = [("struct_size", u32), ("batch", i32), ("R", i32), ("C", i32),
                ("in_batch_stride", i64), ("in_row_stride", i64), ("in_", vp), ("orient", u32),
                ("row_codes", vp), ("row_scales", vp), ("col_codes", vp), ("col_scales", vp), ("tensor_scale", vp),
                ("seg_offsets", vp), ("num_segments", i32), ("workspace", vp), ("workspace_bytes", C.c_size_t)]


class TensorScaleArgs(C.Structure):
    _fields_ = [("struct_size", u32), ("batch", i32), ("n", i64), ("batch_stride", i64), ("in_", vp),
                ("scale", vp), ("workspace", vp), ("workspace_bytes", C.c_size_t)]


class FwdArgs(C.Structure):
    _fields_ = [("struct_size", u32), ("prec", i32), ("E", i32), ("H", i32), ("F", i32), ("T", i32),
                ("k", i32), ("align", i32),
                ("split_sizes", vp), ("group_offsets", vp), ("prob_perm", vp), ("x_perm", vp),
                ("x_perm_scale", vp), ("w_gate_up", vp), ("w_gate_up_scale", vp), ("w_down", vp),
                ("w_down_scale", vp), ("y_dtype", i32), ("y_perm", vp), ("h", vp), ("h_scale", vp),
                ("saved_gu", vp), ("h_col", vp), ("h_col_scale", vp), ("workspace", vp),
                ("workspace_bytes", C.c_size_t)]


class FwdUnfusedArgs(C.Structure):
    _fields_ = [("struct_size", u32), ("fwd", FwdArgs), ("gu", vp), ("h_bf16", vp), ("h_tensor_scale", vp)]


class BwdArgs(C.Structure):
    _fields_ = [("struct_size", u32), ("prec", i32), ("E", i32), ("H", i32), ("F", i32), ("T", i32),
                ("k", i32), ("align", i32),
                ("dy", vp), ("split_sizes", vp), ("group_offsets", vp), ("perm_src", vp), ("perm_pos", vp),
                ("prob_perm", vp), ("saved_gu", vp), ("h_col", vp), ("h_col_scale", vp), ("x_col", vp),
                ("x_col_scale", vp), ("w_gate_up", vp), ("w_gate_up_scale", vp), ("w_down", vp),
                ("w_down_scale", vp), ("dx_perm", vp), ("dw_gate_up", vp), ("dw_down", vp), ("d_prob", vp),
                ("accumulate", i32),
                ("dy_row", vp), ("dy_row_scale", vp), ("dy_col", vp), ("dy_col_scale", vp),
                ("dgu_row", vp), ("dgu_row_scale", vp), ("dgu_col", vp), ("dgu_col_scale", vp),
                ("workspace", vp), ("workspace_bytes", C.c_size_t), ("dw_bf16", i32),
                ("dy_tensor_scale", vp), ("dgu_tensor_scale", vp), ("dgu_bf16", vp)]


class FwdSavedSizes(C.Structure):
    _fields_ = [("struct_size", u32), ("rows", i64), ("saved_gu", C.c_size_t), ("h_col", C.c_size_t),
                ("h_col_scale", C.c_size_t), ("total", C.c_size_t)]


class CombineArgs(C.Structure):
    _fields_ = [("struct_size", u32), ("T", i32), ("k", i32), ("H", i32), ("in_dtype", i32), ("out_dtype", i32),
                ("in_", vp), ("perm_pos", vp), ("weights", vp), ("out", vp), ("in_rows", i64)]


class RouterBwdArgs(C.Structure):
    _fields_ = [("struct_size", u32), ("T", i32), ("E", i32), ("k", i32), ("topk_idx", vp), ("topk_prob", vp),
                ("d_prob", vp), ("d_logits", vp)]


_LIB = None
EXPORTS = ["mge_perm_rows", "mge_route_workspace_bytes", "moe_route_permute", "moe_route_permute_noalloc",
           "mxfp8_quantize",
           "mge_fwd_workspace_bytes", "grouped_mlp_fwd", "mge_fwd_saved_bytes", "mge_fwd_unfused_workspace_bytes", "grouped_mlp_fwd_unfused",
           "mge_tensor_scale_workspace_bytes", "mge_tensor_scale", "mge_quant_workspace_bytes",
           "mge_bwd_workspace_bytes", "grouped_mlp_bwd",
           "unpermute_combine", "moe_router_bwd", "mge_status_string", "mge_last_error", "mge_check_device_errors", "mge_version",
           "mge_profile_start", "mge_profile_stop"]


class KernelTime(C.Structure):
    _fields_ = [("name", C.c_char * 56), ("ms", C.c_float)]


def lib():
    """Loads libmge.so (raises if it is not built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m moe_grouped_expert_amd.build`")
        L = C.CDLL(LIB_PATH)
        L.mge_perm_rows.restype = i64
        L.mge_perm_rows.argtypes = [i32, i32, i32, i32]
        L.mge_route_workspace_bytes.restype = C.c_size_t
        L.mge_route_workspace_bytes.argtypes = [i32, i32]
        L.mge_fwd_workspace_bytes.restype = C.c_size_t
        L.mge_fwd_workspace_bytes.argtypes = [C.POINTER(FwdArgs)]
        L.mge_fwd_saved_bytes.restype = C.c_int
        L.mge_fwd_saved_bytes.argtypes = [i32, i32, i32, i32, i32, i32, C.POINTER(FwdSavedSizes)]
        L.mge_fwd_unfused_workspace_bytes.restype = C.c_size_t
        L.mge_fwd_unfused_workspace_bytes.argtypes = [C.POINTER(FwdUnfusedArgs)]
        L.mge_quant_workspace_bytes.restype = C.c_size_t
        L.mge_quant_workspace_bytes.argtypes = [C.POINTER(QuantArgs)]
        L.mge_tensor_scale_workspace_bytes.restype = C.c_size_t
        L.mge_tensor_scale_workspace_bytes.argtypes = [i32, i64]
        L.mge_bwd_workspace_bytes.restype = C.c_size_t
        L.mge_bwd_workspace_bytes.argtypes = [C.POINTER(BwdArgs)]
        for name, st in (("moe_route_permute", RouteArgs), ("moe_route_permute_noalloc", RouteArgs),
                         ("mxfp8_quantize", QuantArgs),
                         ("mge_tensor_scale", TensorScaleArgs),
                         ("grouped_mlp_fwd", FwdArgs), ("grouped_mlp_fwd_unfused", FwdUnfusedArgs),
                         ("grouped_mlp_bwd", BwdArgs),
                         ("unpermute_combine", CombineArgs), ("moe_router_bwd", RouterBwdArgs)):
            f = getattr(L, name)
            f.restype = C.c_int
            f.argtypes = [C.POINTER(st), vp]
        L.mge_status_string.restype = C.c_char_p
        L.mge_status_string.argtypes = [C.c_int]
        L.mge_last_error.restype = C.c_char_p
        L.mge_last_error.argtypes = []
        L.mge_check_device_errors.restype = C.c_int
        L.mge_check_device_errors.argtypes = [vp, vp]
        L.mge_version.restype = C.c_char_p
        L.mge_profile_start.restype = C.c_int
        L.mge_profile_start.argtypes = []
        L.mge_profile_stop.restype = i32
        L.mge_profile_stop.argtypes = [C.c_void_p, i32]
        _LIB = L
    return _LIB


class MgeError(RuntimeError):
    def __init__(self, code: int, where: str):
        L = lib()
        super().__init__(f"{where}: {L.mge_status_string(code).decode()}: {L.mge_last_error().decode()}")
        self.code = code


def _check(code: int, where: str):
    if code != MGE_OK:
        raise MgeError(code, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr_array(ts: Sequence[torch.Tensor]):
    arr = (vp * len(ts))(*[t.data_ptr() for t in ts])
    return arr


def perm_rows(T: int, k: int, E: int, align: int) -> int:
    """Rows of the permuted buffers for T tokens, top-k over E experts, groups starting at
    multiples of `align`: T*k plus the worst-case padding, E*(align-1)."""
    return int(lib().mge_perm_rows(T, k, E, align))


# ------------------------------------------------------------------------------ routing

@dataclass
class RouteOut:
    T: int
    E: int
    k: int
    H: int
    align: int
    prec: str
    R: int
    topk_idx: torch.Tensor
    topk_prob: torch.Tensor
    split_sizes: torch.Tensor
    group_offsets: torch.Tensor
    perm_src: torch.Tensor
    perm_pos: torch.Tensor
    prob_perm: torch.Tensor
    x_perm: Optional[torch.Tensor] = None
    x_perm_scale: Optional[torch.Tensor] = None
    x_col: Optional[torch.Tensor] = None
    x_col_scale: Optional[torch.Tensor] = None
    workspace: Optional[torch.Tensor] = None


def moe_route_permute(logits: Optional[torch.Tensor], x: Optional[torch.Tensor], k: int, E: Optional[int] = None,
                      align: int = 32, prec: str = "bf16", want_col: bool = False,
                      topk_idx: Optional[torch.Tensor] = None, topk_prob: Optional[torch.Tensor] = None,
                      out: Optional[RouteOut] = None, x_tensor_scale: Optional[torch.Tensor] = None,
                      noalloc: bool = False) -> RouteOut:
    """Top-k routing + stable permutation by expert (+ gather / quantize of x; with
    x_tensor_scale, a uint8 [1] tensor from tensor_scale(x), every block of x takes that
    one scale).  noalloc: call moe_route_permute_noalloc, whose workspace is the library's
    fixed scratch (no workspace tensor is allocated or passed)."""
    given = topk_idx is not None
    ref = logits if logits is not None else topk_idx
    dev = ref.device
    if logits is not None:
        T, E = logits.shape
        assert logits.dtype == torch.float32 and logits.is_contiguous()
    else:
        T = topk_idx.shape[0]
        assert E is not None
    H = x.shape[1] if x is not None else 32
    if x is not None:
        assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.shape[0] == T
    R = perm_rows(T, k, E, align)
    if out is None:
        i = dict(device=dev, dtype=torch.int32)
        f = dict(device=dev, dtype=torch.float32)
        o = RouteOut(T=T, E=E, k=k, H=H, align=align, prec=prec, R=R,
                     topk_idx=topk_idx if given else torch.empty((T, k), **i),
                     topk_prob=topk_prob if given else torch.empty((T, k), **f),
                     split_sizes=torch.empty(E, **i), group_offsets=torch.empty(E + 1, **i),
                     perm_src=torch.empty(R, **i), perm_pos=torch.empty((T, k), **i), prob_perm=torch.empty(R, **f))
        if x is not None:
            if prec == "mxfp8":
                o.x_perm = torch.empty((R, H), device=dev, dtype=torch.uint8)
                o.x_perm_scale = torch.empty((R, H // 32), device=dev, dtype=torch.uint8)
                if want_col:
                    o.x_col = torch.empty((H, R), device=dev, dtype=torch.uint8)
                    o.x_col_scale = torch.empty((H, R // 32), device=dev, dtype=torch.uint8)
            else:
                o.x_perm = torch.empty((R, H), device=dev, dtype=torch.bfloat16)
                if want_col:
                    o.x_col = torch.empty((H, R), device=dev, dtype=torch.bfloat16)
        if not noalloc:
            nbytes = int(lib().mge_route_workspace_bytes(T, E))
            o.workspace = torch.empty(max(nbytes, 256), device=dev, dtype=torch.uint8)
    else:
        o = out
    a = RouteArgs()
    a.struct_size = C.sizeof(RouteArgs)
    a.T, a.E, a.k, a.H, a.align = T, E, k, H, align
    a.prec = PREC[prec]
    a.flags = (ROUTE_WANT_COL if want_col else 0) | (ROUTE_PROB_GIVEN if given else 0)
    a.logits = _ptr(logits)
    a.x = _ptr(x)
    a.topk_idx, a.topk_prob = _ptr(o.topk_idx), _ptr(o.topk_prob)
    a.split_sizes, a.group_offsets = _ptr(o.split_sizes), _ptr(o.group_offsets)
    a.perm_src, a.perm_pos, a.prob_perm = _ptr(o.perm_src), _ptr(o.perm_pos), _ptr(o.prob_perm)
    a.x_perm, a.x_perm_scale = _ptr(o.x_perm), _ptr(o.x_perm_scale)
    a.x_col, a.x_col_scale = _ptr(o.x_col), _ptr(o.x_col_scale)
    a.x_tensor_scale = _ptr(x_tensor_scale)
    if noalloc:
        a.workspace, a.workspace_bytes = None, 0
        _check(lib().moe_route_permute_noalloc(C.byref(a), _stream(dev)), "moe_route_permute_noalloc")
    else:
        a.workspace, a.workspace_bytes = _ptr(o.workspace), o.workspace.numel()
        _check(lib().moe_route_permute(C.byref(a), _stream(dev)), "moe_route_permute")
    return o


def check_device_errors(route: RouteOut) -> int:
    """Synchronise the stream and read the routing call's device flag (set when a given
    top-k index was out of range and clamped); returns the library status code.  For
    tests and debugging: it blocks the host."""
    return lib().mge_check_device_errors(_ptr(route.workspace), _stream(route.workspace.device))


# ------------------------------------------------------------------------------ quantize

def mxfp8_quantize(w: torch.Tensor, orient: str = "row", out=None, tensor_scale: Optional[torch.Tensor] = None,
                   seg_offsets: Optional[torch.Tensor] = None):
    """BF16 [..., R, C] -> (row_codes, row_scales, col_codes, col_scales) (absent ones None).
    tensor_scale: optional uint8 [batch] (one scale per matrix, from tensor_scale(w,
    per_matrix=True)) that every block of its matrix takes instead of its own.
    seg_offsets: optional int32 [S+1] on the device: segments along R, each placed at a
    multiple of 32 rows (zero-padded), in perm_rows(R, 1, S, 32) output rows, so that the
    column form's 32-row blocks restart at every segment."""
    assert w.dtype == torch.bfloat16 and w.is_contiguous()
    R, Cc = w.shape[-2], w.shape[-1]
    lead = tuple(w.shape[:-2])
    batch = 1
    for d in lead:
        batch *= d
    Rp = (R + 31) // 32 * 32
    nseg = 0
    if seg_offsets is not None:
        assert seg_offsets.dtype == torch.int32 and seg_offsets.is_contiguous() and seg_offsets.numel() >= 2
        nseg = seg_offsets.numel() - 1
        Rp = perm_rows(R, 1, nseg, 32)
    Rr = Rp if seg_offsets is not None else R   # rows of the row form
    want_row = orient in ("row", "both")
    want_col = orient in ("col", "both")
    dev = w.device
    if out is None:
        u8 = dict(device=dev, dtype=torch.uint8)
        rc = torch.empty(lead + (Rr, Cc), **u8) if want_row else None
        rs = torch.empty(lead + (Rr, Cc // 32), **u8) if want_row else None
        cc = torch.empty(lead + (Cc, Rp), **u8) if want_col else None
        cs = torch.empty(lead + (Cc, Rp // 32), **u8) if want_col else None
    else:
        rc, rs, cc, cs = out
    a = QuantArgs()
    a.struct_size = C.sizeof(QuantArgs)
    a.batch, a.R, a.C = batch, R, Cc
    a.in_batch_stride, a.in_row_stride = R * Cc, Cc
    a.in_ = _ptr(w)
    a.orient = (ORIENT_ROW if want_row else 0) | (ORIENT_COL if want_col else 0)
    a.row_codes, a.row_scales, a.col_codes, a.col_scales = _ptr(rc), _ptr(rs), _ptr(cc), _ptr(cs)
    if tensor_scale is not None:
        assert tensor_scale.dtype == torch.uint8 and tensor_scale.numel() == batch
    a.tensor_scale = _ptr(tensor_scale)
    ws = None
    if seg_offsets is not None:
        a.seg_offsets, a.num_segments = _ptr(seg_offsets), nseg
        ws = torch.empty(max(int(lib().mge_quant_workspace_bytes(C.byref(a))), 256), device=dev, dtype=torch.uint8)
        a.workspace, a.workspace_bytes = _ptr(ws), ws.numel()
    _check(lib().mxfp8_quantize(C.byref(a), _stream(dev)), "mxfp8_quantize")
    return rc, rs, cc, cs


@dataclass
class TensorScaleOut:
    scale: torch.Tensor        # uint8 [batch]
    workspace: torch.Tensor


def tensor_scale(t: torch.Tensor, per_matrix: bool = False, out: Optional[TensorScaleOut] = None) -> TensorScaleOut:
    """One E8M0 scale per tensor (FP8 with one scale per tensor): of all of t, or with
    per_matrix of each t[b] along the leading dimension."""
    assert t.dtype == torch.bfloat16 and t.is_contiguous()
    batch = t.shape[0] if per_matrix else 1
    n = t.numel() // max(batch, 1)
    dev = t.device
    if out is None:
        ws = int(lib().mge_tensor_scale_workspace_bytes(batch, n))
        out = TensorScaleOut(scale=torch.empty(batch, device=dev, dtype=torch.uint8),
                             workspace=torch.empty(max(ws, 256), device=dev, dtype=torch.uint8))
    a = TensorScaleArgs()
    a.struct_size = C.sizeof(TensorScaleArgs)
    a.batch, a.n, a.batch_stride = batch, n, n
    a.in_, a.scale = _ptr(t), _ptr(out.scale)
    a.workspace, a.workspace_bytes = _ptr(out.workspace), out.workspace.numel()
    _check(lib().mge_tensor_scale(C.byref(a), _stream(dev)), "mge_tensor_scale")
    return out


# ------------------------------------------------------------------------------ forward

def fwd_saved_bytes(prec: str, T: int, k: int, E: int, F: int, align: int = 32) -> FwdSavedSizes:
    """Byte sizes of the activations a training forward saves (mge_fwd_saved_bytes)."""
    o = FwdSavedSizes()
    o.struct_size = C.sizeof(FwdSavedSizes)
    _check(lib().mge_fwd_saved_bytes(PREC[prec], T, k, E, F, align, C.byref(o)), "mge_fwd_saved_bytes")
    return o


@dataclass
class FwdOut:
    y_perm: torch.Tensor
    h: torch.Tensor
    h_scale: Optional[torch.Tensor] = None
    saved_gu: Optional[torch.Tensor] = None
    h_col: Optional[torch.Tensor] = None
    h_col_scale: Optional[torch.Tensor] = None
    workspace: Optional[torch.Tensor] = None
    gu: Optional[torch.Tensor] = None          # unfused forward: [G U] bf16 (kept on request)
    h_bf16: Optional[torch.Tensor] = None      # unfused MXFP8 forward: h before its quantize
    h_tensor_scale: Optional[torch.Tensor] = None  # unfused, one scale for all of h: uint8 [1]


def _split(w, E):
    if isinstance(w, torch.Tensor):
        return [w[e] for e in range(E)]
    return list(w)


def _fwd_args(rt: RouteOut, w_gate_up, w_down, w_gate_up_scale, w_down_scale, y_dtype: str, train: bool,
              out: Optional[FwdOut]):
    """Outputs (allocated unless given) and the filled mge_fwd_args; `keep` holds the
    host pointer arrays alive while the call runs."""
    E, H, R = rt.E, rt.H, rt.R
    wg = _split(w_gate_up, E)
    wd = _split(w_down, E)
    F = wg[0].shape[0] // 2
    mx = rt.prec == "mxfp8"
    dev = rt.x_perm.device
    if out is None:
        o = FwdOut(y_perm=torch.empty((R, H), device=dev, dtype=torch.bfloat16 if y_dtype == "bf16" else torch.float32),
                   h=torch.empty((R, F), device=dev, dtype=torch.uint8 if mx else torch.bfloat16))
        if mx:
            o.h_scale = torch.empty((R, F // 32), device=dev, dtype=torch.uint8)
        if train:
            sz = fwd_saved_bytes(rt.prec, rt.T, rt.k, E, F, rt.align)
            assert sz.rows == R
            o.saved_gu = torch.empty(sz.saved_gu, device=dev, dtype=torch.uint8).view(torch.bfloat16).view(R, 2 * F)
            hdt = torch.uint8 if mx else torch.bfloat16
            o.h_col = torch.empty(sz.h_col, device=dev, dtype=torch.uint8).view(hdt).view(F, R)
            if mx:
                o.h_col_scale = torch.empty(sz.h_col_scale, device=dev, dtype=torch.uint8).view(F, R // 32)
    else:
        o = out
    a = FwdArgs()
    a.struct_size = C.sizeof(FwdArgs)
    a.prec, a.E, a.H, a.F, a.T, a.k, a.align = PREC[rt.prec], E, H, F, rt.T, rt.k, rt.align
    a.split_sizes, a.group_offsets, a.prob_perm = _ptr(rt.split_sizes), _ptr(rt.group_offsets), _ptr(rt.prob_perm)
    a.x_perm, a.x_perm_scale = _ptr(rt.x_perm), _ptr(rt.x_perm_scale)
    keep = [_ptr_array(wg), _ptr_array(wd)]
    a.w_gate_up, a.w_down = C.cast(keep[0], vp), C.cast(keep[1], vp)
    if mx:
        keep += [_ptr_array(_split(w_gate_up_scale, E)), _ptr_array(_split(w_down_scale, E))]
        a.w_gate_up_scale, a.w_down_scale = C.cast(keep[2], vp), C.cast(keep[3], vp)
    a.y_dtype = DTYPE[y_dtype]
    a.y_perm, a.h, a.h_scale = _ptr(o.y_perm), _ptr(o.h), _ptr(o.h_scale)
    a.saved_gu, a.h_col, a.h_col_scale = _ptr(o.saved_gu), _ptr(o.h_col), _ptr(o.h_col_scale)
    return o, a, keep, F, dev


def grouped_mlp_fwd(rt: RouteOut, w_gate_up, w_down, w_gate_up_scale=None, w_down_scale=None,
                    y_dtype: str = "bf16", train: bool = False, out: Optional[FwdOut] = None) -> FwdOut:
    """Grouped gate-up GEMM -> SwiGLU x prob (+ quantize) -> grouped down GEMM over every
    expert of `rt`, one launch per projection.
    w_gate_up: [E, 2F, H] (gate rows first), w_down: [E, H, F]; bf16 masters for a BF16
    route, MXFP8 row codes (with w_*_scale) for an MXFP8 one.  y_dtype "bf16" or "f32".
    train=True also keeps what the backward needs (G and U in bf16, h's column form)."""
    o, a, keep, F, dev = _fwd_args(rt, w_gate_up, w_down, w_gate_up_scale, w_down_scale, y_dtype, train, out)
    if o.workspace is None:
        o.workspace = torch.empty(max(int(lib().mge_fwd_workspace_bytes(C.byref(a))), 256), device=dev,
                                  dtype=torch.uint8)
    a.workspace, a.workspace_bytes = _ptr(o.workspace), o.workspace.numel()
    _check(lib().grouped_mlp_fwd(C.byref(a), _stream(dev)), "grouped_mlp_fwd")
    return o


def grouped_mlp_fwd_unfused(rt: RouteOut, w_gate_up, w_down, w_gate_up_scale=None, w_down_scale=None,
                            y_dtype: str = "bf16", keep_intermediates: bool = False, h_per_tensor: bool = False,
                            train: bool = False, out: Optional[FwdOut] = None) -> FwdOut:
    """The forward without the fusion: [G U] to HBM in bf16, a standalone SwiGLU x prob,
    (MXFP8) a standalone quantize of h, the grouped down GEMM.  With keep_intermediates,
    out.gu ([R][2F] bf16) and (MXFP8) out.h_bf16 ([R][F]) are kept; with h_per_tensor, h
    takes one scale for the whole tensor (out.h_tensor_scale).  train: [G U] is written to
    out.saved_gu (out.gu is the same tensor) and the column form of h to out.h_col."""
    o, a, keep, F, dev = _fwd_args(rt, w_gate_up, w_down, w_gate_up_scale, w_down_scale, y_dtype, train, out)
    u = FwdUnfusedArgs()
    u.struct_size = C.sizeof(FwdUnfusedArgs)
    if h_per_tensor and o.h_tensor_scale is None:
        o.h_tensor_scale = torch.empty(1, device=dev, dtype=torch.uint8)
    u.h_tensor_scale = _ptr(o.h_tensor_scale)
    if train:
        o.gu = o.saved_gu
    if keep_intermediates:
        if o.gu is None:
            o.gu = torch.empty((rt.R, 2 * F), device=dev, dtype=torch.bfloat16)
        if rt.prec == "mxfp8" and o.h_bf16 is None:
            o.h_bf16 = torch.empty((rt.R, F), device=dev, dtype=torch.bfloat16)
    u.gu, u.h_bf16 = _ptr(o.gu), _ptr(o.h_bf16)
    u.fwd = a
    if o.workspace is None:
        o.workspace = torch.empty(max(int(lib().mge_fwd_unfused_workspace_bytes(C.byref(u))), 256), device=dev,
                                  dtype=torch.uint8)
    u.fwd.workspace, u.fwd.workspace_bytes = _ptr(o.workspace), o.workspace.numel()
    _check(lib().grouped_mlp_fwd_unfused(C.byref(u), _stream(dev)), "grouped_mlp_fwd_unfused")
    return o


# ------------------------------------------------------------------------------ backward

@dataclass
class BwdOut:
    dx_perm: torch.Tensor
    dw_gate_up: list
    dw_down: list
    d_prob: torch.Tensor
    dy_row: Optional[torch.Tensor] = None
    dy_row_scale: Optional[torch.Tensor] = None
    dy_col: Optional[torch.Tensor] = None
    dy_col_scale: Optional[torch.Tensor] = None
    dgu_row: Optional[torch.Tensor] = None
    dgu_row_scale: Optional[torch.Tensor] = None
    dgu_col: Optional[torch.Tensor] = None
    dgu_col_scale: Optional[torch.Tensor] = None
    workspace: Optional[torch.Tensor] = None
    dy_tensor_scale: Optional[torch.Tensor] = None    # per-tensor mode: uint8 [1] each
    dgu_tensor_scale: Optional[torch.Tensor] = None
    dgu_bf16: Optional[torch.Tensor] = None           # per-tensor mode, kept on request: [R][2F] bf16


def grouped_mlp_bwd(dy: torch.Tensor, rt: RouteOut, fw: FwdOut, w_gate_up_k, w_down_k, w_gate_up_k_scale=None,
                    w_down_k_scale=None, accumulate: bool = False, keep_intermediates: bool = False,
                    out: Optional[BwdOut] = None, dw_dtype: str = "f32", per_tensor: bool = False) -> BwdOut:
    """Backward of the grouped MLP.  Weights: MXFP8 column forms, or the bf16 masters.
    dw_dtype: "f32" (default) or "bf16" (the fp32 sums rounded to nearest even; no accumulate).
    per_tensor (MXFP8): FP8 with one scale per tensor for dY and [dG dU] (out.dy_tensor_scale,
    out.dgu_tensor_scale; with keep_intermediates also the bf16 [dG dU] in out.dgu_bf16)."""
    if dw_dtype not in ("f32", "bf16"):
        raise ValueError(f"dw_dtype must be 'f32' or 'bf16', not {dw_dtype!r}")
    E, H, R, T, k = rt.E, rt.H, rt.R, rt.T, rt.k
    mx = rt.prec == "mxfp8"
    wg = _split(w_gate_up_k, E)
    wd = _split(w_down_k, E)
    F = fw.h.shape[1]
    dev = dy.device
    if out is None:
        f32 = dict(device=dev, dtype=torch.float32)
        dwt = dict(device=dev, dtype=torch.float32 if dw_dtype == "f32" else torch.bfloat16)
        o = BwdOut(dx_perm=torch.empty((R, H), device=dev, dtype=torch.bfloat16),
                   dw_gate_up=[torch.empty((2 * F, H), **dwt) for _ in range(E)],
                   dw_down=[torch.empty((H, F), **dwt) for _ in range(E)],
                   d_prob=torch.empty((T, k), **f32))
        if keep_intermediates:
            cd = torch.uint8 if mx else torch.bfloat16
            o.dy_row = torch.empty((R, H), device=dev, dtype=cd)
            o.dy_col = torch.empty((H, R), device=dev, dtype=cd)
            o.dgu_row = torch.empty((R, 2 * F), device=dev, dtype=cd)
            o.dgu_col = torch.empty((2 * F, R), device=dev, dtype=cd)
            if mx:
                u8 = dict(device=dev, dtype=torch.uint8)
                o.dy_row_scale = torch.empty((R, H // 32), **u8)
                o.dy_col_scale = torch.empty((H, R // 32), **u8)
                o.dgu_row_scale = torch.empty((R, 2 * F // 32), **u8)
                o.dgu_col_scale = torch.empty((2 * F, R // 32), **u8)
            if per_tensor:
                o.dgu_bf16 = torch.empty((R, 2 * F), device=dev, dtype=torch.bfloat16)
        if per_tensor:
            o.dy_tensor_scale = torch.empty(1, device=dev, dtype=torch.uint8)
            o.dgu_tensor_scale = torch.empty(1, device=dev, dtype=torch.uint8)
    else:
        o = out
    a = BwdArgs()
    a.struct_size = C.sizeof(BwdArgs)
    a.prec, a.E, a.H, a.F, a.T, a.k, a.align = PREC[rt.prec], E, H, F, T, k, rt.align
    a.dy = _ptr(dy)
    a.split_sizes, a.group_offsets = _ptr(rt.split_sizes), _ptr(rt.group_offsets)
    a.perm_src, a.perm_pos, a.prob_perm = _ptr(rt.perm_src), _ptr(rt.perm_pos), _ptr(rt.prob_perm)
    a.saved_gu = _ptr(fw.saved_gu)
    a.h_col, a.h_col_scale = _ptr(fw.h_col), _ptr(fw.h_col_scale)
    a.x_col, a.x_col_scale = _ptr(rt.x_col), _ptr(rt.x_col_scale)
    keep = [_ptr_array(wg), _ptr_array(wd), _ptr_array(o.dw_gate_up), _ptr_array(o.dw_down)]
    a.w_gate_up, a.w_down = C.cast(keep[0], vp), C.cast(keep[1], vp)
    a.dw_gate_up, a.dw_down = C.cast(keep[2], vp), C.cast(keep[3], vp)
    if mx:
        keep += [_ptr_array(_split(w_gate_up_k_scale, E)), _ptr_array(_split(w_down_k_scale, E))]
        a.w_gate_up_scale, a.w_down_scale = C.cast(keep[4], vp), C.cast(keep[5], vp)
    a.dx_perm, a.d_prob = _ptr(o.dx_perm), _ptr(o.d_prob)
    a.accumulate = 1 if accumulate else 0
    a.dw_bf16 = 1 if dw_dtype == "bf16" else 0
    a.dy_row, a.dy_row_scale, a.dy_col, a.dy_col_scale = _ptr(o.dy_row), _ptr(o.dy_row_scale), _ptr(o.dy_col), _ptr(o.dy_col_scale)
    a.dgu_row, a.dgu_row_scale = _ptr(o.dgu_row), _ptr(o.dgu_row_scale)
    a.dgu_col, a.dgu_col_scale = _ptr(o.dgu_col), _ptr(o.dgu_col_scale)
    a.dy_tensor_scale, a.dgu_tensor_scale, a.dgu_bf16 = _ptr(o.dy_tensor_scale), _ptr(o.dgu_tensor_scale), _ptr(o.dgu_bf16)
    if o.workspace is None:
        o.workspace = torch.empty(max(int(lib().mge_bwd_workspace_bytes(C.byref(a))), 256), device=dev,
                                  dtype=torch.uint8)
    a.workspace, a.workspace_bytes = _ptr(o.workspace), o.workspace.numel()
    _check(lib().grouped_mlp_bwd(C.byref(a), _stream(dev)), "grouped_mlp_bwd")
    return o


# ------------------------------------------------------------------------------ timing

def profile_start() -> None:
    """Start recording a HIP event pair around every kernel the library launches."""
    _check(lib().mge_profile_start(), "mge_profile_start")


def profile_stop() -> list:
    """Stop recording; returns [(kernel name, milliseconds)] in launch order."""
    L = lib()
    n = int(L.mge_profile_stop(None, 0))
    buf = (KernelTime * max(n, 1))()
    # records are kept until the next start, so a second read returns the same list
    L.mge_profile_stop(C.cast(buf, C.c_void_p), n)
    return [(buf[i].name.decode(), float(buf[i].ms)) for i in range(n)]


# ------------------------------------------------------------------------------ combine

def unpermute_combine(inp: torch.Tensor, perm_pos: torch.Tensor, weights: Optional[torch.Tensor] = None,
                      out_dtype: str = "bf16", out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[t] = sum over i of weights[t, i] * inp[perm_pos[t, i]] (unweighted when weights
    is None), in slot order and fp32, without atomics; a slot whose entry is outside
    [0, rows of inp), such as -1, adds nothing.  inp: [rows, H] bf16 or f32 (y_perm or
    dx_perm); out_dtype "bf16" or "f32"."""
    T, k = perm_pos.shape
    H = inp.shape[1]
    dev = inp.device
    if out is None:
        out = torch.empty((T, H), device=dev, dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32)
    a = CombineArgs()
    a.struct_size = C.sizeof(CombineArgs)
    a.T, a.k, a.H = T, k, H
    a.in_dtype = DTYPE["bf16"] if inp.dtype == torch.bfloat16 else DTYPE["f32"]
    a.out_dtype = DTYPE["bf16"] if out.dtype == torch.bfloat16 else DTYPE["f32"]
    a.in_, a.perm_pos, a.weights, a.out = _ptr(inp), _ptr(perm_pos), _ptr(weights), _ptr(out)
    a.in_rows = inp.shape[0]
    _check(lib().unpermute_combine(C.byref(a), _stream(dev)), "unpermute_combine")
    return out


# ------------------------------------------------------------------------------ router backward

def moe_router_bwd(topk_idx: torch.Tensor, topk_prob: torch.Tensor, d_prob: torch.Tensor, E: int,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """d_logits fp32 [T][E] from the slots' indices, probabilities and d_prob ([T][k] each)."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    if out is None:
        out = torch.empty((T, E), device=dev, dtype=torch.float32)
    a = RouterBwdArgs()
    a.struct_size = C.sizeof(RouterBwdArgs)
    a.T, a.E, a.k = T, E, k
    a.topk_idx, a.topk_prob, a.d_prob, a.d_logits = _ptr(topk_idx), _ptr(topk_prob), _ptr(d_prob), _ptr(out)
    _check(lib().moe_router_bwd(C.byref(a), _stream(dev)), "moe_router_bwd")
    return out
