"""C-ABI contract tests that need no GPU: the library loads, exports every function
include/mge.h declares, the Python structs match the C layout (a size mismatch is
rejected before anything else), and bad arguments are rejected on the host with the
documented codes before any launch."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mge.h")

from moe_grouped_expert_amd import _binding as b  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(b.LIB_PATH), reason="libmge.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol():
    L = b.lib()
    names = declared_functions()
    assert len(names) >= 13, names
    for n in names:
        assert hasattr(L, n), n
    assert set(b.EXPORTS) <= set(names)


def test_version_and_status_strings():
    L = b.lib()
    assert L.mge_version().decode().count(".") == 2
    for code in range(6):
        assert L.mge_status_string(code).decode().startswith("MGE_")


def test_perm_rows():
    # T*k + E*(align-1), rounded up to 32
    assert b.perm_rows(256, 2, 4, 32) == 640
    assert b.perm_rows(16384, 2, 8, 32) == 32768 + 256
    assert b.perm_rows(3, 1, 1, 1) == 32
    assert b.perm_rows(0, 2, 8, 32) == 256


def _call(fn, st, **fields):
    a = st()
    a.struct_size = C.sizeof(st)
    for k, v in fields.items():
        setattr(a, k, v)
    L = b.lib()
    r = getattr(L, fn)(C.byref(a), None)
    return r, L.mge_last_error().decode()


def test_struct_size_checked():
    a = b.RouteArgs()
    a.struct_size = C.sizeof(b.RouteArgs) - 4
    L = b.lib()
    assert L.moe_route_permute(C.byref(a), None) == b.MGE_ERR_INVALID_ARG
    assert "struct_size" in L.mge_last_error().decode()
    assert L.moe_route_permute(None, None) == b.MGE_ERR_INVALID_ARG
    # a struct that ends before the added last field (x_tensor_scale, tensor_scale) is
    # accepted and goes on to the next check
    for fn, st, size in (("moe_route_permute", b.RouteArgs, b.RouteArgs.x_tensor_scale.offset),
                         ("mxfp8_quantize", b.QuantArgs, b.QuantArgs.tensor_scale.offset),
                         ("mxfp8_quantize", b.QuantArgs, b.QuantArgs.seg_offsets.offset)):
        a = st()
        a.struct_size = size
        if st is b.QuantArgs:
            a.C = 33
        assert getattr(L, fn)(C.byref(a), None) == b.MGE_ERR_INVALID_ARG
        assert "struct_size" not in L.mge_last_error().decode()
    a = b.QuantArgs()
    a.struct_size = C.sizeof(b.QuantArgs) - 8
    assert L.mxfp8_quantize(C.byref(a), None) == b.MGE_ERR_INVALID_ARG
    assert "struct_size" in L.mge_last_error().decode()


def test_quantize_segments_rejects_and_workspace():
    L = b.lib()
    base = dict(batch=1, R=100, C=64, in_row_stride=64, in_=1 << 20, orient=b.ORIENT_COL, col_codes=1 << 21,
                col_scales=1 << 22, seg_offsets=1 << 23)
    r, err = _call("mxfp8_quantize", b.QuantArgs, num_segments=0, **base)
    assert r == b.MGE_ERR_INVALID_ARG and "num_segments" in err
    r, err = _call("mxfp8_quantize", b.QuantArgs, num_segments=1025, **base)
    assert r == b.MGE_ERR_INVALID_ARG and "num_segments" in err
    r, err = _call("mxfp8_quantize", b.QuantArgs, num_segments=5, **base)
    assert r == b.MGE_ERR_WORKSPACE
    a = b.QuantArgs()
    a.struct_size = C.sizeof(b.QuantArgs)
    for k, v in dict(num_segments=5, **base).items():
        setattr(a, k, v)
    # the padded rows: R + 31 per segment, rounded up to 32; one int32 row map entry each
    assert b.perm_rows(100, 1, 5, 32) == 256
    assert L.mge_quant_workspace_bytes(C.byref(a)) == 256 * 4
    a.seg_offsets = None
    assert L.mge_quant_workspace_bytes(C.byref(a)) == 0


def test_tensor_scale_rejects_and_workspace():
    L = b.lib()
    assert L.mge_tensor_scale_workspace_bytes(1, 8 * 256 * 3000) == 1024 * 4
    assert L.mge_tensor_scale_workspace_bytes(3, 100) == 256
    r, err = _call("mge_tensor_scale", b.TensorScaleArgs, batch=70000, n=64)
    assert r == b.MGE_ERR_INVALID_ARG and "batch" in err
    r, err = _call("mge_tensor_scale", b.TensorScaleArgs, batch=2, n=64, batch_stride=32)
    assert r == b.MGE_ERR_INVALID_ARG and "batch_stride" in err
    r, err = _call("mge_tensor_scale", b.TensorScaleArgs, batch=1, n=64)
    assert r == b.MGE_ERR_INVALID_ARG and "NULL" in err
    r, err = _call("mge_tensor_scale", b.TensorScaleArgs, batch=1, n=64, in_=1 << 20, scale=1 << 21)
    assert r == b.MGE_ERR_WORKSPACE
    r, err = _call("mge_tensor_scale", b.TensorScaleArgs, batch=0, n=64)
    assert r == b.MGE_OK
    # the per-tensor scale of x needs MXFP8
    r, err = _call("moe_route_permute", b.RouteArgs, T=8, E=4, k=2, H=64, align=32, prec=0, x_tensor_scale=1 << 20)
    assert r == b.MGE_ERR_INVALID_ARG and "x_tensor_scale" in err


@pytest.mark.parametrize("fields,msg", [
    (dict(T=-1, E=4, k=2, H=64, align=32), "T must"),
    (dict(T=8, E=0, k=1, H=64, align=32), "E must"),
    (dict(T=8, E=300, k=1, H=64, align=32), "E must"),
    (dict(T=8, E=4, k=5, H=64, align=32), "k must"),
    (dict(T=8, E=16, k=9, H=64, align=32), "k must"),
    (dict(T=8, E=4, k=2, H=48, align=32), "H must"),
    (dict(T=8, E=4, k=2, H=64, align=24), "align must"),
    (dict(T=8, E=4, k=2, H=64, align=32, prec=3), "prec"),
])
def test_route_rejects_bad_sizes(fields, msg):
    r, err = _call("moe_route_permute", b.RouteArgs, **fields)
    assert r == b.MGE_ERR_INVALID_ARG and msg in err, err


def test_route_rejects_null_outputs_and_small_workspace():
    base = dict(T=8, E=4, k=2, H=64, align=32, logits=64)
    r, err = _call("moe_route_permute", b.RouteArgs, **base)
    assert r == b.MGE_ERR_INVALID_ARG and "NULL" in err
    ptrs = {n: 256 * (i + 1) for i, n in enumerate(
        ["topk_idx", "topk_prob", "split_sizes", "group_offsets", "perm_src", "perm_pos", "prob_perm"])}
    r, err = _call("moe_route_permute", b.RouteArgs, **base, **ptrs, workspace=4096, workspace_bytes=16)
    assert r == b.MGE_ERR_WORKSPACE and "workspace" in err
    r, err = _call("moe_route_permute", b.RouteArgs, **base, **ptrs, x=4096 + 8, x_perm=8192)
    assert r == b.MGE_ERR_INVALID_ARG and "aligned" in err
    # MXFP8 column form needs align % 32 == 0
    r, err = _call("moe_route_permute", b.RouteArgs, **{**base, "align": 16}, **ptrs, prec=1, x=4096, x_perm=8192,
                   x_perm_scale=16384, flags=b.ROUTE_WANT_COL, x_col=32768, x_col_scale=65536)
    assert r == b.MGE_ERR_INVALID_ARG and "align" in err


def test_route_workspace_query():
    L = b.lib()
    assert L.mge_route_workspace_bytes(256, 4) >= 256 + 4 * 4
    assert L.mge_route_workspace_bytes(32768, 8) >= 128 * 8 * 4


def test_quantize_rejects():
    r, err = _call("mxfp8_quantize", b.QuantArgs, batch=1, R=64, C=48, orient=1, in_=4096, in_row_stride=48)
    assert r == b.MGE_ERR_INVALID_ARG and "multiple of 32" in err
    r, err = _call("mxfp8_quantize", b.QuantArgs, batch=1, R=64, C=64, orient=1, in_=4096, in_row_stride=64)
    assert r == b.MGE_ERR_INVALID_ARG and "row outputs" in err
    r, err = _call("mxfp8_quantize", b.QuantArgs, batch=1, R=64, C=64, orient=4, in_=4096, in_row_stride=64)
    assert r == b.MGE_ERR_INVALID_ARG and "orient" in err
    # empty input is a valid no-op
    r, err = _call("mxfp8_quantize", b.QuantArgs, batch=1, R=0, C=64, orient=1, in_=4096, in_row_stride=64,
                   row_codes=8192, row_scales=16384)
    assert r == b.MGE_OK, err


def test_fwd_bwd_combine_reject():
    r, err = _call("grouped_mlp_fwd", b.FwdArgs, prec=1, E=4, H=64, F=100, T=8, k=2, align=32)
    assert r == b.MGE_ERR_INVALID_ARG and "F must" in err
    r, err = _call("grouped_mlp_fwd", b.FwdArgs, prec=1, E=4, H=64, F=128, T=8, k=2, align=32)
    assert r == b.MGE_ERR_INVALID_ARG and "NULL" in err
    r, err = _call("grouped_mlp_bwd", b.BwdArgs, prec=0, E=4, H=64, F=128, T=8, k=2, align=8)
    assert r == b.MGE_ERR_INVALID_ARG and "align" in err
    r, err = _call("unpermute_combine", b.CombineArgs, T=4, k=9, H=64)
    assert r == b.MGE_ERR_INVALID_ARG
    r, err = _call("unpermute_combine", b.CombineArgs, T=4, k=2, H=64, in_dtype=2)
    assert r == b.MGE_ERR_INVALID_ARG and "dtype" in err
    # host buffers stand in for device ones: the call fails before any launch
    buf = (C.c_uint8 * 4096)()
    addr = (C.addressof(buf) + 15) // 16 * 16
    r, err = _call("unpermute_combine", b.CombineArgs, T=4, k=2, H=64, in_=addr, out=addr, perm_pos=addr, in_rows=-1)
    assert r == b.MGE_ERR_INVALID_ARG and "in_rows" in err


def test_check_device_errors_rejects_null():
    L = b.lib()
    assert L.mge_check_device_errors(None, None) == b.MGE_ERR_INVALID_ARG


@pytest.mark.parametrize("fields,msg", [
    (dict(T=-1, E=8, k=2), "T must"),
    (dict(T=4, E=0, k=1), "E must"),
    (dict(T=4, E=257, k=2), "E must"),
    (dict(T=4, E=4, k=5), "k must"),
    (dict(T=4, E=16, k=9), "k must"),
    (dict(T=4, E=8, k=2), "NULL"),
])
def test_router_bwd_rejects(fields, msg):
    r, err = _call("moe_router_bwd", b.RouterBwdArgs, **fields)
    assert r == b.MGE_ERR_INVALID_ARG and msg in err, err


def test_router_bwd_empty_and_struct_size():
    # T = 0 is a no-op even with NULL pointers; a wrong struct_size is rejected first
    r, err = _call("moe_router_bwd", b.RouterBwdArgs, T=0, E=8, k=2)
    assert r == b.MGE_OK, err
    a = b.RouterBwdArgs()
    a.struct_size = C.sizeof(b.RouterBwdArgs) + 4
    assert b.lib().moe_router_bwd(C.byref(a), None) == b.MGE_ERR_INVALID_ARG


def _unfused_args(**fwd_fields):
    u = b.FwdUnfusedArgs()
    u.struct_size = C.sizeof(b.FwdUnfusedArgs)
    u.fwd.struct_size = C.sizeof(b.FwdArgs)
    for k, v in dict(prec=1, E=4, H=64, F=128, T=8, k=2, align=32, y_dtype=0).items():
        setattr(u.fwd, k, v)
    for k, v in fwd_fields.items():
        setattr(u.fwd, k, v)
    return u


def test_fwd_unfused_rejects_and_workspace():
    L = b.lib()
    u = _unfused_args()
    # workspace: the fused forward's plus [G U] bf16 and the bf16 h (both absent), R = 160 rows
    R = b.perm_rows(8, 2, 4, 32)
    fused = L.mge_fwd_workspace_bytes(C.byref(u.fwd))
    assert L.mge_fwd_unfused_workspace_bytes(C.byref(u)) == fused + R * 2 * 128 * 2 + R * 128 * 2
    u.gu = 1 << 20
    assert L.mge_fwd_unfused_workspace_bytes(C.byref(u)) == fused + R * 128 * 2
    # struct sizes of both levels are checked
    u = _unfused_args()
    u.struct_size -= 8
    assert L.grouped_mlp_fwd_unfused(C.byref(u), None) == b.MGE_ERR_INVALID_ARG
    u = _unfused_args()
    u.fwd.struct_size -= 8
    assert L.grouped_mlp_fwd_unfused(C.byref(u), None) == b.MGE_ERR_INVALID_ARG
    # training: [G U] is written to saved_gu (no workspace for it), and a gu other than
    # saved_gu, or h_col without saved_gu, is rejected before any launch (fake device addresses)
    ptrs = (C.c_void_p * 4)(*[(i + 1) << 20 for i in range(4)])
    dev = {n: (i + 8) << 20 for i, n in enumerate(("split_sizes", "group_offsets", "prob_perm", "x_perm",
                                                     "x_perm_scale", "y_perm"))}
    u = _unfused_args(w_gate_up=C.cast(ptrs, C.c_void_p), w_down=C.cast(ptrs, C.c_void_p),
                      w_gate_up_scale=C.cast(ptrs, C.c_void_p), w_down_scale=C.cast(ptrs, C.c_void_p),
                      saved_gu=1 << 30, h_col=1 << 31, h_col_scale=1 << 32, **dev)
    assert L.mge_fwd_unfused_workspace_bytes(C.byref(u)) == L.mge_fwd_workspace_bytes(C.byref(u.fwd)) + R * 128 * 2
    u.gu = 1 << 20
    assert L.grouped_mlp_fwd_unfused(C.byref(u), None) == b.MGE_ERR_INVALID_ARG
    assert "saved_gu" in L.mge_last_error().decode()
    u.gu = None
    u.fwd.saved_gu = None
    assert L.grouped_mlp_fwd_unfused(C.byref(u), None) == b.MGE_ERR_INVALID_ARG
    assert "h_col" in L.mge_last_error().decode()


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """No fallback: without the built library every call raises instead of computing
    anything another way."""
    import moe_grouped_expert_amd as m

    monkeypatch.setattr(b, "_LIB", None)
    monkeypatch.setattr(b, "LIB_PATH", str(tmp_path / "libmge.so"))
    with pytest.raises(RuntimeError, match="not built"):
        b.lib()
    with pytest.raises(RuntimeError, match="not built"):
        m.perm_rows(8, 2, 4, 32)


def test_fwd_saved_bytes():
    """mge_fwd_saved_bytes is host arithmetic: G, U bf16 [R][2F], h column form [F][R]
    (+ [F][R/32] scales in MXFP8), R = mge_perm_rows."""
    R = b.perm_rows(8192, 2, 8, 32)
    s = b.fwd_saved_bytes("mxfp8", 8192, 2, 8, 14336, 32)
    assert s.rows == R
    assert s.saved_gu == R * 2 * 14336 * 2
    assert s.h_col == 14336 * R and s.h_col_scale == 14336 * (R // 32)
    assert s.total == s.saved_gu + s.h_col + s.h_col_scale
    t = b.fwd_saved_bytes("bf16", 256, 2, 4, 128, 32)
    assert t.h_col == 128 * b.perm_rows(256, 2, 4, 32) * 2 and t.h_col_scale == 0
    z = b.fwd_saved_bytes("mxfp8", 0, 2, 8, 64, 32)
    assert z.rows == 256 and z.total == 256 * (4 * 64 + 64 + 2)
    L = b.lib()
    o = b.FwdSavedSizes()
    o.struct_size = C.sizeof(b.FwdSavedSizes)
    for args in ((1, 10, 2, 8, 48, 32), (1, 10, 2, 8, 64, 8), (2, 10, 2, 8, 64, 32), (1, 10, 9, 8, 64, 32),
                 (1, -1, 2, 8, 64, 32)):
        assert L.mge_fwd_saved_bytes(*args, C.byref(o)) == b.MGE_ERR_INVALID_ARG, args
    o.struct_size = 4
    assert L.mge_fwd_saved_bytes(1, 10, 2, 8, 64, 32, C.byref(o)) == b.MGE_ERR_INVALID_ARG
    assert L.mge_fwd_saved_bytes(1, 10, 2, 8, 64, 32, None) == b.MGE_ERR_INVALID_ARG


def test_noalloc_route_host_checks():
    """moe_route_permute_noalloc rejects a workspace and sizes beyond its fixed scratch on
    the host, before touching the device."""
    L = b.lib()
    a = b.RouteArgs()
    a.struct_size = C.sizeof(b.RouteArgs)
    a.T, a.E, a.k, a.H, a.align = 300000, 256, 2, 64, 32
    for f in ("logits", "topk_idx", "topk_prob", "split_sizes", "group_offsets", "perm_src", "perm_pos", "prob_perm"):
        setattr(a, f, 0x10000)
    assert L.moe_route_permute_noalloc(C.byref(a), None) == b.MGE_ERR_UNSUPPORTED
    assert "scratch" in L.mge_last_error().decode()
    a.workspace, a.workspace_bytes = 0x10000, 1 << 20
    assert L.moe_route_permute_noalloc(C.byref(a), None) == b.MGE_ERR_INVALID_ARG
    a.workspace, a.workspace_bytes = None, 0
    a.T, a.k = 100, 9
    assert L.moe_route_permute_noalloc(C.byref(a), None) == b.MGE_ERR_INVALID_ARG
    assert L.moe_route_permute_noalloc(None, None) == b.MGE_ERR_INVALID_ARG


def test_bwd_per_tensor_fields_checked():
    """grouped_mlp_bwd's added per-tensor fields: the two scale pointers go together, need
    MXFP8, and dgu_bf16 needs them; a struct that ends before the fields is accepted."""
    L = b.lib()
    ptrs = (C.c_void_p * 4)(*[(i + 1) << 20 for i in range(4)])

    def args(**kw):
        a = b.BwdArgs()
        a.struct_size = C.sizeof(b.BwdArgs)
        a.prec, a.E, a.H, a.F, a.T, a.k, a.align = 1, 4, 64, 64, 8, 2, 32
        for n in ("dy", "split_sizes", "group_offsets", "perm_src", "perm_pos", "prob_perm", "saved_gu", "h_col",
                  "h_col_scale", "x_col", "x_col_scale", "dx_perm", "d_prob"):
            setattr(a, n, 1 << 24)
        for n in ("w_gate_up", "w_down", "w_gate_up_scale", "w_down_scale", "dw_gate_up", "dw_down"):
            setattr(a, n, C.cast(ptrs, C.c_void_p))
        for k_, v in kw.items():
            setattr(a, k_, v)
        return a

    a = args(dy_tensor_scale=1 << 25)
    assert L.grouped_mlp_bwd(C.byref(a), None) == b.MGE_ERR_INVALID_ARG
    assert "together" in L.mge_last_error().decode()
    a = args(dy_tensor_scale=1 << 25, dgu_tensor_scale=1 << 26, prec=0)
    assert L.grouped_mlp_bwd(C.byref(a), None) == b.MGE_ERR_INVALID_ARG
    a = args(dgu_bf16=1 << 27)
    assert L.grouped_mlp_bwd(C.byref(a), None) == b.MGE_ERR_INVALID_ARG
    # per-tensor mode needs more workspace ([dG dU] in bf16, the amax partials) unless dgu_bf16 is given
    plain = L.mge_bwd_workspace_bytes(C.byref(args()))
    pt = L.mge_bwd_workspace_bytes(C.byref(args(dy_tensor_scale=1 << 25, dgu_tensor_scale=1 << 26)))
    R = b.perm_rows(8, 2, 4, 32)
    assert pt >= plain + R * 2 * 64 * 2
    given = L.mge_bwd_workspace_bytes(C.byref(args(dy_tensor_scale=1 << 25, dgu_tensor_scale=1 << 26,
                                                   dgu_bf16=1 << 27)))
    assert plain < given < pt
    # the struct before the per-tensor fields: accepted, goes on to the workspace check
    a = args(dy_tensor_scale=1 << 25)
    a.struct_size = b.BwdArgs.dy_tensor_scale.offset
    assert L.grouped_mlp_bwd(C.byref(a), None) == b.MGE_ERR_WORKSPACE
