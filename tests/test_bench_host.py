"""Host logic of bench.py that needs no GPU: the algorithmic work charged to a kernel
launch, the per-kernel aggregation of the timing records, and the source digests that
keep counter-derived traffic from outliving the kernels it was measured on."""
import json
import os
import shutil

import pytest

import bench
import synth


def test_gemm_work_is_shared_by_the_launches_of_a_step():
    w = synth.WORKLOADS[2]
    mhf = float(w.M) * w.H * w.F
    assert bench.kernel_work("gemm_gateup_swiglu_mx", w, 0) == ("flop", 4 * mhf)
    # the per-expert loop launches each projection E times: each launch carries 1/E
    assert bench.kernel_work("gemm_gateup_swiglu_mx", w, 0, 8.0) == ("flop", 4 * mhf / 8)
    assert bench.kernel_work("gemm_down_mx", w, 0, 8.0) == ("flop", 2 * mhf / 8)
    assert bench.kernel_work("gemm_gateup_store_mx", w, 0) == ("flop", 4 * mhf)
    kind, n = bench.kernel_work("swiglu_prob", w, 0)
    assert kind == "byte" and n == 6.0 * w.M * w.F + 4.0 * w.M
    assert bench.kernel_work("tensor_amax", w, 0) is None
    # the BF16 backward's weight transposes: 2 launches per expert, (4 + 8) H F bytes per expert
    assert bench.kernel_work("transpose_bf16", w, 0) == ("byte", 6.0 * w.H * w.F)


def test_summarize_kernels_per_launch_and_share():
    w = synth.WORKLOADS[2]
    recs = [("gemm_down_mx", 1.0)] * 8 + [("combine", 0.5)] * 2 + [("route_topk", -1.0)]
    k, per_step = bench.summarize_kernels(recs, 2, w, 0, "mxfp8")
    assert k["gemm_down_mx"]["launches_per_step"] == 4.0 and k["gemm_down_mx"]["avg_ms"] == 1.0
    tf = 2.0 * w.M * w.H * w.F / 4 / 1e-3 / 1e12
    assert abs(k["gemm_down_mx"]["tflops"] - round(tf, 1)) < 0.11
    assert per_step == pytest.approx((8 * 1.0 + 2 * 0.5) / 2)
    assert "route_topk" not in k       # unreadable events are left out
    assert list(k)[0] == "gemm_down_mx"


def test_source_digests_by_family(tmp_path, monkeypatch):
    root = tmp_path / "r"
    shutil.copytree(os.path.join(bench.ROOT, "moe_grouped_expert_amd", "csrc"), root / "moe_grouped_expert_amd" / "csrc")
    monkeypatch.setattr(bench, "ROOT", str(root))
    g0, a0 = bench.kernel_source_digest("gemm"), bench.kernel_source_digest("all")
    csrc = root / "moe_grouped_expert_amd" / "csrc"
    # comments and blank lines are not code: editing them changes no digest
    gi = (csrc / "gemm_impl.hpp").read_text()
    (csrc / "gemm_impl.hpp").write_text("// note\n\n" + gi.replace("\n", "  // c\n", 3) + "\n/* block\n */\n")
    assert bench.kernel_source_digest("gemm") == g0 and bench.kernel_source_digest("all") == a0
    # a code change outside the GEMM sources leaves the GEMM digest alone
    (csrc / "quant.hip").write_text((csrc / "quant.hip").read_text() + "\nstatic int x_;\n")
    assert bench.kernel_source_digest("gemm") == g0 and bench.kernel_source_digest("all") != a0
    # so does one in mge_internal.hpp above the grouped-GEMM section
    txt = (csrc / "mge_internal.hpp").read_text()
    i = txt.index(bench.GEMM_PARAMS_MARK)
    (csrc / "mge_internal.hpp").write_text(txt[:i] + "static int y_;\n" + txt[i:])
    assert bench.kernel_source_digest("gemm") == g0
    # one inside it, or in a GEMM file, does not
    (csrc / "mge_internal.hpp").write_text(txt + "\nstatic int z_;\n")
    assert bench.kernel_source_digest("gemm") != g0
    (csrc / "mge_internal.hpp").write_text(txt)
    (csrc / "gemm_impl.hpp").write_text(gi + "\nstatic int w_;\n")
    assert bench.kernel_source_digest("gemm") != g0


def test_traffic_is_none_once_the_sources_change(tmp_path, monkeypatch):
    root = tmp_path / "r"
    shutil.copytree(os.path.join(bench.ROOT, "moe_grouped_expert_amd", "csrc"), root / "moe_grouped_expert_amd" / "csrc")
    (root / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(root))
    d = {"source_digests": {"all": bench.kernel_source_digest("all"), "gemm": bench.kernel_source_digest("gemm")},
         "kernels": {"train_mxfp8": {"gemm_dx_mx": {"hbm_bytes_per_launch": 123},
                                     "combine_kernel": {"hbm_bytes_per_launch": 7}}}}
    (root / "profiles" / "traffic.json").write_text(json.dumps(d))
    assert bench.traffic_for("gemm_dx_mx", "train_mxfp8") == 123
    assert bench.traffic_for("combine_kernel", "train_mxfp8") == 7
    assert bench.traffic_for("gemm_dx_mx", "fwd_mxfp8") is None
    csrc = root / "moe_grouped_expert_amd" / "csrc"
    (csrc / "combine.hip").write_text((csrc / "combine.hip").read_text() + "\nstatic int c_;\n")
    assert bench.traffic_for("gemm_dx_mx", "train_mxfp8") == 123
    assert bench.traffic_for("combine_kernel", "train_mxfp8") is None
