"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every source is compiled as the library is (gfx950 device code included) with the
sanitizers on the host compilation only, and linked with tests/host_san/abi_driver.cpp,
which runs every entry point's argument checks, the size queries and the T = 0 paths at and
past the documented limits.  A sanitizer report aborts the driver; the test also fails on
any call that returns a status other than the documented one."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_grouped_expert_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "host_san", "abi_driver.cpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain missing")


def test_host_code_under_asan_ubsan(tmp_path):
    from moe_grouped_expert_amd import build as b
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    import concurrent.futures as cf

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        path = src if os.path.isabs(src) else os.path.join(CSRC, src)
        cmd = [HIPCC, *b.FLAGS, "-O1", "-g", *san, "-c", path, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, b.SOURCES + [DRIVER]))
    exe = str(tmp_path / "abi_driver")
    link = [CLANGXX, "-fsanitize=address,undefined", "-o", exe, *objs, "-L/opt/rocm/lib", "-lamdhip64",
            "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and "abi_driver ok" in r.stdout, out[-4000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
