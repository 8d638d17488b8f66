"""The library's host code under AddressSanitizer (CPU only). The library sources are compiled
with the sanitizer on the host pass only (`-Xarch_host -fsanitize=address`; the device code is
built as usual and never runs here), linked with tests/asan_host_driver.cpp, and run with no GPU
visible. The driver sweeps about 700 k shapes through the size queries, the saved-buffer views
and the argument checks of moe_plan / moe_forward / moe_backward; every call it makes either is
host arithmetic or is rejected before a HIP call. A heap or stack error in any of those paths
aborts the run."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_routed_plan_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
SOURCES = ["abi.hip", "plan.hip", "rowops.hip", "gemm.hip", "router.hip"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s" % (" ".join(cmd), r.stderr[-3000:])
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm clang")
def test_host_code_is_clean_under_address_sanitizer(tmp_path):
    inc = os.path.join(ROOT, "include")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
             "-fno-omit-frame-pointer", "-I", inc]

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        _run([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    drv = str(tmp_path / "driver.o")
    _run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address", "-fno-omit-frame-pointer",
          "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", inc, "-c",
          os.path.join(ROOT, "tests", "asan_host_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "driver")
    _run([HIPCC, "--offload-arch=gfx950", "-fsanitize=address", *objs, drv, "-o", exe])
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "0 failed expectations" in r.stdout
    assert "AddressSanitizer" not in r.stderr
    print(r.stdout)
    shutil.rmtree(tmp_path, ignore_errors=True)
