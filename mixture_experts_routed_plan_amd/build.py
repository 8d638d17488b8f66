"""Build libmoe_routed.so (HIP, gfx950) in-tree with hipcc, and its checked twin.

    python mixture_experts_routed_plan_amd/build.py

Every source under csrc/ is compiled to an object under _build/ and linked into
mixture_experts_routed_plan_amd/libmoe_routed.so; the same sources compiled with MOE_CHECKED
(objects under _build/checked/) make libmoe_routed_checked.so, whose kernels test every global
memory access against the extent of its buffer (a debugging and test build, not the product).
Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe_routed.so")
LIB_CHECKED = os.path.join(HERE, "libmoe_routed_checked.so")
SOURCES = ["abi.hip", "plan.hip", "rowops.hip", "gemm.hip", "router.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# packed-fp32 instruction forms are switched off for all device code
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _compile(src: str, checked: bool = False) -> str:
    out_dir = os.path.join(BUILD, "checked") if checked else BUILD
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DMOE_CHECKED"] if checked else []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)


def build(verbose: bool = False, checked: bool = True) -> str:
    """Builds libmoe_routed.so and, unless checked is False, libmoe_routed_checked.so."""
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        raise RuntimeError("hipcc not found")
    os.makedirs(os.path.join(BUILD, "checked"), exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + ([(src, True) for src in SOURCES] if checked else [])
    with ThreadPoolExecutor(min(len(jobs), 8)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    _link(objs[:len(SOURCES)], LIB)
    if verbose:
        print("built", LIB)
    if checked:
        _link(objs[len(SOURCES):], LIB_CHECKED)
        if verbose:
            print("built", LIB_CHECKED)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
