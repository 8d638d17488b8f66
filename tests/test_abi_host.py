"""The C-ABI library on the host, without a GPU: it loads, exports every entry point the header
declares, and its host-side checks reject bad arguments before anything is enqueued (the failing
calls below never reach a HIP call, so they are safe without a device)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_routed.h")
LIB = os.path.join(ROOT, "mixture_experts_routed_plan_amd", "libmoe_routed.so")


def _load_build_script(root):
    """The build script, loaded by path: the package itself refuses to import unbuilt."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_moe_build_test", os.path.join(root, "mixture_experts_routed_plan_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _ensure_built():
    if not os.path.exists(LIB):
        _load_build_script(ROOT).build()


_ensure_built()
import mixture_experts_routed_plan_amd as M  # noqa: E402


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"moe_plan", "moe_forward", "moe_backward"} <= set(names)
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", nm))
    assert set(names) <= exported
    assert set(M.EXPORTED) == set(names)


def test_checked_library_exports_the_same_entry_points_and_its_own():
    """libmoe_routed_checked.so exports every entry point of moe_routed.h plus those of
    moe_routed_checked.h; the product library exports none of the latter."""
    checked = os.path.join(ROOT, "mixture_experts_routed_plan_amd", "libmoe_routed_checked.so")
    if not os.path.exists(checked):
        _load_build_script(ROOT).build()
    text = open(os.path.join(ROOT, "include", "moe_routed_checked.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    own = set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text))
    assert own == {"moe_checked_violations", "moe_checked_reset", "moe_checked_shrink"}

    def exported(path):
        nm = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                            text=True).stdout
        return set(re.findall(r"\bT (moe_\w+)", nm))

    assert exported(checked) == set(declared_functions()) | own
    assert not (exported(LIB) & own)


def test_abi_version_and_status_strings():
    assert M.moe_abi_version() == 4
    for st in range(0, -9, -1):
        assert M.moe_status_str(st) != "unknown status"
    assert M.moe_status_str(-99) == "unknown status"


def shape(**kw):
    d = dict(T=64, D=256, F=128, E=8, K=2, ids_dtype=M.MOE_IDS_I64, save_for_backward=True)
    d.update(kw)
    return M.make_shape(**d)


def test_sizes_are_closed_forms_of_the_shape():
    s = shape()
    N = 64 * 2
    assert M.moe_plan_bytes(s) >= 4 * (8 + 9 + 2 * N)
    # h13, a, y; xg only with MOE_KEEP_XG (otherwise the GEMMs read x through the plan)
    assert M.moe_saved_bytes(s) >= 2 * N * (2 * 128 + 128 + 256)
    keep = M.make_shape(64, 256, 128, 8, 2, keep_xg=True)
    assert M.moe_saved_bytes(keep) == M.moe_saved_bytes(s) + 2 * N * 256
    assert M.moe_workspace_bytes(s) >= 2 * N * (256 + 2 * 128)
    assert M.moe_saved_bytes(shape(save_for_backward=False)) == 0
    # recompute keeps only y (and xg when kept), and the backward needs room for the recomputed a
    re = M.make_shape(64, 256, 128, 8, 2, recompute=True)
    assert M.moe_saved_bytes(re) == M.moe_saved_bytes(s) - 2 * N * (2 * 128 + 128)
    assert M.moe_workspace_bytes(re) >= 2 * N * (256 + 2 * 128 + 128)  # dy, h13/dh13, a
    big = shape(T=640)
    assert M.moe_plan_bytes(big) > M.moe_plan_bytes(s)
    assert M.moe_saved_bytes(big) > M.moe_saved_bytes(s)


@pytest.mark.parametrize("kw", [dict(T=0), dict(K=0), dict(K=65), dict(E=0), dict(E=1025),
                                dict(D=100), dict(F=96), dict(D=32), dict(T=2 ** 30, K=4),
                                dict(D=2 ** 22 + 64), dict(F=2 ** 22 + 64),
                                dict(D=32768, F=32768 + 64), dict(D=2 ** 22, F=512),
                                dict(T=2 ** 24, K=64, D=2 ** 20, F=1024),
                                dict(T=2 ** 25 - 1023, K=64, D=64, F=64, E=1024)])
def test_bad_shapes_rejected(kw):
    s = shape(**kw)
    assert M.moe_plan_bytes(s) == 0
    assert M.moe_workspace_bytes(s) == 0
    assert M.moe_plan(s, 256, 256, 0) == M.MOE_E_SHAPE


@pytest.mark.parametrize("kw", [dict(D=32768, F=32768), dict(D=2 ** 22, F=256),
                                dict(D=64, F=2 ** 22), dict(T=2 ** 25 - 1024, K=64, D=64, F=64)])
def test_largest_widths_accepted(kw):
    # at the bounds: one expert's gate/up block is exactly 4 GiB, or a width is 2^22
    assert M.moe_plan_bytes(shape(**kw)) > 0


def test_bad_dtype_and_flags_rejected():
    s = shape()
    s.ids_dtype = 7
    assert M.moe_plan(s, 256, 256, 0) == M.MOE_E_DTYPE
    s = shape()
    s.flags = 32
    assert M.moe_plan_bytes(s) == 0
    s2 = shape()
    s2.flags = M.MOE_SAVE_FOR_BACKWARD | M.MOE_WGRAD_ACCUMULATE | M.MOE_WGRAD_F32
    assert M.moe_plan_bytes(s2) > 0
    s.flags = 32
    assert M.moe_forward(s, 256, 256, 256, 256, 256, 256, 256, 256, 0) == M.MOE_E_DTYPE


def test_null_and_alignment_rejected():
    s = shape()
    assert M.moe_plan(s, None, 256, 0) == M.MOE_E_NULL
    assert M.moe_plan(s, 256, None, 0) == M.MOE_E_NULL
    assert M.moe_plan(s, 260, 256, 0) == M.MOE_E_ALIGN  # int64 ids need 8-byte alignment
    assert M.moe_plan(s, 256, 264, 0) == M.MOE_E_ALIGN  # plan needs 16 bytes
    a = 4096
    assert M.moe_forward(s, a, a, a, a, a, None, a, a, 0) == M.MOE_E_NULL
    assert M.moe_forward(s, a, a + 8, a, a, a, a, a, a, 0) == M.MOE_E_ALIGN
    assert M.moe_forward(s, a, a, a + 2, a, a, a, a, a, 0) == M.MOE_E_ALIGN
    # forward with saving needs the saved buffer; without saving it needs the workspace
    assert M.moe_forward(s, a, a, a, a, a, a, None, a, 0) == M.MOE_E_NULL
    s2 = shape(save_for_backward=False)
    assert M.moe_forward(s2, a, a, a, a, a, a, a, None, 0) == M.MOE_E_NULL
    # with recompute the forward also needs the workspace (for a)
    s3 = M.make_shape(64, 256, 128, 8, 2, recompute=True)
    assert M.moe_forward(s3, a, a, a, a, a, a, a, None, 0) == M.MOE_E_NULL
    # backward: plan, saved, x, dout, scores, w13, w2, dx, dw13, dw2, dscores, workspace
    args = [a] * 12
    assert M.moe_backward(s, *args[:3], None, *args[4:], stream=0) == M.MOE_E_NULL  # dout
    assert M.moe_backward(s, *args[:2], None, *args[3:], stream=0) == M.MOE_E_NULL  # x
    assert M.moe_backward(s2, *args, stream=0) == M.MOE_E_STATE
    assert M.moe_backward(s, a, a, a, a, a, a, a, a + 4, a, a, a, a, 0) == M.MOE_E_ALIGN  # dx
    assert M.moe_backward(s, a, a, a + 2, a, a, a, a, a, a, a, a, a, 0) == M.MOE_E_ALIGN  # x
    assert M.moe_plan_export(s, None, stream=0) == M.MOE_E_NULL
    assert M.moe_plan_status(s, None, 0)[0] == M.MOE_E_NULL


def test_noalloc_forward_host_checks():
    """The allocation-free forward rejects, before any HIP call: a shape that saves for the
    backward, null or misaligned pointers, and a shape whose intermediates exceed its scratch."""
    a = 4096
    s = shape(save_for_backward=False)
    assert M.moe_forward_noalloc(shape(), a, a, a, a, a, a, 0) == M.MOE_E_STATE
    assert M.moe_forward_noalloc(s, a, a, a, a, a, None, 0) == M.MOE_E_NULL
    assert M.moe_forward_noalloc(s, a, a + 8, a, a, a, a, 0) == M.MOE_E_ALIGN
    assert M.moe_forward_noalloc(s, a, a, a + 2, a, a, a, 0) == M.MOE_E_ALIGN
    # a[N,F] and y[N,D] must fit: N = 16384 slots with D + F = 2048 is exactly 64 MiB (accepted:
    # the GPU test runs it), one more token is not
    assert 2 * 16384 * 2048 == M.MOE_NOALLOC_SCRATCH_BYTES
    over = M.make_shape(8193, 1024, 1024, 8, 2, save_for_backward=False)
    assert M.moe_forward_noalloc(over, a, a, a, a, a, a, 0) == M.MOE_E_SCRATCH
    # materializing xg takes room too
    keep = M.make_shape(8192, 1024, 1024, 8, 2, save_for_backward=False, keep_xg=True)
    assert M.moe_forward_noalloc(keep, a, a, a, a, a, a, 0) == M.MOE_E_SCRATCH


def test_row_step_arguments_rejected():
    a = 4096
    s = shape()
    assert M.moe_permute(s, a, None, a, 0) == M.MOE_E_NULL
    assert M.moe_permute(s, a, a + 2, a, 0) == M.MOE_E_ALIGN
    assert M.moe_combine(s, a, a, a, None, 0) == M.MOE_E_NULL
    assert M.moe_combine(s, a, a, a + 2, a, 0) == M.MOE_E_ALIGN  # scores
    assert M.moe_combine(s, a, a + 8, None, a, 0) == M.MOE_E_ALIGN
    assert M.moe_combine_backward(s, a, a, a, None, a, a, 0) == M.MOE_E_NULL  # scores required
    assert M.moe_combine_backward(s, a, a, a, a, a + 8, a, 0) == M.MOE_E_ALIGN
    assert M.moe_combine(shape(T=0), a, a, a, a, 0) == M.MOE_E_SHAPE


def test_router_arguments_rejected():
    a = 4096
    s = shape(E=16, K=4)
    r = M.make_router()
    assert M.moe_route(s, r, None, a, a, 0) == M.MOE_E_NULL
    assert M.moe_route(s, r, a + 2, a, a, 0) == M.MOE_E_ALIGN
    assert M.moe_route(s, r, a, a + 4, a, 0) == M.MOE_E_ALIGN  # int64 ids
    assert M.moe_route(s, r, a, a, a + 1, 0) == M.MOE_E_ALIGN
    assert M.moe_route(s, M.make_router(score_fn=5), a, a, a, 0) == M.MOE_E_DTYPE
    for kw in [dict(K=17), dict(E=1025, K=4), dict(K=65, E=128), dict(T=0)]:
        assert M.moe_route(shape(**dict(dict(E=16, K=4), **kw)), r, a, a, a, 0) == M.MOE_E_SHAPE
    # (only invalid configurations here: a valid one would launch on the bogus addresses)
    for rk in [dict(n_group=3, topk_group=1), dict(n_group=4, topk_group=0),
               dict(n_group=4, topk_group=5), dict(n_group=8, topk_group=1),
               dict(n_group=128, topk_group=2)]:
        assert M.moe_route(s, M.make_router(**rk), a, a, a, 0) == M.MOE_E_SHAPE, rk
    # the router does not read D, F or flags
    s3 = shape(E=16, K=4, D=100)
    assert M.moe_route(s3, r, None, a, a, 0) == M.MOE_E_NULL


def test_hip_failures_surface_as_a_status():
    """Calls that pass every argument check and then meet a failing HIP runtime return
    MOE_E_HIP instead of crashing. Forced from the host: a child process sees no GPU at all
    (HIP_VISIBLE_DEVICES=-1, ROCR_VISIBLE_DEVICES=-1), so every launch and copy fails and the
    placeholder pointers are never touched. Skipped where a GPU is present."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: this case needs a process without one")
    code = r"""
import mixture_experts_routed_plan_amd as M
s = M.make_shape(64, 256, 128, 8, 2)
A = 1 << 20  # aligned placeholder address, never dereferenced: no device can run anything
assert M.moe_plan(s, A, A, stream=0) == M.MOE_E_HIP
assert M.moe_forward(s, A, A, A, A, A, A, A, A, stream=0) == M.MOE_E_HIP
assert M.moe_backward(s, A, A, A, A, A, A, A, A, A, A, A, A, stream=0) == M.MOE_E_HIP
assert M.moe_permute(s, A, A, A, stream=0) == M.MOE_E_HIP
assert M.moe_plan_status(s, A, stream=0)[0] == M.MOE_E_HIP
print("ok")
"""
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    r = subprocess.run(["python", "-c", code], capture_output=True, text=True, cwd=ROOT, env=env,
                       timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr[-3000:]


def test_importing_without_the_library_fails_loudly(tmp_path):
    code = ("import sys, os; sys.path.insert(0, %r); import mixture_experts_routed_plan_amd as M"
            % str(tmp_path))
    pkg = tmp_path / "mixture_experts_routed_plan_amd"
    pkg.mkdir()
    src = open(os.path.join(ROOT, "mixture_experts_routed_plan_amd", "__init__.py")).read()
    (pkg / "__init__.py").write_text(src)
    r = subprocess.run(["python", "-c", code], capture_output=True, text=True)
    assert r.returncode != 0 and "not built" in r.stderr


def test_one_hip_runtime_when_imported_before_torch():
    """torch ships its own HIP runtime; the binding loads the library after importing torch, so
    the process maps one runtime even when the package is imported first (a second runtime would
    make launches on torch's streams fail)."""
    code = ("import mixture_experts_routed_plan_amd as M\nimport torch\n"
            "r = M._hip_runtimes()\nassert len(r) == 1, r\n")
    r = subprocess.run(["python", "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stderr


def test_build_entry_point_works_in_a_checkout_without_the_library(tmp_path):
    """__graft_entry__.build() on a tree that has sources only (no libmoe_routed.so, no oracle
    library): it compiles both and imports the package."""
    import shutil
    for d in ("mixture_experts_routed_plan_amd", "include", "oracle"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("*.so", "*.so.tmp*", "__pycache__"))
    shutil.copy(os.path.join(ROOT, "__graft_entry__.py"), tmp_path)
    assert not (tmp_path / "mixture_experts_routed_plan_amd" / "libmoe_routed.so").exists()
    code = ("import sys; sys.path.insert(0, %r); import __graft_entry__ as g; g.build(); "
            "import mixture_experts_routed_plan_amd as M; assert M.LIB_PATH.startswith(%r); "
            "print(M.moe_abi_version())" % (str(tmp_path), str(tmp_path)))
    r = subprocess.run(["python", "-c", code], capture_output=True, text=True, cwd=str(tmp_path))
    assert r.returncode == 0, r.stderr[-2000:]
    assert (tmp_path / "mixture_experts_routed_plan_amd" / "libmoe_routed.so").exists()
    assert r.stdout.strip().splitlines()[-1] == str(M.moe_abi_version())
