"""Python binding of libmoe_routed.so, the MI355X routed-experts layer (C ABI in
include/moe_routed.h). Argument marshalling only: every step of the layer runs in the library's
HIP kernels. The functions keep the C names; tensors are passed as torch tensors (their device
pointers are used), raw integer addresses or None.

The library must be built (``python mixture_experts_routed_plan_amd/build.py``); importing this
package without it raises ImportError -- there is no fallback implementation.

With MOE_ROUTED_LIBRARY=checked in the environment the package loads libmoe_routed_checked.so
instead (include/moe_routed_checked.h: the same entry points, with every global memory access of
the kernels tested against its buffer) and binds moe_checked_violations, moe_checked_reset and
moe_checked_shrink as well. The choice is made once, at import.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
CHECKED = os.environ.get("MOE_ROUTED_LIBRARY", "") == "checked"
LIB_PATH = os.path.join(_HERE, "libmoe_routed_checked.so" if CHECKED else "libmoe_routed.so")

MOE_IDS_I32 = 0
MOE_IDS_I64 = 1
MOE_SAVE_FOR_BACKWARD = 1
MOE_WGRAD_ACCUMULATE = 2
MOE_WGRAD_F32 = 4
MOE_RECOMPUTE = 8
MOE_KEEP_XG = 16
MOE_MAX_EXPERTS = 1024
MOE_MAX_TOPK = 64
MOE_TRACE_MAX_EVENTS = 16
MOE_SCORE_SOFTMAX = 0
MOE_SCORE_SIGMOID = 1
MOE_MAX_GROUPS = 64

MOE_OK = 0
MOE_E_NULL = -1
MOE_E_SHAPE = -2
MOE_E_ALIGN = -3
MOE_E_DTYPE = -4
MOE_E_HIP = -5
MOE_E_BAD_IDS = -6
MOE_E_STATE = -7
MOE_E_SCRATCH = -8
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("D", ctypes.c_int64), ("F", ctypes.c_int64),
                ("E", ctypes.c_int64), ("K", ctypes.c_int64), ("ids_dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32)]

    def __repr__(self):
        return "moe_shape(T=%d, D=%d, F=%d, E=%d, K=%d, ids_dtype=%d, flags=%d)" % (
            self.T, self.D, self.F, self.E, self.K, self.ids_dtype, self.flags)


class moe_trace(ctypes.Structure):
    _fields_ = [("n_events", ctypes.c_int32),
                ("events", ctypes.c_void_p * MOE_TRACE_MAX_EVENTS)]


class moe_router(ctypes.Structure):
    _fields_ = [("score_fn", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what or "moe", moe_status_str(status), status))


def _hip_runtimes():
    """Distinct HIP runtime libraries mapped into this process."""
    found = set()
    try:
        with open("/proc/self/maps") as fh:
            for line in fh:
                path = line.split()[-1]
                if os.path.basename(path).startswith("libamdhip64"):
                    found.add(os.path.realpath(path))
    except OSError:
        pass
    return sorted(found)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("%s is not built; run `python mixture_experts_routed_plan_amd/build.py`"
                          % LIB_PATH)
    # The library and torch must share one HIP runtime: torch's streams and allocations belong to
    # the runtime torch loaded, and torch ships its own copy of the HIP and HSA runtimes. With
    # torch imported first, the library's libamdhip64 dependency resolves to that copy; loading
    # the library first would map a second runtime into the process, and its launches on torch's
    # streams would fail.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are loaded in this process (%s): import torch before "
                          "any other library that links a HIP runtime" % ", ".join(runtimes))
    P, S, St = ctypes.c_void_p, ctypes.POINTER(moe_shape), ctypes.c_int
    Tr = ctypes.POINTER(moe_trace)
    sigs = {
        "moe_plan_bytes": (ctypes.c_size_t, [S]),
        "moe_saved_bytes": (ctypes.c_size_t, [S]),
        "moe_workspace_bytes": (ctypes.c_size_t, [S]),
        "moe_plan": (St, [S, P, P, P, Tr]),
        "moe_forward": (St, [S, P, P, P, P, P, P, P, P, P, Tr]),
        "moe_forward_noalloc": (St, [S, P, P, P, P, P, P, P, Tr]),
        "moe_permute": (St, [S, P, P, P, P]),
        "moe_combine": (St, [S, P, P, P, P, P]),
        "moe_combine_backward": (St, [S, P, P, P, P, P, P, P]),
        "moe_backward": (St, [S, P, P, P, P, P, P, P, P, P, P, P, P, P, Tr]),
        "moe_plan_export": (St, [S, P, P, P, P, P, P]),
        "moe_plan_status": (St, [S, P, ctypes.POINTER(ctypes.c_int64), P]),
        "moe_saved_views": (St, [S, P, ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(P),
                                 ctypes.POINTER(P)]),
        "moe_route": (St, [S, ctypes.POINTER(moe_router), P, P, P, P, Tr]),
        "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_abi_version": (ctypes.c_int, []),
    }
    if CHECKED:
        sigs.update({
            "moe_checked_violations": (St, [ctypes.POINTER(ctypes.c_uint64)]),
            "moe_checked_reset": (St, []),
            "moe_checked_shrink": (St, [ctypes.c_int64]),
        })
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


_lib = _load()
EXPORTED = ("moe_plan_bytes", "moe_saved_bytes", "moe_workspace_bytes", "moe_plan", "moe_forward",
            "moe_forward_noalloc", "moe_backward", "moe_permute", "moe_combine",
            "moe_combine_backward", "moe_plan_export", "moe_plan_status", "moe_saved_views",
            "moe_route", "moe_status_str", "moe_abi_version")


def _ptr(t):
    """Device address of a tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    if t.device.type != "cuda":
        raise ValueError("tensors passed to the library must live on the GPU")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_shape(T, D, F, E, K, ids_dtype=MOE_IDS_I64, save_for_backward=True,
               wgrad_accumulate=False, wgrad_f32=False, recompute=False,
               keep_xg=False) -> moe_shape:
    flags = ((MOE_SAVE_FOR_BACKWARD if save_for_backward else 0)
             | (MOE_WGRAD_ACCUMULATE if wgrad_accumulate else 0) | (MOE_WGRAD_F32 if wgrad_f32 else 0)
             | (MOE_RECOMPUTE if recompute else 0) | (MOE_KEEP_XG if keep_xg else 0))
    return moe_shape(int(T), int(D), int(F), int(E), int(K), int(ids_dtype), flags)


def moe_abi_version() -> int:
    return _lib.moe_abi_version()


def moe_status_str(status: int) -> str:
    return _lib.moe_status_str(int(status)).decode()


def moe_plan_bytes(shape: moe_shape) -> int:
    return _lib.moe_plan_bytes(ctypes.byref(shape))


def moe_saved_bytes(shape: moe_shape) -> int:
    return _lib.moe_saved_bytes(ctypes.byref(shape))


def moe_workspace_bytes(shape: moe_shape) -> int:
    return _lib.moe_workspace_bytes(ctypes.byref(shape))


def moe_plan(shape, topk_ids, plan, stream=None, trace=None) -> int:
    return _lib.moe_plan(ctypes.byref(shape), _ptr(topk_ids), _ptr(plan), _stream(stream),
                         None if trace is None else ctypes.byref(trace))


def moe_forward(shape, plan, x, scores, w13, w2, out, saved=None, workspace=None, stream=None,
                trace=None) -> int:
    return _lib.moe_forward(ctypes.byref(shape), _ptr(plan), _ptr(x), _ptr(scores), _ptr(w13),
                            _ptr(w2), _ptr(out), _ptr(saved), _ptr(workspace), _stream(stream),
                            None if trace is None else ctypes.byref(trace))


def moe_forward_noalloc(shape, plan, x, scores, w13, w2, out, stream=None, trace=None) -> int:
    return _lib.moe_forward_noalloc(ctypes.byref(shape), _ptr(plan), _ptr(x), _ptr(scores),
                                    _ptr(w13), _ptr(w2), _ptr(out), _stream(stream),
                                    None if trace is None else ctypes.byref(trace))


def moe_permute(shape, plan, x, xg, stream=None) -> int:
    return _lib.moe_permute(ctypes.byref(shape), _ptr(plan), _ptr(x), _ptr(xg), _stream(stream))


def moe_combine(shape, plan, rows, scores, out, stream=None) -> int:
    return _lib.moe_combine(ctypes.byref(shape), _ptr(plan), _ptr(rows), _ptr(scores), _ptr(out),
                            _stream(stream))


def moe_combine_backward(shape, plan, dout, y, scores, dy, dscores, stream=None) -> int:
    return _lib.moe_combine_backward(ctypes.byref(shape), _ptr(plan), _ptr(dout), _ptr(y),
                                     _ptr(scores), _ptr(dy), _ptr(dscores), _stream(stream))


def moe_backward(shape, plan, saved, x, dout, scores, w13, w2, dx, dw13, dw2, dscores, workspace,
                 stream=None, trace=None) -> int:
    return _lib.moe_backward(ctypes.byref(shape), _ptr(plan), _ptr(saved), _ptr(x), _ptr(dout),
                             _ptr(scores), _ptr(w13), _ptr(w2), _ptr(dx), _ptr(dw13), _ptr(dw2),
                             _ptr(dscores), _ptr(workspace), _stream(stream),
                             None if trace is None else ctypes.byref(trace))


def make_router(score_fn=MOE_SCORE_SOFTMAX, renormalize=True, n_group=1, topk_group=1) -> moe_router:
    return moe_router(int(score_fn), 1 if renormalize else 0, int(n_group), int(topk_group))


def moe_route(shape, router, logits, topk_ids, scores, stream=None, trace=None) -> int:
    return _lib.moe_route(ctypes.byref(shape), ctypes.byref(router), _ptr(logits), _ptr(topk_ids),
                          _ptr(scores), _stream(stream),
                          None if trace is None else ctypes.byref(trace))


def moe_plan_export(shape, plan, counts=None, offsets=None, pos=None, src=None,
                    stream=None) -> int:
    return _lib.moe_plan_export(ctypes.byref(shape), _ptr(plan), _ptr(counts), _ptr(offsets),
                                _ptr(pos), _ptr(src), _stream(stream))


def moe_plan_status(shape, plan, stream=None):
    """Returns (status, number of out-of-range ids); waits for the stream."""
    bad = ctypes.c_int64(0)
    st = _lib.moe_plan_status(ctypes.byref(shape), _ptr(plan), ctypes.byref(bad), _stream(stream))
    return st, bad.value


def moe_saved_views(shape, saved):
    """Device addresses (xg, h13, a, y) inside a saved buffer."""
    ptrs = [ctypes.c_void_p() for _ in range(4)]
    st = _lib.moe_saved_views(ctypes.byref(shape), _ptr(saved), *[ctypes.byref(p) for p in ptrs])
    if st != MOE_OK:
        raise MoeError(st, "moe_saved_views")
    return tuple(p.value for p in ptrs)


def moe_checked_violations() -> int:
    """Checked library only: accesses found outside their buffer since load or the last reset."""
    n = ctypes.c_uint64(0)
    check(_lib.moe_checked_violations(ctypes.byref(n)), "moe_checked_violations")
    return n.value


def moe_checked_reset() -> None:
    check(_lib.moe_checked_reset(), "moe_checked_reset")


def moe_checked_shrink(nbytes: int) -> None:
    check(_lib.moe_checked_shrink(int(nbytes)), "moe_checked_shrink")


def check(status: int, what: str = "") -> None:
    if status != MOE_OK:
        raise MoeError(status, what)
