"""CPU oracle of the routed-experts layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import this
package. The GPU library never calls it, and it imports nothing from the GPU library.

The arithmetic lives in ``moe_oracle.c`` (plain C, double precision, optional bf16 storage
points); this module builds it with gcc and marshals numpy arrays. See the header of
``moe_oracle.c`` for the definition it follows and the passages it cites.

Modes:
  * ``"bf16"``  -- inputs are bf16 bit patterns; every storage point of the layer is rounded to bf16.
                  This is the contract the GPU path is compared against.
  * ``"exact"`` -- no rounding anywhere; inputs may be bf16 bits or float64 arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

IN_BF16, IN_F64 = 0, 1


class _Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("D", ctypes.c_int64), ("F", ctypes.c_int64),
                ("E", ctypes.c_int64), ("K", ctypes.c_int64), ("round_bf16", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("wgrad_f32", ctypes.c_int32)]


def build(force: bool = True) -> str:
    """Compile moe_oracle.c into liboracle.so (gcc -O2 -fopenmp; no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            L = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            S = ctypes.POINTER(_Shape)
            L.oracle_num_threads.restype = ctypes.c_int
            L.oracle_num_threads.argtypes = []
            L.oracle_round_bf16.restype = ctypes.c_double
            L.oracle_round_bf16.argtypes = [ctypes.c_double]
            L.oracle_plan.restype = I64
            L.oracle_plan.argtypes = [I64, I64, I64, P, P, P, P, P]
            L.oracle_forward.restype = ctypes.c_int
            L.oracle_forward.argtypes = [S] + [P] * 13
            L.oracle_backward.restype = ctypes.c_int
            L.oracle_backward.argtypes = [S] + [P] * 25
            L.oracle_tokens.restype = ctypes.c_int
            L.oracle_tokens.argtypes = [S, P, P, P, P, P, P, I64, P, P, P, P, P, P, P, P]
            L.oracle_store_array.restype = None
            L.oracle_store_array.argtypes = [S, I64, ctypes.c_int32, P, P]
            L.oracle_swiglu_array.restype = None
            L.oracle_swiglu_array.argtypes = [S, I64, P, P, P]
            L.oracle_swiglu_grad_array.restype = None
            L.oracle_swiglu_grad_array.argtypes = [S, I64, P, P, P, P, P]
            L.oracle_wgrad_entries.restype = ctypes.c_int
            L.oracle_wgrad_entries.argtypes = [S, P, P, P, P, P, P, I64, I64, P, P, I64, P, P, P, P,
                                               P, P]
            L.oracle_route.restype = ctypes.c_int
            L.oracle_route.argtypes = [I64, I64, I64, P, ctypes.c_int32, ctypes.c_int32, I64, I64,
                                       P, P]
            _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _shape(T, D, F, E, K, mode, in_dtype, wgrad_f32=False):
    if mode not in ("bf16", "exact"):
        raise ValueError(mode)
    return _Shape(T, D, F, E, K, 1 if mode == "bf16" else 0, in_dtype, 1 if wgrad_f32 else 0)


def _as_input(a, in_dtype):
    if a is None:
        return None
    if in_dtype == IN_BF16:
        if a.dtype != np.uint16:
            raise TypeError("bf16 inputs are passed as uint16 bit patterns")
        return np.ascontiguousarray(a)
    return np.ascontiguousarray(a, dtype=np.float64)


def _in_dtype_of(x):
    return IN_BF16 if x.dtype == np.uint16 else IN_F64


def num_threads() -> int:
    return lib().oracle_num_threads()


def round_bf16(v: float) -> float:
    return lib().oracle_round_bf16(float(v))


def plan(ids: np.ndarray, E: int) -> dict:
    """Stable counting sort of the flat slots by expert id."""
    T, K = ids.shape
    N = T * K
    ids64 = np.ascontiguousarray(ids, dtype=np.int64)
    counts = np.zeros(E, np.int64)
    offsets = np.zeros(E + 1, np.int64)
    pos = np.zeros(N, np.int64)
    src = np.zeros(N, np.int64)
    bad = lib().oracle_plan(T, K, E, _p(ids64), _p(counts), _p(offsets), _p(pos), _p(src))
    return dict(counts=counts, offsets=offsets, pos=pos, src=src, bad=int(bad))


def full(x, ids, scores, w13, w2, dout=None, mode: str = "bf16", wgrad_f32: bool = False,
         dw13_init=None, dw2_init=None, scales: bool = False) -> dict:
    """Whole layer on small shapes: plan, forward, and backward when dout is given.

    Returns every intermediate: xg, h13, a, y, out (+ dy, dscores, dh13, dxg, dx, dw13, dw2),
    all float64, plus the plan arrays. wgrad_f32: the weight gradients are stored in fp32 (not
    rounded to bf16); dw13_init / dw2_init: existing gradients that the new ones accumulate into
    (values, e.g. bf16 bit patterns widened, or float32). scales: also the root-sum-square of the
    terms of every summed output (out_rss, and with dout dscores_rss, dx_rss, dw13_rss,
    dw2_rss)."""
    T, D = x.shape
    E, two, F, D2 = w13.shape
    assert two == 2 and D2 == D and w2.shape == (E, D, F)
    K = ids.shape[1]
    N = T * K
    idt = _in_dtype_of(x)
    x, w13, w2 = (_as_input(a, idt) for a in (x, w13, w2))
    dout = _as_input(dout, idt)
    sh = _shape(T, D, F, E, K, mode, idt, wgrad_f32)
    pl = plan(ids, E)
    i13 = None if dw13_init is None else np.ascontiguousarray(dw13_init, dtype=np.float64)
    i2 = None if dw2_init is None else np.ascontiguousarray(dw2_init, dtype=np.float64)
    ids64 = np.ascontiguousarray(ids, dtype=np.int64)
    sc = np.ascontiguousarray(scores, dtype=np.float64)
    res = dict(pl)
    xg = np.zeros((N, D)); h13 = np.zeros((N, 2 * F)); a = np.zeros((N, F))
    y = np.zeros((N, D)); out = np.zeros((T, D))
    out_rss = np.zeros((T, D)) if scales else None
    L = lib()
    L.oracle_forward(ctypes.byref(sh), _p(x), _p(ids64), _p(sc), _p(w13), _p(w2), _p(pl["pos"]),
                     _p(pl["src"]), _p(xg), _p(h13), _p(a), _p(y), _p(out), _p(out_rss))
    res.update(xg=xg, h13=h13, a=a, y=y, out=out)
    if scales:
        res["out_rss"] = out_rss
    if dout is not None:
        dy = np.zeros((N, D)); dscores = np.zeros((T, K)); dh13 = np.zeros((N, 2 * F))
        dxg = np.zeros((N, D)); dx = np.zeros((T, D)); dw13 = np.zeros((E, 2, F, D))
        dw2 = np.zeros((E, D, F))
        rs = dict(dscores_rss=np.zeros((T, K)), dx_rss=np.zeros((T, D)),
                  dw13_rss=np.zeros((E, 2, F, D)), dw2_rss=np.zeros((E, D, F))) if scales else {}
        L.oracle_backward(ctypes.byref(sh), _p(dout), _p(ids64), _p(sc), _p(w13), _p(w2),
                          _p(pl["offsets"]), _p(pl["pos"]), _p(pl["src"]), _p(xg), _p(h13), _p(a),
                          _p(y), _p(dy), _p(dscores), _p(dh13), _p(dxg), _p(dx), _p(dw13), _p(dw2),
                          _p(i13), _p(i2), _p(rs.get("dscores_rss")), _p(rs.get("dx_rss")),
                          _p(rs.get("dw13_rss")), _p(rs.get("dw2_rss")))
        res.update(dy=dy, dscores=dscores, dh13=dh13, dxg=dxg, dx=dx, dw13=dw13, dw2=dw2, **rs)
    return res


def tokens(x, ids, scores, w13, w2, toks, dout=None, mode: str = "bf16", want_y: bool = False,
           scales: bool = False):
    """out (and dscores, dx when dout is given) for the listed tokens only, at any shape.
    scales: also the root-sum-square of each output's terms (out_rss, dscores_rss, dx_rss)."""
    T, D = x.shape
    E, _, F, _ = w13.shape
    K = ids.shape[1]
    idt = _in_dtype_of(x)
    x, w13, w2 = (_as_input(a, idt) for a in (x, w13, w2))
    dout = _as_input(dout, idt)
    sh = _shape(T, D, F, E, K, mode, idt)
    toks = np.ascontiguousarray(toks, dtype=np.int64)
    n = len(toks)
    ids64 = np.ascontiguousarray(ids, dtype=np.int64)
    sc = np.ascontiguousarray(scores, dtype=np.float64)
    out = np.zeros((n, D)); dsc = np.zeros((n, K)); dx = np.zeros((n, D))
    yr = np.zeros((n, K, D)) if want_y else None
    orss, drss, xrss = ((np.zeros((n, D)), np.zeros((n, K)), np.zeros((n, D))) if scales
                        else (None, None, None))
    lib().oracle_tokens(ctypes.byref(sh), _p(x), _p(ids64), _p(sc), _p(w13), _p(w2), _p(dout), n,
                        _p(toks), _p(out), _p(dsc), _p(dx), _p(yr), _p(orss), _p(drss), _p(xrss))
    res = dict(out=out)
    if dout is not None:
        res.update(dscores=dsc, dx=dx)
    if want_y:
        res["y"] = yr
    if scales:
        res["out_rss"] = orss
        if dout is not None:
            res.update(dscores_rss=drss, dx_rss=xrss)
    return res


def wgrad_entries(x, ids, scores, w13, w2, dout, e: int, jd: np.ndarray, df: np.ndarray,
                  mode: str = "bf16", wgrad_f32: bool = False, init13=None, init2=None,
                  scales: bool = False):
    """dW13[e, j, d] for the (j, d) pairs in jd ([n,2], j in [0,2F)) and dW2[e, d, f] for the
    (d, f) pairs in df ([m,2]); init13 / init2: existing values of those entries to accumulate
    into. Returns (v13, v2), or with scales (v13, v2, rss13, rss2): also each entry's
    root-sum-square of terms."""
    T, D = x.shape
    E, _, F, _ = w13.shape
    K = ids.shape[1]
    idt = _in_dtype_of(x)
    x, w13, w2, dout = (_as_input(a, idt) for a in (x, w13, w2, dout))
    sh = _shape(T, D, F, E, K, mode, idt, wgrad_f32)
    jd = np.ascontiguousarray(jd, dtype=np.int64).reshape(-1, 2)
    i13 = None if init13 is None else np.ascontiguousarray(init13, dtype=np.float64)
    i2 = None if init2 is None else np.ascontiguousarray(init2, dtype=np.float64)
    df = np.ascontiguousarray(df, dtype=np.int64).reshape(-1, 2)
    ids64 = np.ascontiguousarray(ids, dtype=np.int64)
    sc = np.ascontiguousarray(scores, dtype=np.float64)
    v13 = np.zeros(len(jd)); v2 = np.zeros(len(df))
    r13, r2 = (np.zeros(len(jd)), np.zeros(len(df))) if scales else (None, None)
    lib().oracle_wgrad_entries(ctypes.byref(sh), _p(x), _p(ids64), _p(sc), _p(w13), _p(w2),
                               _p(dout), int(e), len(jd), _p(jd), _p(v13), len(df), _p(df), _p(v2),
                               _p(i13), _p(i2), _p(r13), _p(r2))
    return (v13, v2, r13, r2) if scales else (v13, v2)


def _widen(a, in_dtype):
    """bf16 bit patterns (or float64 values) as float64 values."""
    if in_dtype == IN_BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, np.float64)


def expert_wgrad(x, ids, scores, w13, w2, dout, e: int, mode: str = "bf16",
                 wgrad_f32: bool = False, init13=None, init2=None, scales: bool = False) -> dict:
    """The whole weight gradients of expert e at any shape: dw13 [2,F,D] and dw2 [D,F] (float64).

    The expert's rows are its slots i (ids_i = e) in ascending i. Each row goes through the forward
    (h = [g|u] = R(W13[e] x_t), a = R(silu(g) u)) and the input-gradient steps the weight gradients
    consume (dy = R(s_i dout_t), da = W2[e]^T dy, [dg|du] by the SwiGLU derivative); then
    dW2[e] = RW(init + dy^T a) and dW13[e] = RW(init + [dg|du]^T x) over the rows (Dist-MoE,
    "Understand the execution model": WGRAD of W2 and W13; the rounding points of the full
    evaluation). The four contractions are float64 matrix products (a library step: the terms are
    products of bf16 values, exact in float64, so their sums round at most in the last bit of a
    double before the bf16 storage rounding); the rounding, SwiGLU and its derivative are the C
    oracle's own element functions. init13 / init2: existing gradients of that expert to
    accumulate into. scales: also dw13_rss, dw2_rss, the root-sum-square of each entry's terms,
    sqrt(sum_r term_r^2), as matrix products of the squared operands."""
    T, D = x.shape
    E, _, F, _ = w13.shape
    K = ids.shape[1]
    idt = _in_dtype_of(x)
    sh = _shape(T, D, F, E, K, mode, idt, wgrad_f32)
    L = lib()

    def store(v, wgrad=False):
        v = np.ascontiguousarray(v, np.float64)
        out = np.empty_like(v)
        L.oracle_store_array(ctypes.byref(sh), v.size, 1 if wgrad else 0, _p(v), _p(out))
        return out

    flat = np.asarray(ids, np.int64).reshape(-1)
    slots = np.nonzero(flat == e)[0]  # ascending slot index: the stable grouped order
    toks = slots // K
    xr = _widen(np.asarray(x)[toks], idt)                                 # [n, D]
    w13e = _widen(np.asarray(w13)[e], idt).reshape(2 * F, D)             # [2F, D]
    w2e = _widen(np.asarray(w2)[e], idt)                                  # [D, F]
    h = store(xr @ w13e.T)                                                # [n, 2F]
    g = np.ascontiguousarray(h[:, :F])
    u = np.ascontiguousarray(h[:, F:])
    a = np.empty_like(g)
    L.oracle_swiglu_array(ctypes.byref(sh), g.size, _p(g), _p(u), _p(a))
    sc = np.asarray(scores, np.float64).reshape(-1)[slots]
    dy = store(sc[:, None] * _widen(np.asarray(dout)[toks], idt))        # [n, D]
    da = np.ascontiguousarray(dy @ w2e)                                   # [n, F]
    dg = np.empty_like(da)
    du = np.empty_like(da)
    L.oracle_swiglu_grad_array(ctypes.byref(sh), da.size, _p(da), _p(g), _p(u), _p(dg), _p(du))
    dh = np.concatenate([dg, du], axis=1)                                 # [n, 2F]
    s2 = dy.T @ a                                                         # [D, F]
    s13 = dh.T @ xr                                                       # [2F, D]
    if init2 is not None:
        s2 = np.asarray(init2, np.float64).reshape(D, F) + s2
    if init13 is not None:
        s13 = np.asarray(init13, np.float64).reshape(2 * F, D) + s13
    res = dict(dw13=store(s13, wgrad=True).reshape(2, F, D), dw2=store(s2, wgrad=True))
    if scales:
        res["dw2_rss"] = np.sqrt((dy * dy).T @ (a * a))
        res["dw13_rss"] = np.sqrt((dh * dh).T @ (xr * xr)).reshape(2, F, D)
    return res


SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1


def route(logits: np.ndarray, K: int, score_fn: int = SCORE_SOFTMAX, renormalize: bool = True,
          n_group: int = 1, topk_group: int = 1):
    """Router: expert ids [T,K] (int64, selection order) and weights [T,K] (float64) from fp32
    logits [T,E]; see the router section of moe_oracle.c for the definition."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.zeros((T, K), np.int64)
    w = np.zeros((T, K), np.float64)
    rc = lib().oracle_route(T, E, K, _p(logits), int(score_fn), 1 if renormalize else 0,
                            int(n_group), int(topk_group if n_group > 1 else 1), _p(ids), _p(w))
    if rc != 0:
        raise ValueError("bad router configuration")
    return ids, w
