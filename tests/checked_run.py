"""Runs the layer through the checked library and exits non-zero on any failure (not a test module:
tests/test_gpu_checked.py starts it as a child process with MOE_ROUTED_LIBRARY=checked, since the
binding picks its library once per process).

For each shape (ragged, skewed with an empty expert, one token, 1024 experts with K=64, a 257-row
expert, K=6) and every flag combination (saving or not, recompute, xg kept, weight gradients in
bf16 or fp32, overwritten or accumulated): plan, forward, backward (when saving) or the
allocation-free forward, and the three row steps as entry points; after each, the violation
count of the checked kernels must be zero. The same at the four full-size workloads and with x
just under 4 GiB. The default-flag results at the small shapes are also held to the oracle's
elementwise bar, so the checks change nothing in what is computed. Finally the checks
themselves: with every GEMM extent taken 16 bytes short, a forward must report violations.
"""
import itertools
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import mixture_experts_routed_plan_amd as M  # noqa: E402
from mixture_experts_routed_plan_amd import device as dv  # noqa: E402
import oracle  # noqa: E402
import workloads as W  # noqa: E402
from parity_check import check, log  # noqa: E402

SHAPES = {
    "p_ragged": W.PARITY_WORKLOADS["p_ragged"],
    "p_skew": W.PARITY_WORKLOADS["p_skew"],
    "one": W.Workload("one", T=1, D=64, F=64, E=1, K=1, routing="even", backward=True, seed=31),
    "many": W.Workload("many", T=64, D=64, F=64, E=1024, K=64, routing="uniform_distinct",
                       backward=True, seed=32),
    "tail": W.Workload("tail", T=257, D=64, F=128, E=1, K=1, routing="even", backward=True,
                       seed=33),
    "k6": W.Workload("k6", T=200, D=128, F=64, E=9, K=6, routing="uniform_distinct",
                     backward=True, seed=34),
}

# (save, recompute, keep_xg, accumulate, f32)
FLAGS = [(False, False, kx, False, False) for kx in (False, True)] + [
    (True, re, kx, acc, f32)
    for re, kx, acc, f32 in itertools.product((False, True), repeat=4)]


def violations(what):
    n = M.moe_checked_violations()
    assert n == 0, "%s: %d accesses outside their buffers" % (what, n)


def bits(t):
    return dv.bits_to_f64(dv.to_host_bits(t))


def run_shape(name, w):
    inp = W.make_inputs(w, with_dout=True, router=oracle.route)
    ref = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, scales=True)
    x, w13, w2, dout = (dv.to_device_bits(a) for a in (inp.x, inp.w13, inp.w2, inp.dout))
    ids = torch.from_numpy(inp.ids).cuda()
    scores = torch.from_numpy(inp.scores).cuda()
    for save, re, kx, acc, f32 in FLAGS:
        tag = "%s save=%d recompute=%d keep_xg=%d accumulate=%d f32=%d" % (name, save, re, kx,
                                                                           acc, f32)
        layer = dv.Layer(w.T, w.D, w.F, w.E, w.K, save_for_backward=save, wgrad_accumulate=acc,
                         wgrad_f32=f32, recompute=re, keep_xg=kx)
        layer.plan(ids)
        layer.forward(x, scores, w13, w2)
        if save:
            layer.backward(dout, scores, w13, w2)
        elif 2 * w.T * w.K * (w.D + w.F) * (2 if kx else 1) <= M.MOE_NOALLOC_SCRATCH_BYTES:
            out2 = torch.empty_like(layer.out)
            M.check(M.moe_forward_noalloc(layer.shape, layer.plan_buf, x, scores, w13, w2, out2),
                    "moe_forward_noalloc")
        torch.cuda.synchronize()
        violations(tag)
        if save and not (re or kx or acc or f32):
            log(tag)
            check("out", bits(layer.out), ref["out"])
            check("dx", bits(layer.dx), ref["dx"])
            check("dscores", layer.dscores.cpu().numpy(), ref["dscores"], ref["dscores_rss"])
            check("dW13", bits(layer.dw13), ref["dw13"], ref["dw13_rss"])
            check("dW2", bits(layer.dw2), ref["dw2"], ref["dw2_rss"])
    # the row steps as entry points
    N, D = w.T * w.K, w.D
    layer = dv.Layer(w.T, w.D, w.F, w.E, w.K)
    layer.plan(ids)
    xg = torch.empty(N, D, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(w.T, D, dtype=torch.bfloat16, device="cuda")
    dy = torch.empty(N, D, dtype=torch.bfloat16, device="cuda")
    dsc = torch.empty(w.T, w.K, dtype=torch.float32, device="cuda")
    s = layer.shape
    M.check(M.moe_permute(s, layer.plan_buf, x, xg), "moe_permute")
    M.check(M.moe_combine(s, layer.plan_buf, xg, scores, out), "moe_combine")
    M.check(M.moe_combine(s, layer.plan_buf, xg, None, out), "moe_combine (unweighted)")
    M.check(M.moe_combine_backward(s, layer.plan_buf, dout, xg, scores, dy, dsc),
            "moe_combine_backward")
    torch.cuda.synchronize()
    violations(name + " row steps")
    log("[%s] %d flag combinations and the row steps: no access outside a buffer"
        % (name, len(FLAGS)))


def checks_detect():
    """Extents taken 16 bytes short: the last 16 bytes of each buffer count as outside."""
    w = SHAPES["p_ragged"]
    inp = W.make_inputs(w, with_dout=True)
    x, w13, w2 = (dv.to_device_bits(a) for a in (inp.x, inp.w13, inp.w2))
    ids = torch.from_numpy(inp.ids).cuda()
    scores = torch.from_numpy(inp.scores).cuda()
    layer = dv.Layer(w.T, w.D, w.F, w.E, w.K)
    layer.plan(ids)
    M.moe_checked_reset()
    M.moe_checked_shrink(16)
    try:
        layer.forward(x, scores, w13, w2)
        torch.cuda.synchronize()
        n = M.moe_checked_violations()
    finally:
        M.moe_checked_shrink(0)
        M.moe_checked_reset()
    assert n > 0, "extents 16 bytes short: no violation reported"
    layer.forward(x, scores, w13, w2)
    torch.cuda.synchronize()
    violations("p_ragged after restoring the extents")
    log("[checks] extents 16 bytes short: %d violations reported; restored: none" % n)


def run_large(name, w):
    """A full-size workload (default flags and fp32 weight-gradient accumulation): plan,
    forward, backward with no access outside a buffer."""
    inp = W.make_inputs(w, with_dout=True, router=oracle.route)
    x, w13, w2, dout = (dv.to_device_bits(a) for a in (inp.x, inp.w13, inp.w2, inp.dout))
    ids = torch.from_numpy(inp.ids).cuda()
    scores = torch.from_numpy(inp.scores).cuda()
    for acc_f32 in (False, True):
        layer = dv.Layer(w.T, w.D, w.F, w.E, w.K, wgrad_accumulate=acc_f32, wgrad_f32=acc_f32)
        layer.plan(ids)
        layer.forward(x, scores, w13, w2)
        layer.backward(dout, scores, w13, w2)
        torch.cuda.synchronize()
        violations("%s accumulate/f32=%d" % (name, acc_f32))
        del layer
    del x, w13, w2, dout, ids, scores, inp
    torch.cuda.empty_cache()
    log("[%s] full size: no access outside a buffer" % name)


def main():
    assert M.CHECKED, "set MOE_ROUTED_LIBRARY=checked"
    assert torch.cuda.is_available()
    M.moe_checked_reset()
    for name, w in SHAPES.items():
        log("[%s] start" % name)
        run_shape(name, w)
    for name in ("fine_grained", "large_hidden", "imbalanced", "training"):
        run_large(name, W.WORKLOADS[name])
    # x just under 4 GiB: the gate/up GEMM gathers token rows up to the end of x
    run_large("x_below_4gib", W.Workload("x_below_4gib", T=2**20 - 1, D=2048, F=64, E=8, K=1,
                                         routing="uniform_distinct", backward=True, seed=12))
    checks_detect()
    log("checked library: all cases clean")


if __name__ == "__main__":
    main()
