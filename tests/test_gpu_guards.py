"""GPU: no call writes outside its buffers. Every buffer the library touches -- the inputs, the plan,
saved and workspace buffers and every output -- is placed inside a larger allocation with
guard regions on both sides, filled with a position-dependent byte pattern. plan, forward and
backward then run under every flag combination (saving or not, recompute, xg kept, weight
gradients in bf16 or fp32, overwritten or accumulated), and the allocation-free forward too,
at ragged, skewed (an empty expert) and degenerate shapes; afterwards every guard byte must
hold its pattern and every input must be bitwise unchanged."""
import itertools

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_check import log

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes on each side (keeps every buffer 256-byte aligned)


class Guarded:
    """A device buffer of `nbytes` inside [guard | buffer | guard] with patterned guards."""

    def __init__(self, nbytes, seed):
        self.nbytes = int(nbytes)
        self.alloc = torch.empty(GUARD + self.nbytes + GUARD, dtype=torch.uint8, device="cuda")
        rng = np.random.default_rng(seed)
        self.pattern = torch.from_numpy(rng.integers(0, 256, 2 * GUARD, dtype=np.uint8)).cuda()
        self.alloc[:GUARD].copy_(self.pattern[:GUARD])
        self.alloc[GUARD + self.nbytes:].copy_(self.pattern[GUARD:])
        # the buffer itself starts with arbitrary bytes as well
        self.alloc[GUARD:GUARD + self.nbytes].copy_(
            torch.from_numpy(rng.integers(0, 256, self.nbytes, dtype=np.uint8)).cuda())

    @property
    def ptr(self):
        return self.alloc.data_ptr() + GUARD

    def view(self):
        return self.alloc[GUARD:GUARD + self.nbytes]

    def fill_from(self, t):
        b = t.contiguous().view(torch.uint8).reshape(-1)
        assert b.numel() == self.nbytes
        self.view().copy_(b)

    def guards_intact(self):
        return bool(torch.equal(self.alloc[:GUARD], self.pattern[:GUARD])) and bool(
            torch.equal(self.alloc[GUARD + self.nbytes:], self.pattern[GUARD:]))


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


@pytest.mark.parametrize("name", list(SHAPES))
def test_no_write_outside_any_buffer(name):
    import mixture_experts_routed_plan_amd as M
    from mixture_experts_routed_plan_amd import device as dv
    w = SHAPES[name]
    inp = W.make_inputs(w, with_dout=True, router=oracle.route)
    T, D, F, E, K = w.T, w.D, w.F, w.E, w.K
    seed = iter(range(1000, 10 ** 6))
    # inputs, guarded and kept for the unchanged-check
    inputs = {}
    for key, t in (("x", dv.to_device_bits(inp.x)), ("w13", dv.to_device_bits(inp.w13)),
                   ("w2", dv.to_device_bits(inp.w2)), ("dout", dv.to_device_bits(inp.dout)),
                   ("ids", torch.from_numpy(inp.ids).cuda()),
                   ("scores", torch.from_numpy(inp.scores).cuda())):
        g = Guarded(t.numel() * t.element_size(), next(seed))
        g.fill_from(t)
        inputs[key] = (g, t.contiguous().view(torch.uint8).reshape(-1).clone())
    runs = 0
    for save, re, kx, acc, f32 in FLAGS:
        s = M.make_shape(T, D, F, E, K, save_for_backward=save, wgrad_accumulate=acc,
                         wgrad_f32=f32, recompute=re, keep_xg=kx)
        gb = 4 if f32 else 2
        bufs = {
            "plan": Guarded(M.moe_plan_bytes(s), next(seed)),
            "workspace": Guarded(M.moe_workspace_bytes(s), next(seed)),
            "out": Guarded(2 * T * D, next(seed)),
        }
        if save:
            bufs.update(saved=Guarded(M.moe_saved_bytes(s), next(seed)),
                        dx=Guarded(2 * T * D, next(seed)),
                        dw13=Guarded(gb * E * 2 * F * D, next(seed)),
                        dw2=Guarded(gb * E * D * F, next(seed)),
                        dscores=Guarded(4 * T * K, next(seed)))
        p = {k: g.ptr for k, g in bufs.items()}
        i = {k: g.ptr for k, (g, _) in inputs.items()}
        M.check(M.moe_plan(s, i["ids"], p["plan"]), "moe_plan")
        M.check(M.moe_forward(s, p["plan"], i["x"], i["scores"], i["w13"], i["w2"], p["out"],
                              p.get("saved"), p["workspace"]), "moe_forward")
        if save:
            M.check(M.moe_backward(s, p["plan"], p["saved"], i["x"], i["dout"], i["scores"],
                                   i["w13"], i["w2"], p["dx"], p["dw13"], p["dw2"], p["dscores"],
                                   p["workspace"]), "moe_backward")
        elif 2 * T * K * (D + F) * (2 if kx else 1) <= M.MOE_NOALLOC_SCRATCH_BYTES:
            M.check(M.moe_forward_noalloc(s, p["plan"], i["x"], i["scores"], i["w13"], i["w2"],
                                          p["out"]), "moe_forward_noalloc")
        torch.cuda.synchronize()
        bad = [k for k, g in bufs.items() if not g.guards_intact()]
        bad += ["input " + k for k, (g, _) in inputs.items() if not g.guards_intact()]
        bad += ["input %s changed" % k for k, (g, orig) in inputs.items()
                if not torch.equal(g.view(), orig)]
        assert not bad, "%s flags save=%s recompute=%s keep_xg=%s accumulate=%s f32=%s: %s" % (
            name, save, re, kx, acc, f32, bad)
        runs += 1
        del bufs
    log("[%s] %d flag combinations: every guard byte intact, inputs unchanged" % (name, runs))
