"""GPU parity of the weight-gradient storage modes (MOE_WGRAD_ACCUMULATE, MOE_WGRAD_F32) against
the oracle (Dist-MoE, "In-place WGRAD accumulation": gradients accumulate into existing BF16 or
FP32 storage, the same dtype for W13 and W2).

Every element on small shapes (ragged tiles, an expert without rows), with seeded nonzero initial
gradients; twice-accumulated fp32 gradients; every element of the gradients of 4 experts at the
full-size training workload with fp32 accumulation. Tolerance as for the layer, element by
element: |gpu - oracle| <= 2e-2 * max(1, |oracle|, rss), rss the root-sum-square of the new
contribution's terms."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_check import check as close, log

pytestmark = pytest.mark.gpu


def _init_grads(shape13, shape2, f32, seed):
    from mixture_experts_routed_plan_amd import device as dv
    rng = np.random.default_rng(seed)
    a13 = (rng.standard_normal(shape13) * 0.05).astype(np.float32)
    a2 = (rng.standard_normal(shape2) * 0.05).astype(np.float32)
    if f32:
        return a13, a2, torch.from_numpy(a13).cuda(), torch.from_numpy(a2).cuda()
    b13, b2 = W.f32_to_bf16_bits(a13), W.f32_to_bf16_bits(a2)
    return (W.bf16_bits_to_f32(b13), W.bf16_bits_to_f32(b2), dv.to_device_bits(b13),
            dv.to_device_bits(b2))


def _grads(layer, f32):
    from mixture_experts_routed_plan_amd import device as dv
    if f32:
        return layer.dw13.cpu().numpy().astype(np.float64), layer.dw2.cpu().numpy().astype(np.float64)
    return (dv.bits_to_f64(dv.to_host_bits(layer.dw13)), dv.bits_to_f64(dv.to_host_bits(layer.dw2)))


def _run(inp, accumulate, f32, init=None, calls=1):
    from mixture_experts_routed_plan_amd import device as dv
    w = inp.w
    layer = dv.Layer(w.T, w.D, w.F, w.E, w.K, wgrad_accumulate=accumulate, wgrad_f32=f32)
    if init is not None:
        layer.dw13.copy_(init[0])
        layer.dw2.copy_(init[1])
    x, w13, w2, dout = (dv.to_device_bits(a) for a in (inp.x, inp.w13, inp.w2, inp.dout))
    ids = torch.from_numpy(inp.ids).cuda()
    sc = torch.from_numpy(inp.scores).cuda()
    layer.plan(ids)
    layer.forward(x, sc, w13, w2)
    for _ in range(calls):
        layer.backward(dout, sc, w13, w2)
    torch.cuda.synchronize()
    return layer


MODES = [(False, True), (True, False), (True, True)]  # (accumulate, f32); overwrite+bf16 elsewhere


@pytest.mark.parametrize("accumulate,f32", MODES)
@pytest.mark.parametrize("name", ["tiny", "p_ragged", "p_skew"])
def test_wgrad_modes_every_element(name, accumulate, f32):
    w = {**W.WORKLOADS, **W.PARITY_WORKLOADS}[name]
    inp = W.make_inputs(w, with_dout=True, router=oracle.route)
    if name == "p_skew":
        inp.ids[inp.ids == w.E - 1] = 0  # the last expert gets no rows
    log("\n[%s] accumulate=%s f32=%s" % (name, accumulate, f32))
    h13, h2, d13, d2 = _init_grads((w.E, 2, w.F, w.D), (w.E, w.D, w.F), f32, 5)
    layer = _run(inp, accumulate, f32, init=(d13, d2) if accumulate else None)
    ref = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, wgrad_f32=f32,
                      dw13_init=h13 if accumulate else None, dw2_init=h2 if accumulate else None,
                      scales=True)
    g13, g2 = _grads(layer, f32)
    close("dw13", g13, ref["dw13"], ref["dw13_rss"])
    close("dw2", g2, ref["dw2"], ref["dw2_rss"])
    if name == "p_skew":
        e = w.E - 1
        assert ref["counts"][e] == 0
        if accumulate:  # untouched: the old gradient, bit for bit
            np.testing.assert_array_equal(g13[e], h13[e])
            np.testing.assert_array_equal(g2[e], h2[e])
        else:
            assert (g13[e] == 0).all() and (g2[e] == 0).all()


def test_fp32_accumulation_twice():
    w = W.PARITY_WORKLOADS["p_ragged"]
    inp = W.make_inputs(w, with_dout=True, router=oracle.route)
    h13, h2, d13, d2 = _init_grads((w.E, 2, w.F, w.D), (w.E, w.D, w.F), True, 6)
    layer = _run(inp, True, True, init=(d13, d2), calls=2)
    one = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, wgrad_f32=True,
                      scales=True)
    g13, g2 = _grads(layer, True)
    # two calls: twice the terms, so sqrt(2) * rss; 2 * rss bounds it
    close("dw13 x2", g13, h13 + 2 * one["dw13"], 2 * one["dw13_rss"])
    close("dw2 x2", g2, h2 + 2 * one["dw2"], 2 * one["dw2_rss"])


def test_fp32_accumulation_full_size_four_experts():
    """Training workload (16 experts, 8192 rows each on average), fp32 accumulation onto seeded
    gradients: every element of dW13 and dW2 for the most and least loaded expert and two seeded
    others."""
    w = W.WORKLOADS["training"]
    inp = W.make_inputs(w, with_dout=True, router=oracle.route)
    h13, h2, d13, d2 = _init_grads((w.E, 2, w.F, w.D), (w.E, w.D, w.F), True, 7)
    layer = _run(inp, True, True, init=(d13, d2))
    g13 = layer.dw13.cpu().numpy()
    g2 = layer.dw2.cpu().numpy()
    counts = oracle.plan(inp.ids, w.E)["counts"]
    rng = np.random.default_rng(18)
    experts = [int(np.argmax(counts)), int(np.argmin(counts))]
    experts += [int(e) for e in rng.choice([e for e in range(w.E) if e not in experts], 2, replace=False)]
    for e in experts:
        ref = oracle.expert_wgrad(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, e,
                                  wgrad_f32=True, init13=h13[e], init2=h2[e], scales=True)
        log("\n[training] expert %d (%d rows)" % (e, counts[e]))
        close("dw13", g13[e], ref["dw13"], ref["dw13_rss"])
        close("dw2", g2[e], ref["dw2"], ref["dw2_rss"])
