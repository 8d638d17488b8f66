"""GPU: the recompute policy (MOE_RECOMPUTE: the forward saves only y -- and xg with MOE_KEEP_XG --
and the backward rebuilds h13 and a with the same kernel) gives every output bit for bit equal to
the saving path -- so the oracle parity of the saving path carries over -- and is also checked
against the oracle directly on a small shape. Likewise keeping xg (the permute, MOE_KEEP_XG) gives
every output bit for bit equal to gathering x's rows inside the GEMMs. Full size: the training
workload, every element of out, dx, dscores, dW13, dW2."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_check import check

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)


def _run(inp, recompute, keep_xg=False):
    from mixture_experts_routed_plan_amd import device as dv
    w = inp.w
    layer = dv.Layer(w.T, w.D, w.F, w.E, w.K, recompute=recompute, keep_xg=keep_xg)
    x, w13, w2, dout = (dv.to_device_bits(a) for a in (inp.x, inp.w13, inp.w2, inp.dout))
    ids = torch.from_numpy(inp.ids).cuda()
    sc = torch.from_numpy(inp.scores).cuda()
    layer.plan(ids)
    layer.forward(x, sc, w13, w2)
    layer.backward(dout, sc, w13, w2)
    torch.cuda.synchronize()
    return layer


def _outputs(layer):
    from mixture_experts_routed_plan_amd import device as dv
    return {"out": dv.to_host_bits(layer.out), "dx": dv.to_host_bits(layer.dx),
            "dscores": layer.dscores.cpu().numpy(), "dw13": dv.to_host_bits(layer.dw13),
            "dw2": dv.to_host_bits(layer.dw2)}


@pytest.mark.parametrize("name", ["tiny", "p_ragged", "p_skew", "p_wide", "training"])
def test_recompute_is_bitwise_the_saving_path(name):
    w = {**W.WORKLOADS, **W.PARITY_WORKLOADS}[name]
    inp = W.make_inputs(w, with_dout=True, router=oracle.route)
    a = _outputs(_run(inp, False))
    lr = _run(inp, True)
    b = _outputs(lr)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    sv = lr.saved_arrays()
    assert set(sv) == {"y"}
    log("[%s] recompute: all outputs bitwise equal to the saving path" % name)


@pytest.mark.parametrize("name", ["tiny", "p_ragged", "p_skew", "p_wide", "training"])
def test_keep_xg_is_bitwise_the_gather_path(name):
    w = {**W.WORKLOADS, **W.PARITY_WORKLOADS}[name]
    inp = W.make_inputs(w, with_dout=True, router=oracle.route)
    a = _outputs(_run(inp, False))
    for recompute in (False, True):
        lk = _run(inp, recompute, keep_xg=True)
        b = _outputs(lk)
        for k in a:
            np.testing.assert_array_equal(a[k], b[k], err_msg="%s recompute=%s" % (k, recompute))
        assert "xg" in lk.saved_arrays()
        del lk
    log("[%s] keep_xg (with and without recompute): all outputs bitwise equal" % name)


def test_recompute_against_oracle():
    from mixture_experts_routed_plan_amd import device as dv
    w = W.PARITY_WORKLOADS["p_ragged"]
    inp = W.make_inputs(w, with_dout=True, router=oracle.route)
    layer = _run(inp, True)
    ref = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, mode="bf16",
                      scales=True)
    check("out", dv.bits_to_f64(dv.to_host_bits(layer.out)), ref["out"])
    check("dx", dv.bits_to_f64(dv.to_host_bits(layer.dx)), ref["dx"])
    check("dscores", layer.dscores.cpu().numpy(), ref["dscores"], ref["dscores_rss"])
    check("dw13", dv.bits_to_f64(dv.to_host_bits(layer.dw13)), ref["dw13"], ref["dw13_rss"])
    check("dw2", dv.bits_to_f64(dv.to_host_bits(layer.dw2)), ref["dw2"], ref["dw2_rss"])
