"""GPU parity of the router (moe_route) against the oracle's router on the same fp32 logits.

Expert ids bit-exact (the selection compares the same fp32 logits on both sides, so no rounding
decides an id); weights within 1e-5 absolute (fp32 expf and fp32 sums against double; every
weight lies in [0, 1]) -- well inside the layer's 2e-2 bound. Cases: the two logit-routed
workloads at full size (64 experts top-6, 16 experts top-8), group-limited sigmoid routing,
many exact ties, the largest E and K, E not a multiple of 64, a single expert, NaN and infinite
logits, int32 ids; and the chain router -> plan -> forward/backward against oracle route -> full."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_check import check

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)


def _gpu_route(logits, K, score_fn=0, renorm=True, n_group=1, topk_group=1, ids_dtype=np.int64):
    import mixture_experts_routed_plan_amd as M
    T, E = logits.shape
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    tdt = torch.int64 if ids_dtype == np.int64 else torch.int32
    ids = torch.full((T, K), -7, dtype=tdt, device="cuda")
    sc = torch.full((T, K), -7.0, dtype=torch.float32, device="cuda")
    shape = M.make_shape(T, 64, 64, E, K,
                         ids_dtype=M.MOE_IDS_I64 if ids_dtype == np.int64 else M.MOE_IDS_I32)
    r = M.make_router(score_fn, renorm, n_group, topk_group)
    M.check(M.moe_route(shape, r, lg, ids, sc), "moe_route")
    torch.cuda.synchronize()
    return ids.cpu().numpy(), sc.cpu().numpy()


def _check(logits, K, **kw):
    ids_dtype = kw.pop("ids_dtype", np.int64)
    gi, gw = _gpu_route(logits, K, ids_dtype=ids_dtype, **kw)
    oi, ow = oracle.route(logits, K, score_fn=kw.get("score_fn", 0),
                          renormalize=kw.get("renorm", True), n_group=kw.get("n_group", 1),
                          topk_group=kw.get("topk_group", 1))
    assert gi.dtype == ids_dtype
    np.testing.assert_array_equal(gi.astype(np.int64), oi)
    fin = np.isfinite(ow)
    np.testing.assert_array_equal(np.isfinite(gw), fin)
    err = float(np.abs(gw[fin] - ow[fin]).max()) if fin.any() else 0.0
    log("  T=%d E=%d K=%d %s: ids exact, weight max err %.2e" % (logits.shape[0], logits.shape[1], K,
                                                                   kw, err))
    assert err <= 1e-5


@pytest.mark.parametrize("name", ["fine_grained", "training"])
def test_router_on_logit_routed_workloads(name):
    w = W.WORKLOADS[name]
    _check(W.router_logits(w), w.K)


def _normal(T, E, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal((T, E)) * scale).astype(np.float32)


def _tied(T, E, seed):
    return (np.round(np.random.default_rng(seed).standard_normal((T, E)) * 4) / 4).astype(np.float32)


@pytest.mark.parametrize("case", [
    dict(T=2048, E=256, K=8, score_fn=1, renorm=True, n_group=8, topk_group=4),
    dict(T=777, E=64, K=6, score_fn=0, renorm=False, n_group=8, topk_group=3),
    dict(T=300, E=96, K=5, score_fn=1, renorm=False, n_group=3, topk_group=1),
    dict(T=64, E=1024, K=64, score_fn=0, renorm=True, n_group=64, topk_group=8),
])
def test_router_group_limited(case):
    c = dict(case)
    T, E, K = c.pop("T"), c.pop("E"), c.pop("K")
    _check(_tied(T, E, T + E), K, **c)
    _check(_normal(T, E, T * E, 3.0), K, **c)


@pytest.mark.parametrize("T,E,K,kw", [
    (1000, 128, 10, dict(score_fn=0, renorm=False)),
    (999, 300, 17, dict(score_fn=1, renorm=False)),
    (64, 1024, 64, dict(score_fn=0, renorm=True)),
    (50, 1, 1, dict(score_fn=0, renorm=True)),
    (513, 16, 16, dict(score_fn=1, renorm=True)),
    (333, 40, 7, dict(score_fn=0, renorm=True, ids_dtype=np.int32)),
])
def test_router_ties_and_sizes(T, E, K, kw):
    _check(_tied(T, E, 7 * T + E), K, **kw)


def test_router_nan_and_infinite_logits():
    lg = _tied(200, 32, 9)
    rng = np.random.default_rng(10)
    lg[rng.random(lg.shape) < 0.05] = np.nan
    lg[rng.random(lg.shape) < 0.03] = np.inf
    lg[rng.random(lg.shape) < 0.03] = -np.inf
    _check(lg, 6, score_fn=1, renorm=False)
    ids, _ = _gpu_route(lg, 6)
    oi, _ = oracle.route(lg, 6)
    np.testing.assert_array_equal(ids, oi)


def test_router_then_layer_matches_oracle():
    """GPU router -> plan -> forward -> backward on a logit-routed parity shape, against the
    oracle's router and layer."""
    from mixture_experts_routed_plan_amd import device as dv
    w = W.PARITY_WORKLOADS["p_wide"]
    logits = W.router_logits(w)
    gi, gw = _gpu_route(logits, w.K)
    inp = W.make_inputs(w, with_dout=True, router=oracle.route)  # oracle-routed inputs
    np.testing.assert_array_equal(gi, inp.ids)
    layer = dv.Layer(w.T, w.D, w.F, w.E, w.K, save_for_backward=True)
    x, w13, w2, dout = (dv.to_device_bits(a) for a in (inp.x, inp.w13, inp.w2, inp.dout))
    ids_d = torch.from_numpy(gi).cuda()
    sc_d = torch.from_numpy(gw).cuda()
    layer.plan(ids_d)
    out = layer.forward(x, sc_d, w13, w2)
    layer.backward(dout, sc_d, w13, w2)
    torch.cuda.synchronize()
    ref = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, mode="bf16",
                      scales=True)
    check("out", dv.bits_to_f64(dv.to_host_bits(out)), ref["out"])
    check("dx", dv.bits_to_f64(dv.to_host_bits(layer.dx)), ref["dx"])
    check("dscores", layer.dscores.cpu().numpy(), ref["dscores"], ref["dscores_rss"])
