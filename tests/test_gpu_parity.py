"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded inputs.

* plan (counts, offsets, pos, src): bit-exact, every workload, int32 and int64 ids;
* permute (xg): bit-exact (a copy);
* every floating output, widened to double, element by element (parity_check.check):
  |gpu - oracle| <= 2e-2 * max(1, |oracle|), and for the long reductions (dscores, dW13, dW2)
  <= 2e-2 * max(1, |oracle|, rss) with rss the oracle's root-sum-square of that element's terms;
* an expert without rows: dW13[e] and dW2[e] exactly zero; a token whose scores are all zero
  (padding): out[t] and dx[t] exactly zero;
* small shapes (several 256-row tiles per expert, ragged tails, an intermediate width that is not
  a multiple of 128, skewed and duplicate routing, an empty expert): every element;
* the five full-size workloads, in the launch configuration the benchmark times: the plan and xg
  in full, out/dx/dscores on a seeded sample of 256 tokens, and every element of the weight
  gradients of 4 experts (most loaded, least loaded, two seeded others).
"""
import time

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_check import check, log

pytestmark = pytest.mark.gpu


def _lib():
    import mixture_experts_routed_plan_amd as M
    from mixture_experts_routed_plan_amd import device as dv
    return M, dv


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def upload(inp, ids_dtype=np.int64):
    _, dv = _lib()
    d = dict(x=dv.to_device_bits(inp.x), w13=dv.to_device_bits(inp.w13),
             w2=dv.to_device_bits(inp.w2),
             ids=torch.from_numpy(np.ascontiguousarray(inp.ids.astype(ids_dtype))).cuda(),
             scores=torch.from_numpy(inp.scores).cuda())
    if inp.dout is not None:
        d["dout"] = dv.to_device_bits(inp.dout)
    return d


def run(inp, ids_dtype=np.int64, backward=True, save=True, keep_xg=False):
    _, dv = _lib()
    w = inp.w
    d = upload(inp, ids_dtype)
    layer = dv.Layer(w.T, w.D, w.F, w.E, w.K, ids_dtype=ids_dtype, save_for_backward=save,
                     keep_xg=keep_xg)
    layer.plan(d["ids"])
    layer.forward(d["x"], d["scores"], d["w13"], d["w2"])
    if backward:
        layer.backward(d["dout"], d["scores"], d["w13"], d["w2"])
    torch.cuda.synchronize()
    return layer, d


def plan_check(layer, ids, E):
    got = layer.plan_arrays()
    ref = oracle.plan(ids, E)
    for k in ("counts", "offsets", "pos", "src"):
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
    st, bad = layer.plan_status()
    assert bad == ref["bad"]
    return got


# ------------------------------------------------------------------------------------------------
# plan

PLAN_CASES = list(W.WORKLOADS) + list(W.PARITY_WORKLOADS)


@pytest.mark.parametrize("ids_dtype", [np.int64, np.int32])
@pytest.mark.parametrize("name", PLAN_CASES)
def test_plan_bit_exact(name, ids_dtype):
    M, dv = _lib()
    w = {**W.WORKLOADS, **W.PARITY_WORKLOADS}[name]
    ids, _ = W.routing(w, ids_dtype, router=oracle.route)
    layer = dv.Layer(w.T, w.D, w.F, w.E, w.K, ids_dtype=ids_dtype, save_for_backward=False,
                     alloc_grads=False)
    layer.plan(torch.from_numpy(ids).cuda())
    plan_check(layer, ids, w.E)
    assert layer.plan_status() == (M.MOE_OK, 0)


@pytest.mark.parametrize("ids_dtype", [np.int64, np.int32])
def test_plan_out_of_range_and_duplicate_ids(ids_dtype):
    M, dv = _lib()
    rng = np.random.default_rng(5)
    T, K, E = 3000, 4, 37
    ids = rng.integers(0, E, (T, K))  # duplicates within a token
    bad_at = rng.choice(T * K, 50, replace=False)
    ids.ravel()[bad_at] = rng.choice([-1, -7, E, E + 100, 2 ** 31 - 1], 50)
    ids = ids.astype(ids_dtype)
    layer = dv.Layer(T, 64, 64, E, K, ids_dtype=ids_dtype, save_for_backward=False,
                     alloc_grads=False)
    layer.plan(torch.from_numpy(ids).cuda())
    plan_check(layer, ids, E)
    st, bad = layer.plan_status()
    assert st == M.MOE_E_BAD_IDS and bad == 50


def test_plan_many_experts_single_token_chunks():
    _, dv = _lib()
    rng = np.random.default_rng(6)
    for T, K, E in ((1, 1, 1), (1, 64, 1024), (5, 3, 1000), (2049, 1, 1024), (777, 13, 2)):
        ids = rng.integers(0, E, (T, K)).astype(np.int64)
        layer = dv.Layer(T, 64, 64, E, K, save_for_backward=False, alloc_grads=False)
        layer.plan(torch.from_numpy(ids).cuda())
        plan_check(layer, ids, E)


# ------------------------------------------------------------------------------------------------
# whole layer, every element

FULL_CASES = ["tiny", "p_ragged", "p_skew", "p_wide"]


def _full_check(inp, layer):
    _, dv = _lib()
    w = inp.w
    ref = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, mode="bf16",
                      scales=True)
    pl = plan_check(layer, inp.ids, w.E)
    sv = layer.saved_arrays()
    nv = int(ref["offsets"][-1])
    if layer.shape.flags & 16:  # MOE_KEEP_XG: the permute wrote xg and the forward saved it
        np.testing.assert_array_equal(sv["xg"][:nv], inp.x[pl["src"][:nv] // w.K])
    else:  # the GEMMs read x through the plan: no xg anywhere
        assert "xg" not in sv
    if "h13" in sv:  # not saved under MOE_RECOMPUTE
        check("h13", dv.bits_to_f64(sv["h13"][:nv]), ref["h13"][:nv])
        check("a", dv.bits_to_f64(sv["a"][:nv]), ref["a"][:nv])
    check("y", dv.bits_to_f64(sv["y"][:nv]), ref["y"][:nv])
    check("out", dv.bits_to_f64(dv.to_host_bits(layer.out)), ref["out"])
    check("dscores", layer.dscores.cpu().numpy(), ref["dscores"], ref["dscores_rss"])
    check("dx", dv.bits_to_f64(dv.to_host_bits(layer.dx)), ref["dx"])
    dw2 = dv.bits_to_f64(dv.to_host_bits(layer.dw2))
    dw13 = dv.bits_to_f64(dv.to_host_bits(layer.dw13))
    check("dw2", dw2, ref["dw2"], ref["dw2_rss"])
    check("dw13", dw13, ref["dw13"], ref["dw13_rss"])
    for e in np.nonzero(ref["counts"] == 0)[0]:  # an expert without rows: zero gradients
        assert (dw13[e] == 0).all() and (dw2[e] == 0).all(), "empty expert %d" % e
    return ref


@pytest.mark.parametrize("keep_xg", [False, True])  # x gathered inside the GEMMs / permute + xg
@pytest.mark.parametrize("name", FULL_CASES)
def test_layer_parity_every_element(name, keep_xg):
    w = {**W.WORKLOADS, **W.PARITY_WORKLOADS}[name]
    inp = W.make_inputs(w, router=oracle.route)
    log("\n[%s] T=%d D=%d F=%d E=%d K=%d keep_xg=%s" % (name, w.T, w.D, w.F, w.E, w.K, keep_xg))
    layer, _ = run(inp, keep_xg=keep_xg)
    _full_check(inp, layer)


def test_zero_score_padding():
    """Padded tokens carry zero scores in every slot (Dist-MoE, "Understand the execution model"):
    their rows are still computed, out[t] and dx[t] are exactly zero, their rows add nothing to
    the weight gradients, and dscores = <dout, y> stays nonzero; every element against the
    oracle."""
    w = W.PARITY_WORKLOADS["p_ragged"]
    inp = W.make_inputs(w, router=oracle.route)
    pad = np.random.default_rng(4).choice(w.T, 70, replace=False)
    inp.scores[pad] = 0.0
    _, dv = _lib()
    layer, _ = run(inp)
    ref = _full_check(inp, layer)
    out = dv.bits_to_f64(dv.to_host_bits(layer.out))
    dx = dv.bits_to_f64(dv.to_host_bits(layer.dx))
    assert (out[pad] == 0).all() and (dx[pad] == 0).all()
    assert (ref["out"][pad] == 0).all() and (ref["dx"][pad] == 0).all()
    assert (layer.dscores.cpu().numpy()[pad] != 0).mean() > 0.99


@pytest.mark.parametrize("name", ["p_ragged", "p_wide"])  # K = 3 (any-K combine), K = 4 (per-K)
def test_layer_parity_int32_ids_and_bad_ids(name):
    w = W.PARITY_WORKLOADS[name].with_(T=333)
    inp = W.make_inputs(w, ids_dtype=np.int32, router=oracle.route)
    inp.ids[5, 1] = w.E + 3
    inp.ids[77, 0] = -1
    layer, _ = run(inp, ids_dtype=np.int32)
    ref = _full_check(inp, layer)
    ds = layer.dscores.cpu().numpy()
    assert ds[5, 1] == 0 and ds[77, 0] == 0 and ref["bad"] == 2


def test_forward_without_save_matches_saving_forward():
    _, dv = _lib()
    inp = W.make_inputs(W.PARITY_WORKLOADS["p_ragged"], router=oracle.route)
    l1, _ = run(inp, backward=False, save=True)
    l2, _ = run(inp, backward=False, save=False)
    np.testing.assert_array_equal(dv.to_host_bits(l1.out), dv.to_host_bits(l2.out))


def test_repeated_calls_are_bitwise_identical():
    _, dv = _lib()
    inp = W.make_inputs(W.PARITY_WORKLOADS["p_skew"], router=oracle.route)
    l1, d = run(inp)
    outs = [dv.to_host_bits(t) for t in (l1.out, l1.dx, l1.dw13, l1.dw2)] + [
        l1.dscores.cpu().numpy()]
    l1.plan(d["ids"])
    l1.forward(d["x"], d["scores"], d["w13"], d["w2"])
    l1.backward(d["dout"], d["scores"], d["w13"], d["w2"])
    torch.cuda.synchronize()
    again = [dv.to_host_bits(t) for t in (l1.out, l1.dx, l1.dw13, l1.dw2)] + [
        l1.dscores.cpu().numpy()]
    for a, b in zip(outs, again):
        np.testing.assert_array_equal(a, b)


# ------------------------------------------------------------------------------------------------
# full-size workloads, sampled

_cache = {}


def _large(name):
    if name in _cache:
        return _cache[name]
    _cache.clear()
    _, dv = _lib()
    w = W.WORKLOADS[name]
    t0 = time.time()
    inp = W.make_inputs(w, with_dout=True, router=oracle.route)
    log("\n[%s] inputs drawn in %.1fs" % (name, time.time() - t0))
    layer, d = run(inp, backward=True, save=True)
    log("[%s] gpu forward+backward done" % name)
    _cache[name] = (inp, layer)
    return _cache[name]


LARGE = ["fine_grained", "large_hidden", "imbalanced", "training"]


@pytest.mark.parametrize("name", LARGE)
def test_large_plan_and_permute_in_full(name):
    inp, layer = _large(name)
    w = inp.w
    pl = plan_check(layer, inp.ids, w.E)
    assert "xg" not in layer.saved_arrays()  # the timed configuration gathers x in the GEMMs
    # the permute (MOE_KEEP_XG) at the same size, every row
    kl, _ = run(inp, backward=False, save=True, keep_xg=True)
    sv = kl.saved_arrays()
    np.testing.assert_array_equal(sv["xg"], inp.x[pl["src"] // w.K])
    del kl, sv


@pytest.mark.parametrize("half", [0, 1])
@pytest.mark.parametrize("name", LARGE)
def test_large_sampled_tokens(name, half):
    _, dv = _lib()
    inp, layer = _large(name)
    w = inp.w
    toks = W.sample_tokens(w.T, 256, seed=1)[half * 128:(half + 1) * 128]
    t0 = time.time()
    ref = oracle.tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, toks, inp.dout,
                        scales=True)
    log("\n[%s] oracle on %d tokens: %.1fs" % (name, len(toks), time.time() - t0))
    check("out", dv.bits_to_f64(dv.to_host_bits(layer.out))[toks], ref["out"])
    check("dscores", layer.dscores.cpu().numpy()[toks], ref["dscores"], ref["dscores_rss"])
    check("dx", dv.bits_to_f64(dv.to_host_bits(layer.dx))[toks], ref["dx"])


def four_experts(counts, seed):
    """The most loaded, the least loaded and two seeded other experts."""
    E = len(counts)
    rng = np.random.default_rng(seed)
    experts = [int(np.argmax(counts)), int(np.argmin(counts))]
    others = [e for e in range(E) if e not in experts]
    experts += [int(e) for e in rng.choice(others, min(2, len(others)), replace=False)]
    return experts


@pytest.mark.parametrize("name", LARGE)
def test_large_weight_grads_four_experts(name):
    """Every element of dW13[e] and dW2[e] for 4 experts (at the imbalanced workload the most
    loaded one is the 3x hot expert), in the launch configuration the benchmark times."""
    _, dv = _lib()
    inp, layer = _large(name)
    w = inp.w
    counts = oracle.plan(inp.ids, w.E)["counts"]
    dw13 = dv.to_host_bits(layer.dw13).reshape(w.E, 2, w.F, w.D)
    dw2 = dv.to_host_bits(layer.dw2)
    t0 = time.time()
    for e in four_experts(counts, 17):
        ref = oracle.expert_wgrad(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, e,
                                  scales=True)
        log("\n[%s] expert %d (%d rows), oracle %.1fs" % (name, e, counts[e], time.time() - t0))
        check("dw13", dv.bits_to_f64(dw13[e]), ref["dw13"], ref["dw13_rss"])
        check("dw2", dv.bits_to_f64(dw2[e]), ref["dw2"], ref["dw2_rss"])
        if counts[e] == 0:
            assert (dw13[e] == 0).all() and (dw2[e] == 0).all()
    log("[%s] oracle whole-expert weight gradients: %.1fs" % (name, time.time() - t0))


@pytest.mark.parametrize("name", ["fine_grained", "large_hidden"])
def test_large_forward_without_save_sampled(name):
    """Forward without saving (the permute fused into the gate/up GEMM, xg never written) at the
    two forward-only workloads: out on 256 sampled tokens against the oracle, and every element of
    out bitwise equal to the saving forward (which runs the separate permute)."""
    _, dv = _lib()
    w = W.WORKLOADS[name]
    inp = W.make_inputs(w, with_dout=False, router=oracle.route)
    ls, _ = run(inp, backward=False, save=True)
    ln, _ = run(inp, backward=False, save=False)
    np.testing.assert_array_equal(dv.to_host_bits(ln.out), dv.to_host_bits(ls.out))
    toks = W.sample_tokens(w.T, 256, seed=1)
    ref = oracle.tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, toks)
    log("\n[%s] forward without saving" % name)
    check("out", dv.bits_to_f64(dv.to_host_bits(ln.out))[toks], ref["out"])


# ------------------------------------------------------------------------------------------------
# degenerate shapes, every element

DEGENERATE = [
    # (T, D, F, E, K, routing, seed): one token, one expert, one slot; more experts than slots
    # (most experts empty); K = E with every expert in every token; a single 64-wide hidden and
    # intermediate; row tiles of exactly 256 rows; one ragged row after a full tile; the largest
    # E and K
    (1, 64, 64, 1, 1, "even", 11),
    (3, 128, 64, 16, 2, "uniform_distinct", 12),
    (40, 192, 128, 4, 4, "uniform_distinct", 13),
    (64, 64, 64, 2, 1, "even", 14),
    (512, 128, 192, 2, 1, "even", 15),
    (257, 64, 128, 1, 1, "even", 16),
    (64, 64, 64, 1024, 64, "uniform_distinct", 17),  # the largest E and K: 1024 tiny segments
    (200, 128, 64, 9, 6, "uniform_distinct", 18),    # K = 6: combine kernels compiled for K
    (100, 64, 64, 20, 13, "uniform_distinct", 19),   # K = 13: one 8-slot group and a remainder
]


@pytest.mark.parametrize("T,D,F,E,K,routing,seed", DEGENERATE)
def test_layer_parity_degenerate_shapes(T, D, F, E, K, routing, seed):
    w = W.Workload("degenerate", T=T, D=D, F=F, E=E, K=K, routing=routing, backward=True,
                   seed=seed)
    inp = W.make_inputs(w, router=oracle.route)
    log("\n[degenerate] T=%d D=%d F=%d E=%d K=%d %s" % (T, D, F, E, K, routing))
    layer, _ = run(inp)
    _full_check(inp, layer)


@pytest.mark.parametrize("seed", range(8))
def test_layer_parity_random_shapes(seed):
    """Seeded random shapes and options -- tokens, widths, experts, slots, routing rule, xg kept
    or gathered, recompute or save -- every element against the oracle."""
    _, dv = _lib()
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.integers(1, 41))
    K = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(1, 301))
    D = 64 * int(rng.integers(1, 9))
    F = 64 * int(rng.integers(1, 7))
    rules = ["even", "uniform_distinct", "topk_softmax"] + (["skewed"] if E >= 2 else [])
    routing = rules[int(rng.integers(len(rules)))]
    keep_xg, recompute = bool(rng.integers(2)), bool(rng.integers(2))
    w = W.Workload("random", T=T, D=D, F=F, E=E, K=K, routing=routing, backward=True,
                   seed=2000 + seed)
    inp = W.make_inputs(w, router=oracle.route)
    log("\n[random %d] T=%d D=%d F=%d E=%d K=%d %s keep_xg=%s recompute=%s"
        % (seed, T, D, F, E, K, routing, keep_xg, recompute))
    d = upload(inp)
    layer = dv.Layer(T, D, F, E, K, keep_xg=keep_xg, recompute=recompute)
    layer.plan(d["ids"])
    layer.forward(d["x"], d["scores"], d["w13"], d["w2"])
    layer.backward(d["dout"], d["scores"], d["w13"], d["w2"])
    torch.cuda.synchronize()
    _full_check(inp, layer)
