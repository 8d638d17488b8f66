"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties one part of the oracle to a library routine, a closed form, a brute-force dense
evaluation, calculus (finite differences) or an exact algebraic invariant, so that a dropped term,
a wrong sign, a transposed operand or a wrong index in the oracle fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------------------------------------
# helpers (inputs only; no layer arithmetic here except the dense reference formulations)

def small_inputs(T=12, D=64, F=48, E=5, K=3, seed=0, dup=False, bad=False, f64=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, D))
    w13 = rng.standard_normal((E, 2, F, D)) / math.sqrt(D)
    w2 = rng.standard_normal((E, D, F)) / math.sqrt(F)
    dout = rng.standard_normal((T, D))
    if dup:
        ids = rng.integers(0, E, (T, K))
    else:
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    if bad:
        ids[1, 0] = E
        ids[3, K - 1] = -1
    scores = rng.uniform(0.1, 1.0, (T, K))
    if not f64:
        x, w13, w2, dout = (W.f32_to_bf16_bits(a.astype(np.float32)) for a in (x, w13, w2, dout))
        scores = scores.astype(np.float32)
    return x, ids.astype(np.int64), scores, w13, w2, dout


def as_f64(a):
    return W.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else np.asarray(a, np.float64)


def dense_torch(x, ids, scores, w13, w2, dout):
    """Dense brute force in float64 with torch autograd: every expert applied to every token, the
    results masked and weighted by the routing. Returns out and the gradients of sum(out*dout)."""
    E = w13.shape[0]
    x = torch.tensor(as_f64(x), requires_grad=True)
    w13 = torch.tensor(as_f64(w13), requires_grad=True)
    w2 = torch.tensor(as_f64(w2), requires_grad=True)
    s = torch.tensor(np.asarray(scores, np.float64), requires_grad=True)
    ids_t = torch.tensor(ids)
    valid = (ids_t >= 0) & (ids_t < E)
    onehot = torch.nn.functional.one_hot(ids_t.clamp(0, E - 1), E).double() * valid[..., None]
    m = (s[..., None] * onehot).sum(1)  # [T,E]
    g = torch.einsum("td,efd->tef", x, w13[:, 0])
    u = torch.einsum("td,efd->tef", x, w13[:, 1])
    a = torch.nn.functional.silu(g) * u
    yall = torch.einsum("tef,edf->ted", a, w2)
    out = torch.einsum("te,ted->td", m, yall)
    (out * torch.tensor(as_f64(dout))).sum().backward()
    return dict(out=out.detach().numpy(), dx=x.grad.numpy(), dw13=w13.grad.numpy(),
                dw2=w2.grad.numpy(), dscores=s.grad.numpy())


def rne_t(a):
    """bf16 rounding by torch's own conversion (a library routine), as float64."""
    return torch.as_tensor(a).to(torch.float32).to(torch.bfloat16).to(torch.float64)


def bf16_ulp(v):
    v = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -126)))
    return 2.0 ** (e - 7)


# ------------------------------------------------------------------------------------------------
# bf16 rounding

def test_round_bf16_ties_and_overflow():
    r = oracle.round_bf16
    assert r(1 + 2 ** -8) == 1.0  # half an ulp above 1: tie -> even (1.0)
    assert r(1 + 3 * 2 ** -8) == 1 + 2 ** -6  # 1.5 ulp: tie -> even mantissa
    assert r(1 + 2 ** -8 + 2 ** -30) == 1 + 2 ** -7  # just above the tie
    assert r(-(1 + 2 ** -8)) == -1.0
    assert r(float.fromhex("0x1.FDp127")) == float.fromhex("0x1.FCp127")  # largest finite
    assert math.isinf(r(float.fromhex("0x1.FEp127")))  # tie with 2^128 -> even -> overflow
    assert r(2.0 ** -133) == 2.0 ** -133  # smallest subnormal bf16
    assert r(2.0 ** -135) == 0.0
    assert r(3 * 2.0 ** -134) == 2 * 2.0 ** -133  # 1.5 subnormal steps: tie -> even (2 steps)
    assert r(0.0) == 0.0 and math.isnan(r(float("nan")))


def test_round_bf16_matches_torch_conversion():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-38).astype(np.float32),
        (rng.standard_normal(5000) * 1e30).astype(np.float32),
        # exact ties: bf16 value + half ulp, built from bit patterns
        (((rng.integers(0, 1 << 15, 5000).astype(np.uint32) << 16) | 0x8000)).view(np.float32),
    ])
    v = v[np.isfinite(v)]
    ref = rne_t(torch.from_numpy(v)).numpy()
    got = np.array([oracle.round_bf16(float(a)) for a in v])
    np.testing.assert_array_equal(got, ref)


# ------------------------------------------------------------------------------------------------
# plan

def test_plan_quickstart_closed_form_and_golden():
    w = W.WORKLOADS["tiny"]
    ids, _ = W.routing(w)
    gold = np.loadtxt(os.path.join(GOLDEN, "quickstart_even_routing.txt"), dtype=np.int64)
    np.testing.assert_array_equal(gold[:, 0], np.arange(16))
    np.testing.assert_array_equal(ids, gold[:, 1:])
    pl = oracle.plan(ids, w.E)
    T, K, E = w.T, w.K, w.E
    # round-robin routing: every expert gets T*K/E slots, and slot i = t*K+k of expert i mod E is
    # the floor(i/E)-th of its expert
    np.testing.assert_array_equal(pl["counts"], np.full(E, T * K // E))
    i = np.arange(T * K)
    np.testing.assert_array_equal(pl["pos"], (i % E) * (T * K // E) + i // E)
    assert pl["bad"] == 0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_plan_matches_stable_argsort(seed):
    rng = np.random.default_rng(seed)
    T, K, E = 97, 5, 11
    ids = rng.integers(0, E, (T, K))  # duplicates inside a token allowed
    ids[rng.integers(0, T, 6), rng.integers(0, K, 6)] = rng.choice([-3, -1, E, E + 4], 6)
    pl = oracle.plan(ids, E)
    flat = ids.ravel()
    valid = (flat >= 0) & (flat < E)
    order = np.argsort(np.where(valid, flat, E), kind="stable")  # library stable sort
    nvalid = int(valid.sum())
    np.testing.assert_array_equal(pl["src"][:nvalid], order[:nvalid])
    assert (pl["src"][nvalid:] == -1).all()
    np.testing.assert_array_equal(pl["counts"], np.bincount(flat[valid], minlength=E))
    assert pl["bad"] == (~valid).sum()
    # invariants: conservation, monotone offsets, src o pos = id, segment membership, stability
    assert pl["counts"].sum() + pl["bad"] == T * K
    assert pl["offsets"][0] == 0 and pl["offsets"][-1] == nvalid
    assert (np.diff(pl["offsets"]) == pl["counts"]).all()
    vi = np.nonzero(valid)[0]
    np.testing.assert_array_equal(pl["src"][pl["pos"][vi]], vi)
    assert (pl["pos"][~valid] == -1).all()
    for e in range(E):
        seg = pl["src"][pl["offsets"][e]:pl["offsets"][e + 1]]
        assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()


def test_plan_conservation_on_workloads():
    for name in ("fine_grained", "imbalanced", "training"):
        w = W.WORKLOADS[name]
        ids, _ = W.routing(w, router=oracle.route)
        pl = oracle.plan(ids, w.E)
        assert pl["counts"].sum() == w.T * w.K and pl["bad"] == 0
    c = oracle.plan(W.routing(W.WORKLOADS["imbalanced"])[0], 32)["counts"]
    assert c.max() == 3 * c.mean() == 6144


# ------------------------------------------------------------------------------------------------
# forward / backward against dense brute force (library autograd), exact mode

@pytest.mark.parametrize("kw", [dict(), dict(dup=True), dict(bad=True), dict(dup=True, f64=True)])
def test_exact_mode_matches_dense_autograd(kw):
    x, ids, s, w13, w2, dout = small_inputs(**kw)
    ref = dense_torch(x, ids, s, w13, w2, dout)
    got = oracle.full(x, ids, s, w13, w2, dout, mode="exact")
    for k in ("out", "dx", "dw13", "dw2", "dscores"):
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-10, atol=1e-11, err_msg=k)


def test_exact_mode_tiny_workload_matches_dense_autograd():
    inp = W.make_inputs(W.WORKLOADS["tiny"])
    ref = dense_torch(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout)
    got = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, mode="exact")
    for k in ("out", "dx", "dw13", "dw2", "dscores"):
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-10, atol=1e-10, err_msg=k)


def test_exact_mode_central_finite_differences():
    x, ids, s, w13, w2, dout = small_inputs(T=6, D=16, F=12, E=3, K=2, seed=3, f64=True)
    g = oracle.full(x, ids, s, w13, w2, dout, mode="exact")

    def loss(x_, s_, w13_, w2_):
        o = oracle.full(x_, ids, s_, w13_, w2_, None, mode="exact")["out"]
        return float((o * dout).sum())

    rng = np.random.default_rng(0)
    h = 1e-6
    for name, arr, grad in (("x", x, g["dx"]), ("s", s, g["dscores"]), ("w13", w13, g["dw13"]),
                            ("w2", w2, g["dw2"])):
        for _ in range(6):
            idx = tuple(rng.integers(0, n) for n in arr.shape)
            args = dict(x_=x, s_=s, w13_=w13, w2_=w2)
            key = {"x": "x_", "s": "s_", "w13": "w13_", "w2": "w2_"}[name]
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            fd = (loss(**{**args, key: ap}) - loss(**{**args, key: am})) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


# ------------------------------------------------------------------------------------------------
# bf16 contract

def dense_bf16_reference(x, ids, s, w13, w2, dout):
    """Dense every-expert-on-every-token evaluation with bf16 rounding (torch's conversion) at
    the same storage points; sums in float64 in a different order from the oracle."""
    E = w13.shape[0]
    x = torch.tensor(as_f64(x)); w13 = torch.tensor(as_f64(w13)); w2 = torch.tensor(as_f64(w2))
    do = torch.tensor(as_f64(dout)); s = torch.tensor(np.asarray(s, np.float64))
    T, K = ids.shape
    g = rne_t(torch.einsum("td,efd->tef", x, w13[:, 0]))
    u = rne_t(torch.einsum("td,efd->tef", x, w13[:, 1]))
    a = rne_t(g * torch.sigmoid(g) * u)
    yall = rne_t(torch.einsum("tef,edf->ted", a, w2))
    out = torch.zeros_like(x)
    dx = torch.zeros_like(x)
    dw13 = torch.zeros_like(w13)
    dw2 = torch.zeros_like(w2)
    dsc = torch.zeros(T, K, dtype=torch.float64)
    routed = torch.zeros(T, E, dtype=torch.bool)
    dy_all = torch.zeros(T, E, x.shape[1], dtype=torch.float64)
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            routed[t, e] = True
            dy_all[t, e] = rne_t(s[t, k] * do[t])
            dsc[t, k] = (do[t] * yall[t, e]).sum()
    out = rne_t(torch.stack([sum(s[t, k] * yall[t, int(ids[t, k])] for k in range(K))
                             for t in range(T)]))
    da = torch.einsum("ted,edf->tef", dy_all, w2)
    sg = torch.sigmoid(g)
    dg = rne_t(da * u * sg * (1 + g * (1 - sg)))
    du = rne_t(da * g * sg)
    dh = torch.cat([dg, du], dim=2)  # [T,E,2F]
    dxg = rne_t(torch.einsum("tej,ejd->ted", dh, w13.reshape(E, -1, w13.shape[-1])))
    dx = rne_t(torch.stack([sum(dxg[t, int(ids[t, k])] for k in range(K)) for t in range(T)]))
    mask = routed.double()[..., None]
    dw2 = rne_t(torch.einsum("ted,tef->edf", dy_all * mask, a * mask))
    dw13 = rne_t(torch.einsum("tej,td->ejd", dh * mask, x)).reshape(w13.shape)
    return dict(out=out.numpy(), dx=dx.numpy(), dw13=dw13.numpy(), dw2=dw2.numpy(),
                dscores=dsc.numpy())


@pytest.mark.parametrize("kw", [dict(), dict(T=20, D=128, F=64, E=4, K=2, seed=9)])
def test_bf16_mode_matches_dense_bf16_brute_force(kw):
    x, ids, s, w13, w2, dout = small_inputs(**kw)
    ref = dense_bf16_reference(x, ids, s, w13, w2, dout)
    got = oracle.full(x, ids, s, w13, w2, dout, mode="bf16")
    for k in ("out", "dx", "dw13", "dw2"):
        diff = np.abs(got[k] - ref[k])
        # identical up to a one-ulp flip where the two float64 summation orders straddle a
        # rounding boundary (expected to be vanishingly rare)
        assert (diff <= bf16_ulp(ref[k]) * 1.0001).all(), k
        assert (diff > 0).mean() < 1e-3, k
    np.testing.assert_allclose(got["dscores"], ref["dscores"], rtol=1e-12, atol=1e-12)


def test_bf16_mode_close_to_exact_evaluation():
    inp = W.make_inputs(W.PARITY_WORKLOADS["p_wide"].with_(T=64), router=oracle.route)
    b = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, mode="bf16")
    e = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, mode="exact")
    for k in ("out", "dx", "dw13", "dw2", "dscores"):
        err = np.abs(b[k] - e[k]).max() / max(1.0, np.abs(e[k]).max())
        assert err < 2e-2, (k, err)
        assert err > 0  # the rounding points are active


def test_dense_ffn_special_case_numpy_matmul():
    # E=1, K=1, score 1: the layer is a dense SwiGLU FFN; numpy matmul with the same rounding
    rng = np.random.default_rng(11)
    T, D, F = 16, 96, 80
    x = W.f32_to_bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    w13 = W.f32_to_bf16_bits((rng.standard_normal((1, 2, F, D)) / math.sqrt(D)).astype(np.float32))
    w2 = W.f32_to_bf16_bits((rng.standard_normal((1, D, F)) / math.sqrt(F)).astype(np.float32))
    ids = np.zeros((T, 1), np.int64)
    s = np.ones((T, 1), np.float32)
    got = oracle.full(x, ids, s, w13, w2, None, mode="bf16")["out"]
    X, A, B = as_f64(x), as_f64(w13)[0], as_f64(w2)[0]
    g = rne_t(X @ A[0].T).numpy()
    u = rne_t(X @ A[1].T).numpy()
    a = rne_t(g / (1 + np.exp(-g)) * u).numpy()
    y = rne_t(a @ B.T).numpy()
    diff = np.abs(got - y)
    assert (diff <= bf16_ulp(y) * 1.0001).all() and (diff > 0).mean() < 1e-3


# ------------------------------------------------------------------------------------------------
# algebraic invariants (bitwise)

def test_k1_unit_score_identity():
    x, ids, s, w13, w2, dout = small_inputs(K=1)
    s = np.ones_like(s)
    r = oracle.full(x, ids, s, w13, w2, dout)
    np.testing.assert_array_equal(r["out"], r["y"][r["pos"]])


def test_linearity_in_scores_and_dout():
    x, ids, s, w13, w2, dout = small_inputs(dup=True)
    r1 = oracle.full(x, ids, s, w13, w2, dout)
    r2 = oracle.full(x, ids, 2 * s, w13, w2, dout)
    np.testing.assert_array_equal(r2["out"], 2 * r1["out"])
    np.testing.assert_array_equal(r2["dscores"], r1["dscores"])  # dscore does not depend on s
    d2 = W.f32_to_bf16_bits(2 * W.bf16_bits_to_f32(dout))
    r3 = oracle.full(x, ids, s, w13, w2, d2)
    for k in ("dx", "dw13", "dw2", "dscores", "dy", "dh13"):
        np.testing.assert_array_equal(r3[k], 2 * r1[k], err_msg=k)


def test_zero_score_padding_changes_nothing():
    x, ids, s, w13, w2, dout = small_inputs(K=2)
    s0 = s.copy()
    s0[:, 1] = 0.0
    r = oracle.full(x, ids, s0, w13, w2, dout)
    r1 = oracle.full(x, ids[:, :1], s[:, :1], w13, w2, dout)
    np.testing.assert_array_equal(r["out"], r1["out"])
    np.testing.assert_array_equal(r["dx"], r1["dx"])
    np.testing.assert_array_equal(r["dscores"][:, 0], r1["dscores"][:, 0])
    # a padded token (all scores 0) contributes exactly zero everywhere but its own dscores
    s0[4] = 0.0
    r = oracle.full(x, ids, s0, w13, w2, dout)
    assert (r["out"][4] == 0).all() and (r["dx"][4] == 0).all()
    assert (r["dscores"][4] != 0).all()


def test_token_permutation_equivariance():
    x, ids, s, w13, w2, dout = small_inputs(T=16, dup=True)
    perm = np.random.default_rng(2).permutation(16)
    r = oracle.full(x, ids, s, w13, w2, dout)
    rp = oracle.full(x[perm], ids[perm], s[perm], w13, w2, dout[perm])
    for k in ("out", "dx", "dscores"):
        np.testing.assert_array_equal(rp[k], r[k][perm], err_msg=k)
    for k in ("dw13", "dw2"):
        assert (np.abs(rp[k] - r[k]) <= bf16_ulp(r[k]) * 1.0001).all()


def test_dscore_equals_dout_dot_onehot_output():
    x, ids, s, w13, w2, dout = small_inputs()
    r = oracle.full(x, ids, s, w13, w2, dout)
    T, K = ids.shape
    for k in range(K):
        oh = np.zeros_like(s)
        oh[:, k] = 1.0
        out_k = oracle.full(x, ids, oh, w13, w2, None)["out"]
        np.testing.assert_array_equal(r["dscores"][:, k], (as_f64(dout) * out_k).sum(1))


def test_empty_expert_weight_grads_are_zero():
    x, ids, s, w13, w2, dout = small_inputs(E=6)
    ids[ids == 5] = 0  # expert 5 receives nothing (duplicates are legal)
    r = oracle.full(x, ids, s, w13, w2, dout)
    assert r["counts"][5] == 0
    assert (r["dw13"][5] == 0).all() and (r["dw2"][5] == 0).all()
    assert (r["dw13"][0] != 0).any()


# ------------------------------------------------------------------------------------------------
# the sampled entry points agree with the full evaluation

def test_sampled_functions_agree_with_full():
    w = W.PARITY_WORKLOADS["p_skew"].with_(T=60)
    inp = W.make_inputs(w)
    full = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, scales=True)
    toks = np.array([0, 7, 59])
    tk = oracle.tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, toks, inp.dout, want_y=True)
    np.testing.assert_array_equal(tk["out"], full["out"][toks])
    np.testing.assert_array_equal(tk["dx"], full["dx"][toks])
    np.testing.assert_array_equal(tk["dscores"], full["dscores"][toks])
    np.testing.assert_array_equal(tk["y"][1, 1], full["y"][full["pos"][7 * w.K + 1]])
    jd = W.sample_pairs(2 * w.F, w.D, 40, 1, 1)
    df = W.sample_pairs(w.D, w.F, 40, 1, 2)
    for e in (0, 3):
        v13, v2, r13, r2 = oracle.wgrad_entries(inp.x, inp.ids, inp.scores, inp.w13, inp.w2,
                                                inp.dout, e, jd, df, scales=True)
        np.testing.assert_array_equal(v13, full["dw13"][e].reshape(2 * w.F, w.D)[jd[:, 0], jd[:, 1]])
        np.testing.assert_array_equal(v2, full["dw2"][e][df[:, 0], df[:, 1]])
        # the per-entry root-sum-square of terms: the same terms in the same order as the
        # whole-layer evaluation
        np.testing.assert_allclose(
            r13, full["dw13_rss"][e].reshape(2 * w.F, w.D)[jd[:, 0], jd[:, 1]], rtol=1e-13, atol=0)
        np.testing.assert_allclose(r2, full["dw2_rss"][e][df[:, 0], df[:, 1]], rtol=1e-13, atol=0)


# ------------------------------------------------------------------------------------------------
# weight gradients kept in fp32, and accumulation into existing gradients (Dist-MoE, "In-place
# WGRAD accumulation": BF16 or FP32 gradient storage, the same dtype for W13 and W2)

def _bf16_values(a):
    return np.array([oracle.round_bf16(float(v)) for v in np.ravel(a)]).reshape(np.shape(a))


def test_wgrad_storage_modes_are_one_rounding_apart():
    x, ids, s, w13, w2, dout = small_inputs(E=6)
    ids[ids == 5] = 0  # expert 5 has no rows
    ov = oracle.full(x, ids, s, w13, w2, dout)
    f32 = oracle.full(x, ids, s, w13, w2, dout, wgrad_f32=True)
    # the fp32 storage keeps the sum unrounded; rounding it gives the bf16 storage bit for bit
    for k in ("dw13", "dw2"):
        np.testing.assert_array_equal(_bf16_values(f32[k]), ov[k])
        assert (f32[k] != ov[k]).mean() > 0.5  # most sums are not bf16 values
    # nothing else changes
    for k in ("out", "dx", "dscores", "dh13"):
        np.testing.assert_array_equal(f32[k], ov[k])
    rng = np.random.default_rng(9)
    i13 = _bf16_values(rng.standard_normal(ov["dw13"].shape) * 0.1)
    i2 = _bf16_values(rng.standard_normal(ov["dw2"].shape) * 0.1)
    # accumulating onto zeros is the overwrite
    z = oracle.full(x, ids, s, w13, w2, dout, dw13_init=np.zeros_like(i13), dw2_init=np.zeros_like(i2))
    for k in ("dw13", "dw2"):
        np.testing.assert_array_equal(z[k], ov[k])
    # bf16 accumulation rounds once, after adding the unrounded contribution to the old value
    acc = oracle.full(x, ids, s, w13, w2, dout, dw13_init=i13, dw2_init=i2)
    for k, init in (("dw13", i13), ("dw2", i2)):
        np.testing.assert_array_equal(acc[k], _bf16_values(init + f32[k]))
        double_rounded = _bf16_values(init + ov[k])
        assert (acc[k] != double_rounded).any()  # a second rounding would be visible
    # an expert without rows keeps its old gradient
    np.testing.assert_array_equal(acc["dw13"][5], i13[5])
    np.testing.assert_array_equal(acc["dw2"][5], i2[5])
    # fp32 accumulation twice adds the contribution twice
    a1 = oracle.full(x, ids, s, w13, w2, dout, wgrad_f32=True, dw13_init=i13, dw2_init=i2)
    a2 = oracle.full(x, ids, s, w13, w2, dout, wgrad_f32=True, dw13_init=a1["dw13"], dw2_init=a1["dw2"])
    for k, init in (("dw13", i13), ("dw2", i2)):
        np.testing.assert_allclose(a2[k], init + 2 * f32[k], rtol=0, atol=1e-12)


def test_sampled_wgrad_entries_follow_the_storage_mode():
    w = W.PARITY_WORKLOADS["p_skew"].with_(T=60)
    inp = W.make_inputs(w)
    full = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, wgrad_f32=True)
    e = int(np.argmax(full["counts"]))
    jd = np.array([[0, 0], [w.F + 3, 17], [2 * w.F - 1, w.D - 1]])
    df = np.array([[1, 2], [w.D - 1, w.F - 1]])
    i13 = np.array([0.25, -1.5, 3.0])
    i2 = np.array([0.125, 7.0])
    v13, v2 = oracle.wgrad_entries(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, e, jd, df,
                                   wgrad_f32=True, init13=i13, init2=i2)
    np.testing.assert_allclose(v13, i13 + full["dw13"][e].reshape(2 * w.F, w.D)[jd[:, 0], jd[:, 1]],
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(v2, i2 + full["dw2"][e][df[:, 0], df[:, 1]], rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# whole weight gradients of one expert (the large-workload check of 4 experts' gradients)

@pytest.mark.parametrize("name", ["p_skew", "p_ragged"])
def test_expert_wgrad_is_the_full_evaluation(name):
    """Every expert, the empty one included: bitwise the full evaluation's dW13[e], dW2[e] (bf16
    storage); in fp32 storage and with accumulation onto existing gradients to the last bits of a
    double; the root-sum-square scales to the last bits of a double."""
    w = W.PARITY_WORKLOADS[name]
    inp = W.make_inputs(w, router=oracle.route)
    full = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, scales=True)
    rng = np.random.default_rng(3)
    i13 = _bf16_values(rng.standard_normal(full["dw13"].shape) * 0.1)
    i2 = _bf16_values(rng.standard_normal(full["dw2"].shape) * 0.1)
    f32 = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, wgrad_f32=True,
                      dw13_init=i13, dw2_init=i2)
    acc = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, dw13_init=i13,
                      dw2_init=i2)
    if name == "p_skew":
        assert (full["counts"] == 0).any()
    for e in range(w.E):
        r = oracle.expert_wgrad(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, e,
                                scales=True)
        np.testing.assert_array_equal(r["dw13"], full["dw13"][e])
        np.testing.assert_array_equal(r["dw2"], full["dw2"][e])
        for k in ("dw13_rss", "dw2_rss"):
            np.testing.assert_allclose(r[k], full[k][e], rtol=1e-13, atol=0)
        if full["counts"][e] == 0:
            assert (r["dw13"] == 0).all() and (r["dw2"] == 0).all()
        ra = oracle.expert_wgrad(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, e,
                                 init13=i13[e], init2=i2[e])
        np.testing.assert_array_equal(ra["dw13"], acc["dw13"][e])
        np.testing.assert_array_equal(ra["dw2"], acc["dw2"][e])
        rf = oracle.expert_wgrad(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, e,
                                 wgrad_f32=True, init13=i13[e], init2=i2[e])
        np.testing.assert_allclose(rf["dw13"], f32["dw13"][e], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(rf["dw2"], f32["dw2"][e], rtol=1e-13, atol=1e-15)


def test_expert_wgrad_exact_mode_against_dense_autograd():
    """float64 inputs, no rounding: the whole expert gradients against the dense torch autograd
    brute force (every expert on every token, masked by the routing)."""
    x, ids, s, w13, w2, dout = small_inputs(f64=True, dup=True, bad=True)
    ref = dense_torch(x, ids, s, w13, w2, dout)
    for e in range(w13.shape[0]):
        r = oracle.expert_wgrad(x, ids, s, w13, w2, dout, e, mode="exact")
        np.testing.assert_allclose(r["dw13"], ref["dw13"][e], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(r["dw2"], ref["dw2"][e], rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# error scales: root-sum-square of a summed output's terms

def test_error_scales_single_term_is_the_magnitude():
    """A sum with one term: its root-sum-square is its magnitude (sqrt of a rounded square of a
    double returns the magnitude exactly). One routed row per expert gives dW terms of one row;
    K = 1 gives out and dx terms of one slot; a one-hot dout row gives one dscores term."""
    T, D, F, E = 5, 64, 48, 5
    x, _, s, w13, w2, dout = small_inputs(T=T, D=D, F=F, E=E, K=1, f64=True)
    ids = np.arange(T, dtype=np.int64).reshape(T, 1)  # every expert has exactly one row
    r = oracle.full(x, ids, s, w13, w2, dout, mode="exact", scales=True)
    for k in ("out", "dx", "dw13", "dw2"):
        np.testing.assert_array_equal(r[k + "_rss"], np.abs(r[k]))
    oh = np.zeros_like(dout)
    oh[np.arange(T), np.arange(T) * 3] = 1.5
    r = oracle.full(x, ids, s, w13, w2, oh, mode="exact", scales=True)
    np.testing.assert_array_equal(r["dscores_rss"], np.abs(r["dscores"]))
    tk = oracle.tokens(x, ids, s, w13, w2, np.arange(T), oh, mode="exact", scales=True)
    for k in ("out", "dscores", "dx"):
        np.testing.assert_array_equal(tk[k + "_rss"], r[k + "_rss"])


def test_error_scales_bound_the_sums_and_the_rounding_contract():
    """Cauchy-Schwarz: |sum of n terms| <= sqrt(n) * rss; the bf16 contract, which rounds every
    operand of every sum, stays within four bf16 ulps of the scale, 2^-5 * max(1, |exact|, rss),
    of the exact layer for every summed output (measured: at most 2.2e-2 of it for dW13 on this
    shape, 1.6e-2 for the others); scaling dout scales the backward's rss."""
    inp = W.make_inputs(W.PARITY_WORKLOADS["p_skew"], router=oracle.route)
    b = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, scales=True)
    e = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, mode="exact",
                    scales=True)
    w = inp.w
    n_dw = np.maximum(b["counts"], 1)[:, None, None]
    assert (np.abs(e["dw2"]) <= np.sqrt(n_dw) * e["dw2_rss"] * (1 + 1e-12)).all()
    assert (np.abs(e["dw13"]).reshape(w.E, 2 * w.F, w.D)
            <= np.sqrt(n_dw) * e["dw13_rss"].reshape(w.E, 2 * w.F, w.D) * (1 + 1e-12)).all()
    assert (np.abs(e["dscores"]) <= math.sqrt(w.D) * e["dscores_rss"] * (1 + 1e-12)).all()
    assert (np.abs(e["out"]) <= math.sqrt(w.K) * e["out_rss"] * (1 + 1e-12)).all()
    for k in ("out", "dx", "dscores", "dw13", "dw2"):
        tol = 2.0 ** -5 * np.maximum(np.maximum(1.0, np.abs(e[k])), e[k + "_rss"])
        assert (np.abs(b[k] - e[k]) <= tol).all(), k
    d2 = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, W.f32_to_bf16_bits(
        2 * W.bf16_bits_to_f32(inp.dout)), mode="exact", scales=True)
    for k in ("dscores_rss", "dx_rss", "dw13_rss", "dw2_rss"):
        np.testing.assert_allclose(d2[k], 2 * e[k], rtol=1e-12, atol=0)
