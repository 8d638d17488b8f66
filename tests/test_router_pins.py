"""Pins of the oracle's router (score function + group-limited top-k) to things other than itself:
a hand-worked example, numpy/scipy library routines on the same inputs, and invariants.

The pages (MegaMoE, introduction) name the router's parts without formulas; the readings the
oracle takes are stated in its router section. Sorting (numpy stable argsort / lexsort) and
scipy's softmax/expit stand in here as independent evaluations of those readings."""
import os

import numpy as np
import pytest
from scipy import special

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "router_group_example.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        vals[k.strip()] = v.split()
    return vals


def test_hand_worked_group_example():
    g = _golden()
    logits = np.array([[float(v) for v in g["logits"]]], np.float32)
    ids, w = oracle.route(logits, int(g["K"][0]), n_group=int(g["n_group"][0]),
                          topk_group=int(g["topk_group"][0]))
    assert ids[0].tolist() == [int(v) for v in g["ids"]]
    np.testing.assert_allclose(w[0], [float(v) for v in g["weights"]], rtol=0, atol=1e-15)


def _tied_logits(T, E, seed):
    rng = np.random.default_rng(seed)
    # quarter steps: many exact ties between experts of one token
    return (np.round(rng.standard_normal((T, E)) * 4) / 4).astype(np.float32)


@pytest.mark.parametrize("T,E,K", [(64, 8, 2), (50, 64, 6), (40, 16, 8), (9, 300, 17), (5, 13, 13)])
def test_topk_matches_stable_sort(T, E, K):
    logits = _tied_logits(T, E, T * 1000 + E)
    ids, _ = oracle.route(logits, K)
    ref = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :K]
    np.testing.assert_array_equal(ids, ref)


@pytest.mark.parametrize("renorm", [True, False])
def test_softmax_weights_match_scipy(renorm):
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((33, 24)).astype(np.float32)
    ids, w = oracle.route(logits, 5, renormalize=renorm)
    l64 = logits.astype(np.float64)
    if renorm:
        ref = special.softmax(np.take_along_axis(l64, ids, axis=1), axis=1)
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    else:
        ref = np.take_along_axis(special.softmax(l64, axis=1), ids, axis=1)
    np.testing.assert_allclose(w, ref, rtol=1e-13, atol=0)


@pytest.mark.parametrize("renorm", [True, False])
def test_sigmoid_weights_match_scipy(renorm):
    rng = np.random.default_rng(4)
    logits = (rng.standard_normal((21, 40)) * 3).astype(np.float32)
    ids, w = oracle.route(logits, 7, score_fn=oracle.SCORE_SIGMOID, renormalize=renorm)
    # sigmoid is increasing, so the choice is the same as softmax's
    ids_soft, _ = oracle.route(logits, 7)
    np.testing.assert_array_equal(ids, ids_soft)
    s = special.expit(np.take_along_axis(logits.astype(np.float64), ids, axis=1))
    ref = s / s.sum(axis=1, keepdims=True) if renorm else s
    np.testing.assert_allclose(w, ref, rtol=1e-13, atol=0)


@pytest.mark.parametrize("E,G,TG,K", [(16, 4, 2, 3), (64, 8, 3, 8), (256, 8, 4, 8), (12, 6, 1, 2)])
def test_group_limited_matches_sorts(E, G, TG, K):
    logits = _tied_logits(47, E, E * 7 + G)
    ids, _ = oracle.route(logits, K, n_group=G, topk_group=TG)
    gs = E // G
    l64 = logits.astype(np.float64)
    for t in range(logits.shape[0]):
        grp = l64[t].reshape(G, gs)
        gbest = grp.max(axis=1)
        kept = np.lexsort((np.arange(G), -gbest))[:TG]  # by best logit, then lower group
        masked = np.full(E, -np.inf)
        for g in kept:
            masked[g * gs:(g + 1) * gs] = l64[t, g * gs:(g + 1) * gs]
        ref = np.argsort(-masked, kind="stable")[:K]
        assert ids[t].tolist() == ref.tolist(), t


def test_all_groups_kept_equals_plain_topk():
    logits = _tied_logits(30, 32, 11)
    a, wa = oracle.route(logits, 6, n_group=4, topk_group=4)
    b, wb = oracle.route(logits, 6)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(wa, wb)


def test_shift_invariance_of_softmax_router():
    rng = np.random.default_rng(5)
    # multiples of 2^-10 below 4 in magnitude: adding 8 is exact in fp32
    logits = (np.round(rng.standard_normal((25, 20)) * 0.5 * 1024) / 1024).clip(-3.9, 3.9)
    logits = logits.astype(np.float32)
    shifted = (logits + np.float32(8.0)).astype(np.float32)
    assert np.array_equal(shifted - np.float32(8.0), logits)
    a, wa = oracle.route(logits, 4, renormalize=False)
    b, wb = oracle.route(shifted, 4, renormalize=False)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_allclose(wa, wb, rtol=1e-12, atol=0)


def test_k_equals_e_is_a_full_descending_sort():
    logits = _tied_logits(10, 9, 2)
    ids, w = oracle.route(logits, 9)
    np.testing.assert_array_equal(ids, np.argsort(-logits.astype(np.float64), axis=1, kind="stable"))
    np.testing.assert_allclose(w, np.take_along_axis(special.softmax(logits.astype(np.float64), axis=1), ids, axis=1),
                               rtol=1e-13)


def test_nan_logits_rank_last():
    logits = np.array([[np.nan, 1.0, np.nan, -5.0, 0.0]], np.float32)
    ids, _ = oracle.route(logits, 4)
    assert ids[0].tolist() == [1, 4, 3, 0]


def test_bad_configurations_rejected():
    logits = np.zeros((2, 8), np.float32)
    for kw in [dict(K=9), dict(K=3, n_group=3, topk_group=1), dict(K=5, n_group=4, topk_group=2),
               dict(K=2, n_group=4, topk_group=5)]:
        K = kw.pop("K")
        with pytest.raises(ValueError):
            oracle.route(logits, K, **kw)
