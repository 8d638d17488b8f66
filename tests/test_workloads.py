"""The seeded input generators: determinism, shapes and the routing rules' stated properties."""
import numpy as np
import pytest

import oracle
import workloads as W

ROUTER = oracle.route  # (logits, K) -> (ids, weights): softmax top-K, renormalised


def test_inputs_deterministic_and_shaped():
    w = W.PARITY_WORKLOADS["p_ragged"]
    a = W.make_inputs(w)
    b = W.make_inputs(w, ids_dtype=np.int32)
    assert a.x.shape == (w.T, w.D) and a.x.dtype == np.uint16
    assert a.w13.shape == (w.E, 2, w.F, w.D) and a.w2.shape == (w.E, w.D, w.F)
    assert a.ids.shape == (w.T, w.K) and a.scores.dtype == np.float32
    assert b.ids.dtype == np.int32
    for k in ("x", "w13", "w2", "dout", "scores"):
        np.testing.assert_array_equal(getattr(a, k), getattr(b, k))
    np.testing.assert_array_equal(a.ids, b.ids)


def test_block_streams_do_not_depend_on_thread_count(monkeypatch):
    a = W.normal_bf16(3, 99, (3 * W.BLOCK // 1024 + 5, 1024), 0.5)
    monkeypatch.setattr(W, "_pool_size", lambda: 1)
    b = W.normal_bf16(3, 99, (3 * W.BLOCK // 1024 + 5, 1024), 0.5)
    np.testing.assert_array_equal(a, b)
    v = W.bf16_bits_to_f32(a)
    assert abs(v.std() - 0.5) < 0.01 and abs(v.mean()) < 0.01


def test_weight_scale_is_inverse_sqrt_fan_in():
    inp = W.make_inputs(W.PARITY_WORKLOADS["p_wide"], router=ROUTER)
    w = inp.w
    assert abs(W.bf16_bits_to_f32(inp.w13).std() * np.sqrt(w.D) - 1) < 0.02
    assert abs(W.bf16_bits_to_f32(inp.w2).std() * np.sqrt(w.F) - 1) < 0.02


def test_routing_rules():
    # even: closed form, scores 1/K
    w = W.WORKLOADS["tiny"]
    ids, s = W.routing(w)
    t = np.arange(w.T)[:, None]
    k = np.arange(w.K)[None, :]
    np.testing.assert_array_equal(ids, (t * w.K + k) % w.E)
    assert (s == 0.5).all()
    # top-k of softmax (routed by the oracle's router): ids distinct, scores renormalised and
    # descending; without a router the generator refuses
    for name in ("fine_grained", "training"):
        w = W.WORKLOADS[name]
        with pytest.raises(ValueError):
            W.routing(w)
        ids, s = W.routing(w, router=ROUTER)
        assert W.router_logits(w).shape == (w.T, w.E)
        assert ids.shape == (w.T, w.K)
        srt = np.sort(ids, 1)
        assert (srt[:, 1:] != srt[:, :-1]).all()
        np.testing.assert_allclose(s.sum(1), 1, rtol=1e-5)
        assert (np.diff(s, axis=1) <= 1e-7).all()
    # balanced uniform: distinct ids, counts near T*K/E
    w = W.WORKLOADS["large_hidden"]
    ids, s = W.routing(w)
    srt = np.sort(ids, 1)
    assert (srt[:, 1:] != srt[:, :-1]).all()
    c = np.bincount(ids.ravel(), minlength=w.E)
    assert c.sum() == w.N and abs(c.max() / c.mean() - 1) < 0.1
    # imbalanced: exact peak/mean 3.0, Zipf tail, distinct ids per token
    w = W.WORKLOADS["imbalanced"]
    ids, _ = W.routing(w)
    c = np.sort(np.bincount(ids.ravel(), minlength=w.E))[::-1]
    assert c[0] == 6144 and c.sum() == w.N and list(c[1:4]) == [4446, 3680, 3217]
    assert list(c[-2:]) == [1237, 1219]
    srt = np.sort(ids, 1)
    assert (srt[:, 1:] != srt[:, :-1]).all()


def test_samples():
    s = W.sample_tokens(8192, 256)
    assert len(np.unique(s)) == 256 and (np.diff(s) > 0).all()
    np.testing.assert_array_equal(W.sample_tokens(10, 256), np.arange(10))
    p = W.sample_pairs(100, 7, 50, 1, 3)
    assert p.shape == (50, 2) and p[:, 0].max() < 100 and p[:, 1].max() < 7
