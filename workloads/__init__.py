"""Seeded synthetic inputs for the routed-experts layer.

This module only draws random numbers and shapes them into the arrays the layer consumes:
``x[T,D]``, ``w13[E,2,F,D]``, ``w2[E,D,F]`` and ``dout[T,D]`` as bf16 bit patterns (uint16),
``topk_ids[T,K]`` (int32 or int64) and ``topk_scores[T,K]`` (float32). It holds none of the layer's
arithmetic. Both the CPU oracle and the GPU path read the bytes produced here.

Recipe (every config):

* Every random tensor has its own stream family: ``SeedSequence([seed, TAG])`` spawns one PCG64
  stream per fixed block of ``BLOCK`` elements of the flattened tensor, so the values do not depend on
  how many threads fill them.
* Dense tensors: float32 standard normal, scaled by ``std`` in float32, then rounded to bf16
  (round-to-nearest-even). ``x`` and ``dout`` use std 1; ``w13`` uses 1/sqrt(D) and ``w2`` uses
  1/sqrt(F) (std = 1/sqrt(fan_in), fan_in being the contracted width).
* Routing follows the workload's rule (see ``ROUTINGS``); scores are float32. Logit-routed
  workloads (``LOGIT_ROUTINGS``) draw only the router logits here (``router_logits``); their ids
  and scores come from a router the caller passes in (the GPU router, or the oracle's in tests).

The workloads are the five shapes the pages' systems run at one GPU's share (Dist-MoE quickstart
shape; a fine-grained 64-expert shard; a 7168-hidden expert-parallel shard, balanced and at
peak-to-mean load 3.0; a 16-expert training shard) plus small parity shapes.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

BLOCK = 1 << 22  # elements per independent stream block

# tags that separate the stream families of one seed
TAG_X, TAG_W13, TAG_W2, TAG_ROUTE, TAG_SCORES, TAG_DOUT = 11, 12, 13, 14, 15, 16


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    D: int
    F: int
    E: int
    K: int
    routing: str  # key of ROUTINGS
    backward: bool  # whether the workload runs the backward pass (draws dout)
    seed: int = 0
    description: str = ""
    extra: dict = field(default_factory=dict, hash=False, compare=False)

    @property
    def N(self) -> int:
        return self.T * self.K

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def flops_forward(self) -> int:
        """Algorithmic forward FLOPs: 4NDF for the gate/up GEMM plus 2NDF for the down GEMM."""
        return 6 * self.N * self.D * self.F

    def flops_backward(self) -> int:
        """Algorithmic backward FLOPs: DGRAD2 2NDF, WGRAD2 2NDF, DGRAD1 4NDF, WGRAD1 4NDF."""
        return 12 * self.N * self.D * self.F


WORKLOADS = {
    "tiny": Workload(
        "tiny", T=16, D=256, F=256, E=8, K=2, routing="even", backward=True,
        description="Dist-MoE BF16 quickstart shape (T=16, D=F=256, K=2, 8 experts), "
                    "round-robin ids (t*K+k) mod E, scores 1/K"),
    "fine_grained": Workload(
        "fine_grained", T=4096, D=2048, F=1408, E=64, K=6, routing="topk_softmax", backward=False,
        description="fine-grained shard: 64 experts, top-6 of softmax(N(0,1) logits)"),
    "large_hidden": Workload(
        "large_hidden", T=8192, D=7168, F=2048, E=32, K=8, routing="uniform_distinct",
        backward=False,
        description="7168-hidden expert-parallel shard: 8192 received tokens, 32 local experts, "
                    "8 distinct uniform-random ids per token"),
    "imbalanced": Workload(
        "imbalanced", T=8192, D=7168, F=2048, E=32, K=8, routing="zipf_peak3", backward=True,
        description="7168-hidden shard at expert-load peak-to-mean 3.0 (one expert at 3x mean, "
                    "the rest Zipf-decaying), distinct ids per token"),
    "training": Workload(
        "training", T=16384, D=4096, F=1536, E=16, K=8, routing="topk_softmax", backward=True,
        description="training shard: 16 experts, top-8 of softmax(N(0,1) logits)"),
}

# Small shapes for element-by-element parity: several 256-row tiles per expert, ragged tails,
# an intermediate width that is not a multiple of 128, duplicates/empty experts.
PARITY_WORKLOADS = {
    "p_ragged": Workload("p_ragged", T=700, D=512, F=320, E=6, K=3, routing="uniform_distinct",
                         backward=True, seed=3),
    "p_skew": Workload("p_skew", T=600, D=256, F=192, E=8, K=2, routing="skewed", backward=True,
                       seed=4),
    "p_wide": Workload("p_wide", T=256, D=1024, F=512, E=4, K=4, routing="topk_softmax",
                       backward=True, seed=5),
}


# ----------------------------------------------------------------------------------------------
# dense draws

def _pool_size() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even) and return the 16-bit patterns (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).copy()
    tmp = u >> 16
    tmp &= 1
    tmp += 0x7FFF
    u += tmp
    u >>= 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed: int, tag: int, shape, std: float) -> np.ndarray:
    """bf16 bits of std * N(0,1), block-parallel and thread-count independent."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nblk = (n + BLOCK - 1) // BLOCK
    seqs = np.random.SeedSequence([seed, tag]).spawn(nblk)
    std32 = np.float32(std)

    def fill(b):
        lo = b * BLOCK
        hi = min(n, lo + BLOCK)
        g = np.random.Generator(np.random.PCG64(seqs[b]))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if std32 != np.float32(1.0):
            v *= std32
        out[lo:hi] = f32_to_bf16_bits(v)

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_pool_size()) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


# ----------------------------------------------------------------------------------------------
# routing rules

def _softmax_rows(v: np.ndarray) -> np.ndarray:
    v = v.astype(np.float64)
    v = v - v.max(axis=1, keepdims=True)
    ex = np.exp(v)
    return (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)


def _route_even(w: Workload, rng):
    # Primus "even" forced balancing and the Dist-MoE quickstart: (token*K + k) mod E
    t = np.arange(w.T, dtype=np.int64)[:, None]
    k = np.arange(w.K, dtype=np.int64)[None, :]
    ids = (t * w.K + k) % w.E
    scores = np.full((w.T, w.K), 1.0 / w.K, dtype=np.float32)
    return ids, scores


def _logits(w: Workload, rng):
    # router logits ~ N(0,1) (Primus "uniform" forced balancing: random logits, then routing)
    return rng.standard_normal((w.T, w.E), dtype=np.float32)


def _route_uniform_distinct(w: Workload, rng):
    # per token the first K entries of a seeded permutation of [0, E)
    perm = rng.permuted(np.tile(np.arange(w.E, dtype=np.int64), (w.T, 1)), axis=1)
    ids = perm[:, : w.K].copy()
    scores = _softmax_rows(rng.standard_normal((w.T, w.K), dtype=np.float32))
    return ids, scores


def zipf_peak_counts(total: int, n_experts: int, peak_to_mean: float):
    """Per-expert counts with the hottest at peak_to_mean x mean and a rank^-alpha law.

    alpha solves  n_experts / sum_r r^-alpha = peak_to_mean  (the same law over all ranks gives the
    requested peak/mean); the hottest count is fixed at peak_to_mean * mean and the remaining
    tokens are split over ranks 2..E in proportion to r^-alpha, rounded by largest remainder.
    Returns (counts by rank, alpha).
    """
    r = np.arange(1, n_experts + 1, dtype=np.float64)

    def ratio(a):
        return n_experts / np.sum(r ** -a)

    lo, hi = 0.0, 8.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if ratio(mid) < peak_to_mean:
            lo = mid
        else:
            hi = mid
    alpha = 0.5 * (lo + hi)
    hot = int(round(peak_to_mean * total / n_experts))
    rest = total - hot
    wts = r[1:] ** -alpha
    real = rest * wts / wts.sum()
    base = np.floor(real).astype(np.int64)
    short = rest - int(base.sum())
    frac_order = np.argsort(-(real - base), kind="stable")
    base[frac_order[:short]] += 1
    return np.concatenate([[hot], base]).astype(np.int64), alpha


def _route_zipf_peak3(w: Workload, rng):
    counts, _ = zipf_peak_counts(w.N, w.E, 3.0)
    if counts.max() > w.T:
        raise ValueError("a count above T cannot keep ids distinct per token")
    by_slot = np.repeat(np.arange(w.E, dtype=np.int64), counts)  # expert rank per slot j
    j = np.arange(w.N)
    ids = np.empty((w.T, w.K), dtype=np.int64)
    ids[j % w.T, j // w.T] = by_slot
    label = rng.permutation(w.E)  # rank -> expert label
    ids = label[ids]
    ids = ids[rng.permutation(w.T)]
    ids = rng.permuted(ids, axis=1)
    scores = _softmax_rows(rng.standard_normal((w.T, w.K), dtype=np.float32))
    return ids, scores


def _route_skewed(w: Workload, rng):
    # ragged, lopsided loads with duplicates allowed: expert e drawn with probability ~ 2^-e,
    # the last expert never chosen (an empty expert); scores are arbitrary positive weights
    p = 0.5 ** np.arange(w.E - 1, dtype=np.float64)
    p /= p.sum()
    ids = rng.choice(w.E - 1, size=(w.T, w.K), p=p).astype(np.int64)
    scores = rng.uniform(0.0, 1.0, size=(w.T, w.K)).astype(np.float32)
    return ids, scores


ROUTINGS = {
    "even": _route_even,
    "uniform_distinct": _route_uniform_distinct,
    "zipf_peak3": _route_zipf_peak3,
    "skewed": _route_skewed,
}


# routing rules that start from router logits: the ids and scores come from a router (softmax
# top-K, renormalised over the K chosen) that the caller supplies
LOGIT_ROUTINGS = ("topk_softmax",)


def router_logits(w: Workload) -> np.ndarray:
    """fp32 router logits [T,E] of a logit-routed workload."""
    if w.routing not in LOGIT_ROUTINGS:
        raise ValueError("workload %s is not routed from logits" % w.name)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, TAG_ROUTE])))
    return np.ascontiguousarray(_logits(w, rng))


def routing(w: Workload, ids_dtype=np.int64, router=None):
    """(ids [T,K], scores [T,K] fp32). For logit-routed workloads ``router(logits, K)`` must be
    given and returns (ids, weights) of the softmax top-K router, renormalised over the K chosen."""
    if w.routing in LOGIT_ROUTINGS:
        if router is None:
            raise ValueError("workload %s is routed from logits: pass a router" % w.name)
        ids, scores = router(router_logits(w), w.K)
    else:
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, TAG_ROUTE])))
        ids, scores = ROUTINGS[w.routing](w, rng)
    ids = np.asarray(ids)
    scores = np.asarray(scores)
    return np.ascontiguousarray(ids.astype(ids_dtype)), np.ascontiguousarray(scores, dtype=np.float32)


@dataclass
class Inputs:
    w: Workload
    x: np.ndarray  # [T,D] uint16 (bf16 bits)
    w13: np.ndarray  # [E,2,F,D] uint16
    w2: np.ndarray  # [E,D,F] uint16
    ids: np.ndarray  # [T,K] int32/int64
    scores: np.ndarray  # [T,K] float32
    dout: np.ndarray | None  # [T,D] uint16 or None


def make_inputs(w: Workload, ids_dtype=np.int64, with_dout: bool | None = None,
                router=None) -> Inputs:
    """Draw every input of workload ``w`` (deterministic in ``w.seed``); ``router`` as in
    ``routing`` for logit-routed workloads."""
    if with_dout is None:
        with_dout = w.backward
    x = normal_bf16(w.seed, TAG_X, (w.T, w.D), 1.0)
    w13 = normal_bf16(w.seed, TAG_W13, (w.E, 2, w.F, w.D), 1.0 / math.sqrt(w.D))
    w2 = normal_bf16(w.seed, TAG_W2, (w.E, w.D, w.F), 1.0 / math.sqrt(w.F))
    ids, scores = routing(w, ids_dtype, router)
    dout = normal_bf16(w.seed, TAG_DOUT, (w.T, w.D), 1.0) if with_dout else None
    return Inputs(w, x, w13, w2, ids, scores, dout)


def sample_tokens(T: int, n: int, seed: int = 1) -> np.ndarray:
    """Sorted seeded sample of n distinct token indices (all of them when n >= T)."""
    if n >= T:
        return np.arange(T, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 21])))
    return np.sort(rng.choice(T, size=n, replace=False)).astype(np.int64)


def sample_pairs(rows: int, cols: int, n: int, seed: int, tag: int) -> np.ndarray:
    """n seeded (row, col) index pairs, shape [n,2] int64."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag])))
    return np.stack([rng.integers(0, rows, n), rng.integers(0, cols, n)], axis=1).astype(np.int64)
