"""GPU parity at the edges of the address ranges the library accepts (the shape limits of the C
ABI's header), in the launch configuration of the timed path.

* One expert's gate/up block of exactly 4 GiB (4*F*D = 2^32 bytes, F = D = 32768) with two
  experts: expert 1's weights and weight gradients start 4 GiB (w13, dW13) and 2 GiB (w2, dW2)
  into their buffers, and the GEMM copies take 32-bit offsets from the expert's base up to the
  last byte of the block. Checked: out, dscores and dx on sampled tokens (every token visits
  both experts), and dW13 / dW2 entries of both experts at the corners of each block and at
  seeded positions.
* x just under 4 GiB (T*D*2 = 2^32 - 4096 bytes): the gate/up GEMM gathers the token rows
  itself with 32-bit offsets up to the end of x; and x of exactly 4 GiB, where the forward keeps
  the gathered rows instead. Checked: out, dscores, dx on sampled tokens including the last,
  and dW entries of three experts.
* The plan at the largest slot count accepted (T*K = 2^31 - 2^16 slots: T = 2^25 - 1024, K = 64,
  1024 experts, int32 ids): counts, offsets, pos and src bit-exact. At this size the stable
  grouping is checked through the properties that determine it uniquely (a full stable argsort
  of 2^31 ids would take the oracle minutes): counts = the histogram of the ids, offsets = their
  exclusive prefix sum, every grouped row r of segment e holds a slot src[r] routed to e, src
  increases within each segment (stability), and pos[src[r]] = r for every r (src is the
  inverse permutation of pos).

The bar for floating outputs is the elementwise one of every GPU parity test (parity_check).
Inputs are the seeded draws of the workloads module at these shapes; the slot-limit ids are
seeded uniform draws.
"""
import gc
import time

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_check import check, log

pytestmark = pytest.mark.gpu


def _lib():
    from mixture_experts_routed_plan_amd import device as dv
    return dv


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()


def _rows_f64(dv, t, idx):
    """Rows idx of a bf16 device tensor, as float64 on the host (no full-size copy)."""
    sel = t[torch.as_tensor(idx, device=t.device)]
    return dv.bits_to_f64(dv.to_host_bits(sel))


def _entries_f64(dv, t, idx):
    """Entries of a bf16 device tensor at the index tuple idx (host arrays), as float64."""
    sel = t[tuple(torch.as_tensor(i, device=t.device) for i in idx)]
    return dv.bits_to_f64(dv.to_host_bits(sel))


def _run_and_check(w, toks, experts, jd, df):
    dv = _lib()
    t0 = time.time()
    inp = W.make_inputs(w, with_dout=True)
    log("\n[%s] T=%d D=%d F=%d E=%d K=%d: inputs drawn in %.1fs"
        % (w.name, w.T, w.D, w.F, w.E, w.K, time.time() - t0))
    d = dict(x=dv.to_device_bits(inp.x), w13=dv.to_device_bits(inp.w13),
             w2=dv.to_device_bits(inp.w2), dout=dv.to_device_bits(inp.dout),
             ids=torch.from_numpy(inp.ids).cuda(), scores=torch.from_numpy(inp.scores).cuda())
    layer = dv.Layer(w.T, w.D, w.F, w.E, w.K)
    log("[%s] device buffers: %.1f GiB" % (w.name, torch.cuda.memory_allocated() / 2**30))
    layer.plan(d["ids"])
    layer.forward(d["x"], d["scores"], d["w13"], d["w2"])
    layer.backward(d["dout"], d["scores"], d["w13"], d["w2"])
    torch.cuda.synchronize()
    st, bad = layer.plan_status()
    assert bad == 0
    log("[%s] gpu forward+backward done" % w.name)

    t0 = time.time()
    ref = oracle.tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, toks, inp.dout, scales=True)
    log("[%s] oracle on %d tokens: %.1fs" % (w.name, len(toks), time.time() - t0))
    check("out", _rows_f64(dv, layer.out, toks), ref["out"])
    check("dscores", layer.dscores[torch.as_tensor(toks).cuda()].cpu().numpy(), ref["dscores"],
          ref["dscores_rss"])
    check("dx", _rows_f64(dv, layer.dx, toks), ref["dx"])

    dw13 = layer.dw13.view(w.E, 2 * w.F, w.D)
    for e in experts:
        t0 = time.time()
        v13, v2, r13, r2 = oracle.wgrad_entries(inp.x, inp.ids, inp.scores, inp.w13, inp.w2,
                                                inp.dout, e, jd, df, scales=True)
        log("[%s] expert %d: oracle weight-gradient entries %.1fs" % (w.name, e, time.time() - t0))
        ev13 = np.full(len(jd), e)
        ev2 = np.full(len(df), e)
        check("dW13", _entries_f64(dv, dw13, (ev13, jd[:, 0], jd[:, 1])), v13, r13)
        check("dW2", _entries_f64(dv, layer.dw2, (ev2, df[:, 0], df[:, 1])), v2, r2)
    del layer, d, inp
    gc.collect()
    torch.cuda.empty_cache()


def _corners_and_seeded(rows, cols, n, seed, tag):
    corners = np.array([[0, 0], [0, cols - 1], [rows - 1, 0], [rows - 1, cols - 1],
                        [rows // 2, cols // 2]], dtype=np.int64)
    return np.concatenate([corners, W.sample_pairs(rows, cols, n, seed, tag)])


def test_expert_gate_up_block_of_4_gib():
    D = F = 32768
    assert 4 * F * D == 2**32
    w = W.Workload("limit_expert_block", T=96, D=D, F=F, E=2, K=2, routing="uniform_distinct",
                   backward=True, seed=11)
    toks = np.array([0, 1, 47, 95], dtype=np.int64)
    # the j (row of the gate/up block) values also name the intermediate columns the oracle
    # evaluates: keep their number small
    jd = _corners_and_seeded(2 * F, D, 6, 11, 1)
    df = _corners_and_seeded(D, F, 6, 11, 2)
    _run_and_check(w, toks, [0, 1], jd, df)


@pytest.mark.parametrize("T", [2**20 - 1, 2**20])
def test_token_rows_at_4_gib(T):
    D, F, E = 2048, 64, 8
    w = W.Workload("limit_x_%d" % T, T=T, D=D, F=F, E=E, K=1, routing="uniform_distinct",
                   backward=True, seed=12)
    assert (T * D * 2 < 2**32) == (T < 2**20)
    toks = np.concatenate([[0, 1], W.sample_tokens(T, 12, seed=3), [T - 2, T - 1]]).astype(np.int64)
    toks = np.unique(toks)
    jd = _corners_and_seeded(2 * F, D, 4, 12, 1)
    df = _corners_and_seeded(D, F, 4, 12, 2)
    _run_and_check(w, toks, [0, 3, E - 1], jd, df)


def _uniform_ids(n, E, seed, block=1 << 26):
    """Seeded uniform int32 expert ids, drawn in independent blocks on a few threads."""
    from concurrent.futures import ThreadPoolExecutor
    out = np.empty(n, dtype=np.int32)
    nblk = (n + block - 1) // block
    seqs = np.random.SeedSequence([seed, 31]).spawn(nblk)

    def fill(b):
        lo, hi = b * block, min(n, (b + 1) * block)
        g = np.random.Generator(np.random.PCG64(seqs[b]))
        out[lo:hi] = g.integers(0, E, hi - lo, dtype=np.int32)

    with ThreadPoolExecutor(8) as ex:
        list(ex.map(fill, range(nblk)))
    return out


def test_plan_at_the_slot_limit():
    import mixture_experts_routed_plan_amd as M
    T, K, E = 2**25 - 1024, 64, 1024
    N = T * K
    assert N == 2**31 - 2**16
    s = M.make_shape(T, 64, 64, E, K, M.MOE_IDS_I32, False)
    nb = M.moe_plan_bytes(s)
    assert nb > 0
    t0 = time.time()
    ids = _uniform_ids(N, E, 13)
    log("\n[slot limit] %d ids drawn in %.1fs" % (N, time.time() - t0))
    d_ids = torch.from_numpy(ids).cuda()
    plan = torch.empty(nb, dtype=torch.uint8, device="cuda")
    M.check(M.moe_plan(s, d_ids, plan), "moe_plan")
    st, bad = M.moe_plan_status(s, plan)
    M.check(st, "moe_plan_status")
    assert bad == 0
    del d_ids
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    pos = torch.empty(N, dtype=torch.int32, device="cuda")
    src = torch.empty(N, dtype=torch.int32, device="cuda")
    M.check(M.moe_plan_export(s, plan, counts, offsets, pos, src), "moe_plan_export")
    torch.cuda.synchronize()
    del plan
    counts, offsets = counts.cpu().numpy(), offsets.cpu().numpy()
    pos_h = pos.cpu().numpy()
    del pos
    src_h = src.cpu().numpy()
    del src
    torch.cuda.empty_cache()
    log("[slot limit] gpu plan done, arrays on the host after %.1fs" % (time.time() - t0))

    ref_counts = np.bincount(ids, minlength=E)
    np.testing.assert_array_equal(counts, ref_counts)
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(ref_counts)]))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        seg = src_h[lo:hi]
        assert (ids[seg] == e).all(), "segment %d holds a slot of another expert" % e
        assert (np.diff(seg) > 0).all(), "segment %d is not in ascending slot order" % e
        assert (pos_h[seg] == np.arange(lo, hi, dtype=np.int32)).all(), "pos/src of segment %d" % e
    log("[slot limit] plan checked in %.1fs" % (time.time() - t0))
    del ids, pos_h, src_h
    gc.collect()
