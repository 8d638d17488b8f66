"""GPU: the allocation-free forward (moe_forward_noalloc), through the C ABI, against the forward
that takes a caller workspace (moe_forward without saving) and against the oracle: two calls in a
row on one GPU, the second with a smaller shape, so that it runs on the scratch the first left
behind; then the same with xg materialized (MOE_KEEP_XG)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_check import check, log

pytestmark = pytest.mark.gpu


def _case(w, keep_xg):
    import mixture_experts_routed_plan_amd as M
    from mixture_experts_routed_plan_amd import device as dv
    inp = W.make_inputs(w, with_dout=False, router=oracle.route)
    s = M.make_shape(w.T, w.D, w.F, w.E, w.K, save_for_backward=False, keep_xg=keep_xg)
    x, w13, w2 = (dv.to_device_bits(a) for a in (inp.x, inp.w13, inp.w2))
    ids = torch.from_numpy(inp.ids).cuda()
    sc = torch.from_numpy(inp.scores).cuda()
    plan = torch.empty(M.moe_plan_bytes(s), dtype=torch.uint8, device="cuda")
    ws = torch.empty(M.moe_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    ref_out = torch.empty(w.T, w.D, dtype=torch.bfloat16, device="cuda")
    out = torch.full((w.T, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.check(M.moe_plan(s, ids, plan), "moe_plan")
    M.check(M.moe_forward(s, plan, x, sc, w13, w2, ref_out, None, ws), "moe_forward")
    M.check(M.moe_forward_noalloc(s, plan, x, sc, w13, w2, out), "moe_forward_noalloc")
    torch.cuda.synchronize()
    return inp, dv.to_host_bits(out), dv.to_host_bits(ref_out)


@pytest.mark.parametrize("keep_xg", [False, True])
def test_noalloc_forward_two_calls_second_smaller(keep_xg):
    big = W.PARITY_WORKLOADS["p_ragged"]   # 2100 rows: 3.5 MB of a, y (+xg)
    small = W.WORKLOADS["tiny"]             # 32 rows
    for w in (big, small):
        log("\n[noalloc] %s T=%d D=%d F=%d E=%d K=%d keep_xg=%s"
            % (w.name, w.T, w.D, w.F, w.E, w.K, keep_xg))
        inp, got, ref = _case(w, keep_xg)
        np.testing.assert_array_equal(got, ref)  # the same kernels: the same bits
        want = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, None, mode="bf16")
        check("out", (got.astype(np.uint32) << 16).view(np.float32), want["out"])


def test_noalloc_forward_at_the_scratch_limit():
    """A shape whose a and y fill the scratch exactly (2*N*(F + D) = 64 MiB) runs and matches the
    workspace forward bit for bit; the next token is rejected on the host."""
    import mixture_experts_routed_plan_amd as M
    w = W.Workload("limit", T=8192, D=1024, F=1024, E=8, K=2, routing="uniform_distinct",
                   backward=False, seed=21)
    assert 2 * w.N * (w.D + w.F) == M.MOE_NOALLOC_SCRATCH_BYTES
    log("\n[noalloc] limit T=%d D=%d F=%d E=%d K=%d" % (w.T, w.D, w.F, w.E, w.K))
    _, got, ref = _case(w, False)
    np.testing.assert_array_equal(got, ref)
    over = M.make_shape(w.T + 1, w.D, w.F, w.E, w.K, save_for_backward=False)
    a = 4096
    assert M.moe_forward_noalloc(over, a, a, a, a, a, a, 0) == M.MOE_E_SCRATCH
