"""GPU: the row steps on their own through the C ABI (moe_permute, moe_combine with and without
scores, moe_combine_backward), fed the oracle's own intermediates, against the oracle: the permute
bit-exact, the combines element by element (dscores with the rss scale), with out-of-range ids
dropped."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_check import check, log

pytestmark = pytest.mark.gpu


def _f64_to_bits(a):
    # the oracle's bf16-mode values are bf16-representable: their float32 bit patterns' high
    # halves are the bf16 bits
    b = np.ascontiguousarray(np.asarray(a, np.float32)).view(np.uint32)
    assert ((b & 0xFFFF) == 0).all()
    return (b >> 16).astype(np.uint16)


@pytest.mark.parametrize("name", ["p_ragged", "p_wide", "p_skew"])  # K = 3, 4, 2
def test_row_steps_against_oracle(name):
    import mixture_experts_routed_plan_amd as M
    from mixture_experts_routed_plan_amd import device as dv
    w = W.PARITY_WORKLOADS[name]
    inp = W.make_inputs(w, with_dout=True, router=oracle.route)
    inp.ids[3, 0] = w.E + 1  # a dropped slot
    inp.ids[10, w.K - 1] = -2
    ref = oracle.full(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, scales=True)
    N = w.T * w.K
    s = M.make_shape(w.T, w.D, w.F, w.E, w.K, save_for_backward=False)
    plan = torch.empty(M.moe_plan_bytes(s), dtype=torch.uint8, device="cuda")
    ids = torch.from_numpy(inp.ids).cuda()
    M.check(M.moe_plan(s, ids, plan), "moe_plan")
    nv = int(ref["offsets"][-1])
    log("\n[%s] T=%d D=%d K=%d, %d routed rows" % (name, w.T, w.D, w.K, nv))
    # permute
    x = dv.to_device_bits(inp.x)
    xg = torch.zeros(N, w.D, dtype=torch.bfloat16, device="cuda")
    M.check(M.moe_permute(s, plan, x, xg), "moe_permute")
    # weighted combine of the oracle's y, and the unweighted one of its dxg
    y = dv.to_device_bits(_f64_to_bits(ref["y"]))
    sc = torch.from_numpy(inp.scores).cuda()
    out = torch.empty(w.T, w.D, dtype=torch.bfloat16, device="cuda")
    M.check(M.moe_combine(s, plan, y, sc, out), "moe_combine")
    dxg = dv.to_device_bits(_f64_to_bits(ref["dxg"]))
    dx = torch.empty(w.T, w.D, dtype=torch.bfloat16, device="cuda")
    M.check(M.moe_combine(s, plan, dxg, None, dx), "moe_combine (dX)")
    # combine transpose and dscores
    dout = dv.to_device_bits(inp.dout)
    dy = torch.zeros(N, w.D, dtype=torch.bfloat16, device="cuda")
    dsc = torch.empty(w.T, w.K, dtype=torch.float32, device="cuda")
    M.check(M.moe_combine_backward(s, plan, dout, y, sc, dy, dsc), "moe_combine_backward")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dv.to_host_bits(xg)[:nv], _f64_to_bits(ref["xg"][:nv]))
    check("out", dv.bits_to_f64(dv.to_host_bits(out)), ref["out"])
    check("dx", dv.bits_to_f64(dv.to_host_bits(dx)), ref["dx"])
    # dy = bf16(s * dout): one fp32 product rounded once on the GPU, the exact product rounded
    # once in the oracle
    check("dy", dv.bits_to_f64(dv.to_host_bits(dy))[:nv], ref["dy"][:nv])
    check("dscores", dsc.cpu().numpy(), ref["dscores"], ref["dscores_rss"])
    assert dsc.cpu().numpy()[3, 0] == 0 and dsc.cpu().numpy()[10, w.K - 1] == 0
