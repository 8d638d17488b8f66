"""Device plumbing around the C ABI: torch allocations sized by the library's byte queries,
host<->device copies of bf16 bit patterns, and the fixed call sequence of one layer pass.
No layer arithmetic happens here."""
from __future__ import annotations

import numpy as np
import torch

from . import (MOE_IDS_I32, MOE_IDS_I64, MOE_OK, check, make_shape, moe_backward, moe_forward,
               moe_plan, moe_plan_bytes, moe_plan_export, moe_plan_status, moe_saved_bytes,
               moe_saved_views, moe_workspace_bytes)


def to_device_bits(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch bfloat16 tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Layer:
    """Buffers and calls for one shape. Inputs are device tensors owned by the caller."""

    def __init__(self, T, D, F, E, K, ids_dtype=np.int64, save_for_backward=True,
                 device="cuda", alloc_grads=None, wgrad_accumulate=False, wgrad_f32=False,
                 recompute=False, keep_xg=False):
        self.shape = make_shape(T, D, F, E, K,
                                MOE_IDS_I64 if np.dtype(ids_dtype) == np.int64 else MOE_IDS_I32,
                                save_for_backward, wgrad_accumulate, wgrad_f32, recompute, keep_xg)
        s = self.shape
        self.device = device
        nb = moe_plan_bytes(s)
        if nb == 0:
            raise ValueError("shape rejected by the library: %r" % (s,))
        self.x = None  # the forward's x, kept for the backward
        self.plan_buf = torch.empty(nb, dtype=torch.uint8, device=device)
        sb = moe_saved_bytes(s)
        self.saved = torch.empty(sb, dtype=torch.uint8, device=device) if sb else None
        self.workspace = torch.empty(moe_workspace_bytes(s), dtype=torch.uint8, device=device)
        self.out = torch.empty(T, D, dtype=torch.bfloat16, device=device)
        if alloc_grads is None:
            alloc_grads = save_for_backward
        if alloc_grads:
            self.dx = torch.empty(T, D, dtype=torch.bfloat16, device=device)
            gdt = torch.float32 if wgrad_f32 else torch.bfloat16
            # accumulation reads the existing gradients: start from zeros
            mk = torch.zeros if wgrad_accumulate else torch.empty
            self.dw13 = mk(E, 2, F, D, dtype=gdt, device=device)
            self.dw2 = mk(E, D, F, dtype=gdt, device=device)
            self.dscores = torch.empty(T, K, dtype=torch.float32, device=device)

    # -- calls -----------------------------------------------------------------------------
    def plan(self, ids, stream=None, trace=None):
        check(moe_plan(self.shape, ids, self.plan_buf, stream, trace), "moe_plan")

    def forward(self, x, scores, w13, w2, stream=None, trace=None):
        check(moe_forward(self.shape, self.plan_buf, x, scores, w13, w2, self.out, self.saved,
                          self.workspace, stream, trace), "moe_forward")
        self.x = x  # the backward reads x again (the W13 weight gradient gathers its token rows)
        return self.out

    def backward(self, dout, scores, w13, w2, stream=None, trace=None, x=None):
        x = self.x if x is None else x
        check(moe_backward(self.shape, self.plan_buf, self.saved, x, dout, scores, w13, w2,
                           self.dx, self.dw13, self.dw2, self.dscores, self.workspace, stream,
                           trace), "moe_backward")

    # -- inspection ------------------------------------------------------------------------
    def plan_arrays(self):
        s = self.shape
        N = s.T * s.K
        d = self.device
        counts = torch.empty(s.E, dtype=torch.int32, device=d)
        offsets = torch.empty(s.E + 1, dtype=torch.int32, device=d)
        pos = torch.empty(N, dtype=torch.int32, device=d)
        src = torch.empty(N, dtype=torch.int32, device=d)
        check(moe_plan_export(s, self.plan_buf, counts, offsets, pos, src), "moe_plan_export")
        torch.cuda.synchronize()
        return dict(counts=counts.cpu().numpy(), offsets=offsets.cpu().numpy(),
                    pos=pos.cpu().numpy(), src=src.cpu().numpy())

    def plan_status(self):
        return moe_plan_status(self.shape, self.plan_buf)

    def saved_arrays(self):
        """Host copies (uint16 bits) of xg, h13, a, y from the saved buffer."""
        s = self.shape
        N = s.T * s.K
        xg, h13, a, y = moe_saved_views(s, self.saved)
        base = self.saved.data_ptr()
        out = {}
        for name, addr, cols in (("xg", xg, s.D), ("h13", h13, 2 * s.F), ("a", a, s.F),
                                 ("y", y, s.D)):
            if addr is None:  # not saved (recompute)
                continue
            off = addr - base
            t = self.saved[off:off + 2 * N * cols].view(torch.int16).view(N, cols)
            out[name] = t.cpu().numpy().view(np.uint16)
        return out
