"""Device-memory helpers around the libl3 binding.

`L3Layer` sizes and allocates the plan / save / scratch workspaces with
torch (device memory and streams only) and calls the C entry points in
order. `L3Function` is the torch.autograd glue: forward = plan + l3_forward
with a save workspace, backward = l3_backward. No arithmetic of the layer
runs in Python or torch.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import _lib as L


def torch_dtype(l3_dtype: int):
    return torch.bfloat16 if l3_dtype == L.L3_BF16 else torch.float32


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy array -> device tensor; uint16 arrays are bfloat16 bit patterns."""
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
        return t.to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class L3Layer:
    def __init__(self, desc: L.l3_desc, max_tokens: int, device="cuda",
                 training: bool = False):
        self.desc = desc
        self.device = device
        self.max_tokens = int(max_tokens)
        p, s, c = L.l3_workspace_size(desc, self.max_tokens)
        u8 = dict(dtype=torch.uint8, device=device)
        self.plan_ws = torch.empty(max(p, 256), **u8)
        self.save = torch.empty(max(s, 256), **u8) if training else None
        self.scratch = torch.empty(max(c, 256), **u8)
        self.plan: Optional[L.Plan] = None
        # bumped by every (re)plan: the layer holds one plan and one save
        # workspace, so a backward belongs to the forward of the same plan
        self.generation = 0

    def make_plan(self, ids: torch.Tensor, offsets: torch.Tensor,
                  check_status=True) -> L.Plan:
        if self.plan is None:
            self.plan = L.l3_plan(self.desc, ids, offsets, self.plan_ws,
                                  check_status=check_status)
        else:
            L.l3_replan(self.plan, ids, offsets)
        self.generation += 1
        return self.plan

    def forward(self, x, K, V, W_up, gamma, beta, W_mix, y=None, save=None):
        B = self.plan.tokens
        if y is None:
            y = torch.empty((B, self.desc.d), dtype=torch_dtype(
                self.desc.y_dtype), device=self.device)
        L.l3_forward(self.plan, x, K, V, W_up, gamma, beta, W_mix, y,
                     self.save if save is None else save, self.scratch)
        return y

    def backward(self, dy, x, K, V, W_up, gamma, beta, W_mix, out=None):
        """Gradients (float32) of sum(y * dy); `out` may hold some of the
        output tensors (dx, dK, dV, dW_up, dgamma, dbeta, dW_mix) to write
        into, the others are allocated."""
        d, d_e, R = self.desc.d, self.desc.d_e, self.desc.rows
        f32 = dict(dtype=torch.float32, device=self.device)
        B = self.plan.tokens
        shapes = dict(dx=(B, d), dK=(R, d), dV=(R, d_e), dW_up=(d, d_e),
                      dgamma=(d,), dbeta=(d,), dW_mix=(d, 2 * d))
        out = out or {}
        g = {k: out[k] if k in out else torch.empty(v, **f32)
             for k, v in shapes.items()}
        L.l3_backward(self.plan, dy, x, K, V, W_up, gamma, beta, W_mix,
                      self.save, g["dx"], g["dK"], g["dV"], g["dW_up"],
                      g["dgamma"], g["dbeta"], g["dW_mix"], self.scratch)
        return g


class L3Function(torch.autograd.Function):
    """y = L3(x; ids, K, V, W_up, gamma, beta, W_mix) with libl3 backward.

    The layer object holds one plan and one save workspace (it must be made
    with training=True): a backward needs the forward of the same plan, so a
    second forward through the same layer before the first one's backward
    makes that backward raise. Use one L3Layer per pending forward.
    Gradients are computed in float32 and returned in each input's dtype
    (autograd's rule); L3Layer.backward gives the float32 ones."""

    @staticmethod
    def forward(ctx, layer: L3Layer, ids, offsets, x, K, V, W_up, gamma,
                beta, W_mix):
        if layer.save is None:
            raise ValueError("L3Function needs an L3Layer made with "
                             "training=True (a save workspace)")
        layer.make_plan(ids, offsets)
        y = layer.forward(x, K, V, W_up, gamma, beta, W_mix)
        ctx.layer = layer
        ctx.generation = layer.generation
        ctx.save_for_backward(x, K, V, W_up, gamma, beta, W_mix)
        return y

    @staticmethod
    def backward(ctx, dy):
        if ctx.layer.generation != ctx.generation:
            raise RuntimeError(
                "L3Function.backward: the layer was re-planned by another "
                "forward after this one; its saved state is gone")
        x, K, V, W_up, gamma, beta, W_mix = ctx.saved_tensors
        dy = dy.to(x.dtype).contiguous()
        g = ctx.layer.backward(dy, x, K, V, W_up, gamma, beta, W_mix)
        cast = lambda t, ref: t.to(ref.dtype)
        return (None, None, None, cast(g["dx"], x), cast(g["dK"], K),
                cast(g["dV"], V), cast(g["dW_up"], W_up),
                cast(g["dgamma"], gamma), cast(g["dbeta"], beta),
                cast(g["dW_mix"], W_mix))
