"""MoeLayer: device buffers (torch) around the C-ABI layer entry points.

Allocation and argument marshalling only; every step runs in libmoe.so.
"""
from __future__ import annotations

import torch

from . import binding as B


class MoeLayer:
    """One GPU's share of the MoE layer with caller-visible saved state.

    Weights are device tensors: Wr [d,E], b [E] float32 (or None),
    W1 [E,d,f], W2 [E,f,d], all of the activation dtype (bf16 or fp32).
    With diagnostics (the default when cfg.aux_coeff > 0) every forward also
    writes saved["aux"] = [load-balancing loss, drop rate]; the expert loads
    are saved["counts"].  The backward adds the loss's gradient whenever
    cfg.aux_coeff > 0.  Under MOE_FLAG_RECOMPUTE (make_cfg(recompute=True))
    A and H are not saved (saved["A"] = saved["H"] = None): the forward keeps
    them in the workspace and the backward recomputes them.
    """

    def __init__(self, cfg: B.MoeCfg, Wr, b, W1, W2, device="cuda", diagnostics=None):
        self.cfg = cfg
        T, d, E, k, f = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f
        self.sdt = torch.bfloat16 if cfg.dtype == B.MOE_BF16 else torch.float32
        self.Rmax = B.moe_rows_max(cfg)
        if self.Rmax < 0:
            raise B.MoeError("moe_rows_max", B.moe_check_cfg(cfg))
        dev = torch.device(device)
        e = lambda *s, dt=None: torch.empty(*s, dtype=dt or self.sdt, device=dev)
        self.w = dict(Wr=Wr, b=b, W1=W1, W2=W2)
        self.saved = dict(
            probs=e(T, E, dt=torch.float32), idx=e(T, k, dt=torch.int32),
            gate=e(T, k, dt=torch.float32), counts=e(E, dt=torch.int32),
            offsets=e(E + 1, dt=torch.int32), row_of=e(T, k, dt=torch.int32),
            src_of=e(self.Rmax, dt=torch.int32), x_perm=e(self.Rmax, d),
            A=e(self.Rmax, f), H=e(self.Rmax, f), Y=e(self.Rmax, d))
        if cfg.flags & B.MOE_FLAG_RECOMPUTE:
            self.saved["A"] = self.saved["H"] = None
        if diagnostics is None:
            diagnostics = cfg.aux_coeff > 0
        self.saved["aux"] = e(2, dt=torch.float32) if diagnostics else None
        self.ws = torch.empty(B.moe_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
        self.weights = B.MoeWeights(Wr=B._ptr(Wr), b=B._ptr(b), W1=B._ptr(W1),
                                    W2=B._ptr(W2))
        self.ctx = B.MoeCtx(**{n: B._ptr(t) for n, t in self.saved.items()})

    def forward(self, x, out=None, stream=None):
        if out is None:
            out = torch.empty(self.cfg.T, self.cfg.d, dtype=self.sdt, device=x.device)
        B.moe_layer_fwd(self.cfg, self.weights, x, out, self.ctx, self.ws, stream)
        return out

    def alloc_grads(self):
        w = self.w
        return dict(dWr=torch.empty_like(w["Wr"]),
                    db=torch.empty(self.cfg.E, dtype=torch.float32, device=w["Wr"].device),
                    dW1=torch.empty_like(w["W1"]), dW2=torch.empty_like(w["W2"]))

    def backward(self, x, dOut, dX=None, grads=None, stream=None):
        if dX is None:
            dX = torch.empty_like(x)
        if grads is None:
            grads = self.alloc_grads()
        g = B.MoeGrads(dWr=B._ptr(grads["dWr"]), db=B._ptr(grads["db"]),
                       dW1=B._ptr(grads["dW1"]), dW2=B._ptr(grads["dW2"]))
        B.moe_layer_bwd(self.cfg, self.weights, x, dOut, self.ctx, dX, g, self.ws, stream)
        return dX, grads
