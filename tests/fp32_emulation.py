"""A second, independent implementation of the layer for the tolerance
analysis of the parity tests (test infrastructure only).

It computes what a correct GPU implementation computes: every product in
float32 with float32 accumulation (torch's CPU float32 matmul), rounded to
bf16 at the same storage points as the oracle (A, H, Y, out, dYp, dA, dXp,
dX, dW1, dW2, dWr; probs, gates, dgate, dXe and db stay float32).  Only the
integer routing (top-k, capacity, maps) is taken from the oracle's result,
since routing is compared bit-exactly anyway.  Comparing this emulation with
the oracle shows how far a correct fp32-accumulating implementation lands
from the fp64 reference: a tolerance it exceeds cannot be demanded of the
GPU.
"""
from __future__ import annotations

import math

import numpy as np
import torch

C0 = math.sqrt(2.0 / math.pi)


def _bf(t: torch.Tensor) -> torch.Tensor:
    """float32 -> nearest bf16 value (ties to even), kept as float32."""
    return t.to(torch.bfloat16).to(torch.float32)


def _gelu(a):
    u = C0 * (a + 0.044715 * a * a * a)
    return 0.5 * a * (1.0 + torch.tanh(u))


def _gelu_grad(a):
    u = C0 * (a + 0.044715 * a * a * a)
    th = torch.tanh(u)
    return 0.5 * (1.0 + th) + 0.5 * a * (1.0 - th * th) * C0 * (1.0 + 3 * 0.044715 * a * a)


def _f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def layer(inp, w, fw):
    """Forward and backward of a bf16 workload; fw is the oracle's forward
    (only its integer routing -- or, for the expert-share workload, the given
    ragged layout and gates -- is used).  Returns float64 arrays."""
    to32 = lambda a: torch.from_numpy((np.asarray(a).astype(np.uint32) << 16).view(np.float32))
    dOut = to32(inp["dOut"])
    layer_kind = w.kind == "layer"
    k = w.k
    row_of = np.asarray(fw["row_of"]).astype(np.int64)
    src = np.asarray(fw["src_of"]).astype(np.int64)
    off = np.asarray(fw["offsets"]).astype(np.int64)
    R = int(off[-1])
    T, d = dOut.shape
    if layer_kind:
        x = to32(inp["x"])
        Wr = to32(inp["Wr"])
        b = _f32(inp["b"])
        idx = torch.from_numpy(np.asarray(fw["idx"]).astype(np.int64))
        probs = torch.softmax(x @ Wr + b, dim=1)
        gate = torch.gather(probs, 1, idx)
        xp = x[torch.from_numpy(src // k)]
    else:
        gate = _f32(inp["gate"])
        xp = to32(inp["x_perm"])
    A = torch.zeros(R, w.f)
    H = torch.zeros(R, w.f)
    Y = torch.zeros(R, w.d)
    for e in range(w.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        W1 = to32(inp["W1"][e])
        W2 = to32(inp["W2"][e])
        A[lo:hi] = _bf(xp[lo:hi] @ W1)
        H[lo:hi] = _bf(_gelu(A[lo:hi]))
        Y[lo:hi] = _bf(H[lo:hi] @ W2)
    kept = torch.from_numpy(row_of >= 0)
    rows = torch.from_numpy(np.where(row_of >= 0, row_of, 0))
    out = torch.zeros(T, d)
    for j in range(k):
        m = kept[:, j]
        out[m] += gate[m, j, None] * Y[rows[m, j]]
    out = _bf(out)
    # backward
    dYp = torch.zeros(R, d)
    dg = torch.zeros(T, k)
    for j in range(k):
        m = kept[:, j]
        dYp[rows[m, j]] = _bf(gate[m, j, None] * dOut[m])
        dg[m, j] = (dOut[m] * Y[rows[m, j]]).sum(dim=1)
    dXp = torch.zeros(R, d)
    dA = torch.zeros(R, w.f)
    dW1 = torch.zeros(w.E, w.d, w.f)
    dW2 = torch.zeros(w.E, w.f, w.d)
    for e in range(w.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        W1 = to32(inp["W1"][e])
        W2 = to32(inp["W2"][e])
        dH = dYp[lo:hi] @ W2.T
        dA[lo:hi] = _bf(dH * _gelu_grad(A[lo:hi]))
        dXp[lo:hi] = _bf(dA[lo:hi] @ W1.T)
        dW1[e] = _bf(xp[lo:hi].T @ dA[lo:hi])
        dW2[e] = _bf(H[lo:hi].T @ dYp[lo:hi])
    f64 = lambda t: t.double().numpy()
    res = dict(gate=f64(gate), A=f64(A), H=f64(H), Y=f64(Y), out=f64(out), dYp=f64(dYp),
               dgate=f64(dg), dA=f64(dA), dXp=f64(dXp), dW1=f64(dW1), dW2=f64(dW2))
    if not layer_kind:
        return res
    dXe = torch.zeros(T, d)
    for j in range(k):
        m = kept[:, j]
        dXe[m] += dXp[rows[m, j]]
    dp = torch.zeros(T, w.E)
    for j in range(k):
        m = kept[:, j]
        dp[m, idx[m, j]] += dg[m, j]
    dz = probs * (dp - (probs * dp).sum(dim=1, keepdim=True))
    res.update(probs=f64(probs), dXe=f64(dXe), dX=f64(_bf(dXe + dz @ Wr.T)),
               dWr=f64(_bf(x.T @ dz)), db=f64(dz.sum(dim=0)))
    return res


def ratio(got, ref, rtol=2e-2, atol=1e-2):
    """max over elements of |got - ref| / (atol + rtol |ref|): at most 1 iff
    numpy-allclose at (rtol, atol)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / (atol + rtol * np.abs(ref))))
