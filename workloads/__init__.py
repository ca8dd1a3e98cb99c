"""Seeded synthetic inputs for the MoE layer hot path.

This module is shared by the CPU oracle and by the GPU path (tests, bench).
It produces input *data* only: shapes, random draws and their storage
format.  It holds none of the layer's arithmetic (no routing, capacity,
permutation, GEMM or gradient step).

Workloads (the shapes of the expert-parallel MoE layer of "GPU expert
parallel" (aicassindra.com), sections "The mesh" and "The step timeline",
with the top-k / capacity knobs of the "Expert Parallelism" EP config block
on the distributed-training tutorial page):

  tiny_f32   T=64    d=32   E=4   k=1 f=64   fp32  cf=1.25  bias 0
  c1_bf16    T=4096  d=1024 E=8   k=2 f=4096 bf16  cf=1.25  bias 0 (uniform)
  c2_zipf    T=8192  d=2048 E=64  k=2 f=1408 bf16  no cap   bias -1.2*ln(e+1)
  c3_epshare 16384 rows, 8 local experts, d=4096 f=2048 bf16, ragged counts
  c4_large   T=32768 d=4096 E=128 k=8 f=1536 bf16  cf=1.0   bias ~N(0,1)

Random streams: ``SeedSequence(seed).spawn(8)`` feeds one ``default_rng`` per
tensor, in the fixed order [x, Wr, b, W1, W2, dOut, ep-share aux, spare].
Normal draws are float32 ``standard_normal`` times the std, then rounded to
the storage type (bf16 by round-to-nearest-even through torch's CPU cast).

Storage format of returned arrays:
  * fp32 tensors: numpy float32;
  * bf16 tensors: numpy uint16 holding the bf16 bit patterns.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_inputs", "custom",
           "STREAMS", "bits_to_f32"]

STREAMS = ("x", "Wr", "b", "W1", "W2", "dOut", "aux", "spare")


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and input recipe of one synthetic MoE layer."""
    name: str
    T: int                 # tokens (rows of the ragged batch for 'ep_share')
    d: int                 # model dim
    E: int                 # experts (local experts for 'ep_share')
    k: int                 # top-k
    f: int                 # FFN dim
    dtype: str             # 'f32' or 'bf16'
    cf: Optional[float]    # capacity factor; None = no capacity limit
    bias: str = "zero"     # 'zero' | 'zipf' | 'normal'
    kind: str = "layer"    # 'layer' (full layer) | 'ep_share' (FFN+combine)
    w_std: float = 0.02
    zipf_s: float = 1.2
    dirichlet_alpha: float = 0.5
    pool_experts: int = 0  # size of the whole expert pool ('ep_share' only)
    aux_coeff: float = 0.0  # load-balancing loss coefficient (0 = none)
    renorm: bool = False    # gates renormalised over the selected k experts
    priority: str = "token"  # capacity priority: 'token' (token-major) | 'slot'
    fallback: str = "none"   # dropped assignments: 'none' | 'identity' (pass-through)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny_f32", T=64, d=32, E=4, k=1, f=64, dtype="f32", cf=1.25),
        Workload("c1_bf16", T=4096, d=1024, E=8, k=2, f=4096, dtype="bf16",
                 cf=1.25),
        Workload("c2_zipf", T=8192, d=2048, E=64, k=2, f=1408, dtype="bf16",
                 cf=None, bias="zipf"),
        Workload("c3_epshare", T=16384, d=4096, E=8, k=1, f=2048,
                 dtype="bf16", cf=None, kind="ep_share", pool_experts=64),
        Workload("c4_large", T=32768, d=4096, E=128, k=8, f=1536,
                 dtype="bf16", cf=1.0, bias="normal"),
    ]
}

# positional aliases used by the parity tests and the bench
ALIASES = {"C0": "tiny_f32", "C1": "c1_bf16", "C2": "c2_zipf",
           "C3": "c3_epshare", "C4": "c4_large"}


def get(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]


def custom(T, d, E, k, f, dtype="f32", cf=None, bias="zero",
           kind="layer", name="custom", w_std=0.02, aux_coeff=0.0, renorm=False,
           priority="token", fallback="none") -> Workload:
    return Workload(name, T=T, d=d, E=E, k=k, f=f, dtype=dtype, cf=cf,
                    bias=bias, kind=kind, w_std=w_std, aux_coeff=aux_coeff,
                    renorm=renorm, priority=priority, fallback=fallback)


# ---------------------------------------------------------------- storage
def _to_storage(a32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 array -> storage array (float32, or uint16 bf16 bits)."""
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Storage array -> float32 view of its values (exact for bf16 bits)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32, copy=False)


def _normal(rng, shape, std, dtype, chunk=1 << 24) -> np.ndarray:
    """std * N(0,1) float32 draws in storage format, drawn in chunks
    (chunked draws from one Generator equal a single draw)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        v = rng.standard_normal(m, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[s:s + m] = _to_storage(v, dtype)
    return out.reshape(shape)


def make_inputs(w: Workload, seed: int = 0) -> Dict[str, np.ndarray]:
    """Seeded inputs of workload ``w``.

    'layer' workloads: x[T,d], Wr[d,E], b[E] (f32), W1[E,d,f], W2[E,f,d],
    dOut[T,d].
    'ep_share' workloads: x_perm[T,d] (rows already grouped by expert),
    counts[E], offsets[E+1] (the ragged layout of x_perm), gate[T,1] (f32,
    U(0,1)), src_of[T] (row r holds token src_of[r]), row_of[T,1] (its
    inverse), W1, W2, dOut.
    """
    ss = np.random.SeedSequence(seed).spawn(len(STREAMS))
    rng = {name: np.random.default_rng(s) for name, s in zip(STREAMS, ss)}
    T, d, E, f = w.T, w.d, w.E, w.f
    out: Dict[str, np.ndarray] = {}
    out["W1"] = _normal(rng["W1"], (E, d, f), w.w_std, w.dtype)
    out["W2"] = _normal(rng["W2"], (E, f, d), w.w_std, w.dtype)
    out["dOut"] = _normal(rng["dOut"], (T, d), 1.0, w.dtype)
    if w.kind == "layer":
        out["x"] = _normal(rng["x"], (T, d), 1.0, w.dtype)
        out["Wr"] = _normal(rng["Wr"], (d, E), w.w_std, w.dtype)
        if w.bias == "zero":
            b = np.zeros(E, dtype=np.float32)
        elif w.bias == "zipf":
            # softmax of this bias alone is the Zipf(s) pmf over experts
            b = (-w.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
                 ).astype(np.float32)
        elif w.bias == "normal":
            b = rng["b"].standard_normal(E, dtype=np.float32)
        else:
            raise ValueError(w.bias)
        out["b"] = b
    elif w.kind == "ep_share":
        aux = rng["aux"]
        probs = aux.dirichlet(np.full(E, w.dirichlet_alpha))
        counts = aux.multinomial(T, probs).astype(np.int32)
        offsets = np.zeros(E + 1, dtype=np.int32)
        offsets[1:] = np.cumsum(counts)
        gate = aux.uniform(0.0, 1.0, size=(T, 1)).astype(np.float32)
        src_of = aux.permutation(T).astype(np.int32)
        row_of = np.empty((T, 1), dtype=np.int32)
        row_of[src_of, 0] = np.arange(T, dtype=np.int32)
        out.update(x_perm=_normal(rng["x"], (T, d), 1.0, w.dtype),
                   counts=counts, offsets=offsets, gate=gate,
                   src_of=src_of, row_of=row_of)
    else:
        raise ValueError(w.kind)
    return out
