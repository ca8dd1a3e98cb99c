"""CPU oracle of one GPU's share of the expert-parallel MoE layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never routes through
it, and this module imports nothing from the product package.

What is computed, and where the pages say so:

* Step order of the layer forward -- score each token against every expert,
  lay the routed tokens out contiguously per expert, run every local expert
  on its rows, then undo the permutation back to token order:
  "GPU expert parallel" (aicassindra.com), section "The step timeline".
  The all-to-all exchanges of that section need several GPUs and are not
  part of one GPU's share.
* The backward pass retraces those steps in reverse: same section.
* The router is replicated, must give identical decisions everywhere, and
  its gradient is an ordinary parameter gradient: section "Sharded by
  expert, replicated everywhere else".
* Top-k (k=2 in the example) and the capacity factor (1.25 in the example):
  distributed-training tutorial (deepseekmodel.com), section "The Capacity
  Factor" and the EP configuration block under "The Conflict Between EP
  and TP".  Tokens beyond an expert's capacity are dropped.
* Expert FFN = per-expert feed-forward weights ("Sharded by expert"), here
  W1 (d x f) -> tanh-GELU -> W2 (f x d), no biases.

Readings taken where the pages are silent (numbered R1..R19 throughout; R8
(bias) and R9 (FFN form) are stated with the inputs and the FFN above):
  R1 softmax over all E logits, then top-k; gate = probability of the chosen
     expert, not renormalised.
  R2 selection is made on the fp32 logit z; ties go to the lower expert
     index; the slot order is (z descending, expert ascending).
  R3 canonical logit: z = RN_fp32(sum_i x_i Wr_ie + b_e) with the sum taken
     in fp64 (bf16*bf16 and fp32*fp32 products are exact in fp64).
  R4 capacity C = ceil(cf * T * k / E), evaluated exactly on the decimal cf;
     no limit when cf is None.
  R5 a full expert drops the later tokens: assignments are walked in token
     order and an assignment is kept iff fewer than C earlier tokens chose
     the same expert.
  R6 a dropped assignment contributes nothing; the other gates are not
     renormalised; a token with every assignment dropped gets out = 0.
  R7 counts = routed assignments per expert before the drop; offsets scan
     the kept counts (compact ragged layout of R rows).
  R10 storage rounding (round-to-nearest-even) at A, H, Y, out, dYp, dA, dXp,
     dX, dW1, dW2, dWr to the activation type s; probs, gates, dgate, dXe,
     db are fp32.  Everything between storage points is fp64.
  R11 L = <out, dOut>; index/top-k/capacity steps are piecewise constant and
     carry no gradient.
  R16 auxiliary load-balancing loss (the balancing penalty of the tutorial's
     section "The Capacity Factor", coefficient alpha, 0.01 in its EP
     configuration block): the pages give no formula; this reading is the
     standard published balancing loss L_aux = alpha * E * sum_e f_e P_e with
     f_e = counts_e / (T k) (routed assignments before the drop) and P_e the
     mean router probability of expert e over the tokens.  f is piecewise
     constant, so the gradient flows through P only and joins dgate before
     the softmax backward.  Drop rate = 1 - R / (T k).
  R17 gate renormalisation (an option; the pages fix no gate normalisation):
     g[t,j] = p[t,idx_j] / sum_i p[t,idx_i] over the k selected experts,
     before the capacity drop; a drop does not renormalise again (R6).
  R18 capacity priority (an option; the pages do not say which assignments
     of a full expert go first): 'slot' walks the assignments slot-major,
     every token's first choice before any second choice, (j, t) in
     lexicographic order, instead of token-major (t, j).  Rows of an expert
     are laid out in that walk order.
  R19 fallback path of a dropped assignment (an option; the pages only say
     that excess tokens are dropped or take a fallback path): 'identity'
     sends the token past the expert unchanged, so the dropped assignment
     contributes gate[t,j] * x[t] to out[t]; backward, it adds
     gate[t,j] * dOut[t] to dX[t] and dgate[t,j] = <dOut[t], x[t]>.

Every floating-point result here is fp64 arithmetic on exactly converted
inputs followed by one rounding at the storage point; ``exact=True`` turns
all storage roundings off (used by the finite-difference self-tests).
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Dict, Optional

import numpy as np

SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
GELU_C3 = 0.044715


# ------------------------------------------------------------ number formats
def to_f64(a: np.ndarray) -> np.ndarray:
    """Storage array -> exact float64 values.  uint16 arrays hold bf16 bits:
    the bf16 value is the float32 whose upper 16 bits are those bits."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def bf16_rne(a) -> np.ndarray:
    """Round float64 values to bfloat16 (8 significant bits, 8-bit exponent),
    round-to-nearest, ties-to-even, in ONE rounding step (no fp32 detour).
    Returned as float64 holding the bf16 values.  Finite inputs only."""
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)                 # a = m * 2**e with 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)        # spacing 2**q; bf16 subnormals 2**-133
    return np.ldexp(np.rint(np.ldexp(a, -q)), q)   # rint: ties to even


def fp32_rne(a) -> np.ndarray:
    """Round float64 values to float32 (numpy's cast is correctly rounded)."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def rounder(dtype: str, exact: bool = False):
    """Storage rounding of the activation type s ('f32' | 'bf16')."""
    if exact:
        return lambda a: np.asarray(a, dtype=np.float64)
    if dtype == "bf16":
        return bf16_rne
    if dtype == "f32":
        return fp32_rne
    raise ValueError(dtype)


def bf16_bits(a64: np.ndarray) -> np.ndarray:
    """float64 array of bf16-exact values -> uint16 bit patterns."""
    return (np.asarray(a64, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


# ------------------------------------------------------------ F1: router
def router_logits(x, Wr, b, round32: bool = True) -> np.ndarray:
    """z[t,e] = sum_i x[t,i] Wr[i,e] + b[e], summed in fp64, then rounded
    once to fp32 (reading R3): every token is scored against every expert."""
    z = np.asarray(x, np.float64) @ np.asarray(Wr, np.float64)
    z = z + np.asarray(b, np.float64)[None, :]
    return fp32_rne(z) if round32 else z


def softmax(z) -> np.ndarray:
    """p[t,:] = exp(z - max z) / sum exp(z - max z) over all experts (R1)."""
    z = np.asarray(z, np.float64)
    ez = np.exp(z - z.max(axis=-1, keepdims=True))
    return ez / ez.sum(axis=-1, keepdims=True)


def topk_select(z, k: int) -> np.ndarray:
    """idx[t, j] = the j-th expert in the order (z descending, e ascending):
    k rounds of "take the largest remaining logit"; np.argmax returns the
    first maximum, so equal logits go to the lower expert index (R2)."""
    zw = np.array(z, dtype=np.float64, copy=True)
    T = zw.shape[0]
    idx = np.empty((T, k), dtype=np.int32)
    rows = np.arange(T)
    for j in range(k):
        pick = np.argmax(zw, axis=1)
        idx[:, j] = pick
        zw[rows, pick] = -np.inf
    return idx


# ------------------------------------------------------------ F2: capacity + permute
def capacity(T: int, k: int, E: int, cf: Optional[float]) -> Optional[int]:
    """C = ceil(cf * T * k / E) in exact rational arithmetic on the decimal
    value of cf (R4); None means no capacity limit (drop-free)."""
    if cf is None:
        return None
    return math.ceil(Fraction(str(cf)) * T * k / E)


def assign(idx: np.ndarray, E: int, C: Optional[int], priority: str = "token"):
    """Capacity drop and the permutation map (R5, R7, R18).

    Walk the T*k assignments in token-major order (t, j), or slot-major
    (j, t) for priority 'slot'; pos = how many earlier assignments in the
    walk chose the same expert; kept iff pos < C.  Returns
      counts[E]   routed assignments per expert (before the drop),
      offsets[E+1] exclusive scan of the kept counts (offsets[E] = R),
      row_of[T,k] row of (t,j) in the permuted buffer, or -1 if dropped,
      src_of[R]   t*k + j of the assignment stored in each row.
    """
    T, k = idx.shape
    if priority == "token":
        walk = ((t, j) for t in range(T) for j in range(k))
    elif priority == "slot":
        walk = ((t, j) for j in range(k) for t in range(T))
    else:
        raise ValueError(priority)
    counts = np.zeros(E, dtype=np.int64)
    pos = np.full((T, k), -1, dtype=np.int64)
    for t, j in walk:
        e = int(idx[t, j])
        p = counts[e]
        counts[e] = p + 1
        if C is None or p < C:
            pos[t, j] = p
    kept = counts if C is None else np.minimum(counts, C)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    row_of = np.where(pos >= 0, offsets[idx] + pos, -1)
    R = int(offsets[E])
    src_of = np.full(R, -1, dtype=np.int64)
    t_of, j_of = np.nonzero(row_of >= 0)
    src_of[row_of[t_of, j_of]] = t_of * k + j_of
    return (counts.astype(np.int32), offsets.astype(np.int32),
            row_of.astype(np.int32), src_of.astype(np.int32))


def permute(x, src_of, k: int) -> np.ndarray:
    """x_perm[r] = x[token of row r] -- contiguous per-expert buffers."""
    return np.asarray(x)[np.asarray(src_of) // k]


# ------------------------------------------------------------ F3/F4: expert FFN
def gelu_tanh(a) -> np.ndarray:
    """0.5 a (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3)))."""
    a = np.asarray(a, np.float64)
    return 0.5 * a * (1.0 + np.tanh(SQRT_2_OVER_PI * (a + GELU_C3 * a ** 3)))


def gelu_tanh_grad(a) -> np.ndarray:
    """d/da of gelu_tanh: with u = sqrt(2/pi)(a + 0.044715 a^3),
    0.5 (1 + tanh u) + 0.5 a (1 - tanh^2 u) sqrt(2/pi) (1 + 3*0.044715 a^2)."""
    a = np.asarray(a, np.float64)
    th = np.tanh(SQRT_2_OVER_PI * (a + GELU_C3 * a ** 3))
    return (0.5 * (1.0 + th)
            + 0.5 * a * (1.0 - th * th) * SQRT_2_OVER_PI
            * (1.0 + 3.0 * GELU_C3 * a * a))


def expert_ffn_fwd(xe, W1e, W2e, rnd):
    """One expert over its rows: A = xe W1e, H = gelu(A), Y = H W2e, each
    rounded at its storage point (R10)."""
    A = rnd(np.asarray(xe, np.float64) @ np.asarray(W1e, np.float64))
    H = rnd(gelu_tanh(A))
    Y = rnd(H @ np.asarray(W2e, np.float64))
    return A, H, Y


def expert_ffn_bwd(xe, W1e, W2e, Ae, He, dYe, rnd):
    """Reverse of expert_ffn_fwd for one expert:
    dH = dY W2^T, dA = dH * gelu'(A) (stored), dX = dA W1^T,
    dW1 = xe^T dA, dW2 = H^T dY (zero matrices for an expert with no rows)."""
    W1e = np.asarray(W1e, np.float64)
    W2e = np.asarray(W2e, np.float64)
    dH = dYe @ W2e.T
    dW2 = np.asarray(He, np.float64).T @ dYe
    dA = rnd(dH * gelu_tanh_grad(Ae))
    dX = dA @ W1e.T
    dW1 = np.asarray(xe, np.float64).T @ dA
    return rnd(dX), rnd(dW1), rnd(dW2), dA


# ------------------------------------------------------------ F5: combine
def combine(Y, row_of, gate, rnd, x=None) -> np.ndarray:
    """out[t] = sum over kept j (ascending) of gate[t,j] * Y[row_of[t,j]];
    the inverse permutation back to token order (R6).  With the identity
    fallback (x given, R19) a dropped j adds gate[t,j] * x[t] instead."""
    row_of = np.asarray(row_of)
    T, k = row_of.shape
    g = np.asarray(gate, np.float64)
    acc = np.zeros((T, Y.shape[1]), dtype=np.float64)
    for j in range(k):
        m = row_of[:, j] >= 0
        acc[m] += g[m, j, None] * Y[row_of[m, j]]
        if x is not None:
            acc[~m] += g[~m, j, None] * np.asarray(x, np.float64)[~m]
    return rnd(acc)


# ------------------------------------------------------------ backward
def combine_bwd(dOut, Y, row_of, gate, R: int, rnd, r32, x=None):
    """dYp[row_of[t,j]] = gate[t,j] * dOut[t];  dgate[t,j] = <dOut[t], Y[row]>
    for kept assignments; for dropped ones 0, or <dOut[t], x[t]> with the
    identity fallback (x given, R19)."""
    row_of = np.asarray(row_of)
    T, k = row_of.shape
    dYp = np.zeros((R, dOut.shape[1]), dtype=np.float64)
    dg = np.zeros((T, k), dtype=np.float64)
    for j in range(k):
        m = row_of[:, j] >= 0
        rows = row_of[m, j]
        dYp[rows] = np.asarray(gate, np.float64)[m, j, None] * dOut[m]
        dg[m, j] = np.einsum("td,td->t", dOut[m], Y[rows])
        if x is not None:
            dg[~m, j] = np.einsum("td,td->t", dOut[~m], np.asarray(x, np.float64)[~m])
    return rnd(dYp), r32(dg)


def unpermute_bwd(dXp, row_of, gate=None, dOut=None) -> np.ndarray:
    """dXe[t] = sum over kept j of dXp[row_of[t,j]] (fp64, caller rounds);
    with the identity fallback (gate and dOut given, R19) a dropped j adds
    gate[t,j] * dOut[t]."""
    row_of = np.asarray(row_of)
    T, k = row_of.shape
    acc = np.zeros((T, dXp.shape[1]), dtype=np.float64)
    for j in range(k):
        m = row_of[:, j] >= 0
        acc[m] += dXp[row_of[m, j]]
        if gate is not None:
            acc[~m] += np.asarray(gate, np.float64)[~m, j, None] * np.asarray(dOut)[~m]
    return acc


def renorm_gates(probs, idx) -> np.ndarray:
    """Gates renormalised over the selected experts (R17):
    g[t,j] = p[t,idx_j] / sum_i p[t,idx_i] (fp64; the caller rounds)."""
    sel = np.take_along_axis(np.asarray(probs, np.float64),
                             np.asarray(idx).astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def router_dz(probs, idx, row_of, dg, aux=None, renorm: bool = False) -> np.ndarray:
    """Softmax backward: dp[t, idx[t,j]] = dgate[t,j] for kept j (else 0),
    plus the load-balancing gradient aux[e] (aux_dp) when given;
    dz = p * (dp - sum_e p dp).  With renormalised gates (R17) the gate
    gradient first goes through g_j = p_j / S, S = sum_i p_i over the
    selected experts: dL/dp_j = (dgate_j - sum_i g_i dgate_i) / S for every
    selected j, dropped ones included (their own dgate is 0)."""
    probs = np.asarray(probs, np.float64)
    T, E = probs.shape
    dp = np.zeros((T, E), dtype=np.float64)
    if aux is not None:
        dp += np.asarray(aux, np.float64)[None, :]
    row_of = np.asarray(row_of)
    idx64 = np.asarray(idx).astype(np.int64)
    dg = np.asarray(dg, np.float64)
    if renorm:
        sel = np.take_along_axis(probs, idx64, axis=1)
        S = sel.sum(axis=1, keepdims=True)
        g = sel / S
        dsel = (dg - (g * dg).sum(axis=1, keepdims=True)) / S
        rows = np.arange(T)
        for j in range(idx64.shape[1]):
            dp[rows, idx64[:, j]] += dsel[:, j]
    else:
        # dgate of a dropped assignment is 0 unless a fallback path carries it
        rows = np.arange(T)
        for j in range(row_of.shape[1]):
            dp[rows, idx64[:, j]] += dg[:, j]
    s = (probs * dp).sum(axis=1, keepdims=True)
    return probs * (dp - s)


def aux_loss(probs, counts, k: int, coeff: float) -> float:
    """Load-balancing loss alpha * E * sum_e f_e P_e (reading R16)."""
    probs = np.asarray(probs, np.float64)
    T, E = probs.shape
    if T == 0:
        return 0.0
    f = np.asarray(counts, np.float64) / (T * k)
    P = probs.sum(axis=0) / T
    return float(coeff * E * np.dot(f, P))


def aux_dp(counts, T: int, k: int, coeff: float) -> np.ndarray:
    """dL_aux / dp[t, e] = alpha * E * f_e / T, the same for every token."""
    E = len(counts)
    if T == 0:
        return np.zeros(E)
    return coeff * E * np.asarray(counts, np.float64) / (T * k) / T


def drop_rate(offsets, T: int, k: int) -> float:
    """Fraction of the T k assignments dropped by the capacity limit."""
    if T * k == 0:
        return 0.0
    return 1.0 - float(np.asarray(offsets)[-1]) / (T * k)


def route_bwd(x, Wr, dz, dXe, rnd, r32):
    """Router backward: db = sum_t dz, dWr = x^T dz, dX = dXe + dz Wr^T."""
    db = r32(dz.sum(axis=0))
    dWr = rnd(np.asarray(x, np.float64).T @ dz)
    dX = rnd(dXe + dz @ np.asarray(Wr, np.float64).T)
    return dX, dWr, db


# ------------------------------------------------------------ whole layer
def route(inp: Dict[str, np.ndarray], w, exact: bool = False):
    """F1 + F2 index work: logits, probs, top-k, gates, capacity, maps."""
    r32 = rounder("f32", exact)
    x = to_f64(inp["x"])
    z = router_logits(x, to_f64(inp["Wr"]), to_f64(inp["b"]), round32=not exact)
    probs = r32(softmax(z))
    idx = topk_select(z, w.k)
    if w.renorm:
        gate = r32(renorm_gates(probs, idx))
    else:
        gate = np.take_along_axis(probs, idx.astype(np.int64), axis=1)
    C = capacity(w.T, w.k, w.E, w.cf)
    counts, offsets, row_of, src_of = assign(idx, w.E, C, w.priority)
    return dict(x=x, z=z, probs=probs, idx=idx, gate=gate, C=C, counts=counts,
                offsets=offsets, row_of=row_of, src_of=src_of)


def layer_fwd(inp: Dict[str, np.ndarray], w, exact: bool = False,
              keep_acts: bool = True) -> Dict[str, np.ndarray]:
    """Forward of one GPU's share of the MoE layer.

    'layer' workloads: route -> permute -> per-expert FFN -> combine.
    'ep_share' workloads: the input batch is already permuted (x_perm,
    offsets given); per-expert FFN -> gate-scaled inverse permutation.
    """
    rnd = rounder(w.dtype, exact)
    if w.fallback not in ("none", "identity"):
        raise ValueError(w.fallback)
    if w.kind == "layer":
        fw = route(inp, w, exact)
        fw["x_perm"] = permute(fw["x"], fw["src_of"], w.k)
    else:
        fw = dict(x_perm=to_f64(inp["x_perm"]),
                  offsets=np.asarray(inp["offsets"]),
                  counts=np.asarray(inp["counts"]),
                  row_of=np.asarray(inp["row_of"]),
                  src_of=np.asarray(inp["src_of"]),
                  gate=np.asarray(inp["gate"], np.float64))
    off = fw["offsets"]
    R = int(off[-1])
    A = np.zeros((R, w.f)); H = np.zeros((R, w.f)); Y = np.zeros((R, w.d))
    for e in range(w.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        A[lo:hi], H[lo:hi], Y[lo:hi] = expert_ffn_fwd(
            fw["x_perm"][lo:hi], to_f64(inp["W1"][e]), to_f64(inp["W2"][e]), rnd)
    fw.update(A=A, H=H, Y=Y, R=R)
    fb = w.kind == "layer" and w.fallback == "identity"
    fw["out"] = combine(Y, fw["row_of"], fw["gate"], rnd, fw["x"] if fb else None)
    if w.kind == "layer":
        fw["aux_loss"] = aux_loss(fw["probs"], fw["counts"], w.k, w.aux_coeff)
        fw["drop_rate"] = drop_rate(fw["offsets"], w.T, w.k)
    return fw


def layer_bwd(inp: Dict[str, np.ndarray], w, fw: Dict[str, np.ndarray],
              exact: bool = False) -> Dict[str, np.ndarray]:
    """Backward of the layer for upstream gradient dOut (L = <out, dOut>,
    plus the load-balancing loss when w.aux_coeff > 0)."""
    rnd = rounder(w.dtype, exact)
    r32 = rounder("f32", exact)
    dOut = to_f64(inp["dOut"])
    R = fw["R"]
    fb = w.kind == "layer" and w.fallback == "identity"
    dYp, dg = combine_bwd(dOut, fw["Y"], fw["row_of"], fw["gate"], R, rnd, r32,
                          fw["x"] if fb else None)
    off = fw["offsets"]
    dXp = np.zeros((R, w.d))
    dA = np.zeros((R, w.f))
    dW1 = np.zeros((w.E, w.d, w.f))
    dW2 = np.zeros((w.E, w.f, w.d))
    for e in range(w.E):
        lo, hi = int(off[e]), int(off[e + 1])
        dXp[lo:hi], dW1[e], dW2[e], dA[lo:hi] = expert_ffn_bwd(
            fw["x_perm"][lo:hi], to_f64(inp["W1"][e]), to_f64(inp["W2"][e]),
            fw["A"][lo:hi], fw["H"][lo:hi], dYp[lo:hi], rnd)
    bw = dict(dYp=dYp, dgate=dg, dXp=dXp, dA=dA, dW1=dW1, dW2=dW2)
    if w.kind == "layer":
        dXe = r32(unpermute_bwd(dXp, fw["row_of"], fw["gate"] if fb else None,
                                dOut if fb else None))
        aux = aux_dp(fw["counts"], w.T, w.k, w.aux_coeff) if w.aux_coeff > 0 else None
        dz = router_dz(fw["probs"], fw["idx"], fw["row_of"], dg, aux, w.renorm)
        dX, dWr, db = route_bwd(fw["x"], to_f64(inp["Wr"]), dz, dXe, rnd, r32)
        bw.update(dXe=dXe, dz=dz, dX=dX, dWr=dWr, db=db)
    return bw
