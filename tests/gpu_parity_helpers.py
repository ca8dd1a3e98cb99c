"""Helpers of the GPU parity tests: device transfer, running the HIP path
through the C-ABI, and element-wise comparison against the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle as O
import workloads as W

TOL = {  # (rtol, atol), numpy allclose semantics |g - o| <= atol + rtol |o|
    "bf16": (2e-2, 1e-2),
    "f32": (1e-5, 1e-5),
    "prob": (1e-5, 1e-6),      # probs / gates: fp32 quantities from near-equal logits
}
# Outputs that are sums over the token (row) axis -- dW1, dW2, dWr, db,
# dgate -- of products whose operands were rounded to the storage type
# upstream: two correct implementations that round at the same points still
# flip single upstream roundings (fp32 vs fp64 accumulation before the
# rounding), and a flipped operand moves its summand a_i b_i by at most one
# unit in the last place, u |a_i b_i| (u = 2^-7 for bf16's 8 significant
# bits, 2^-23 for fp32).  Independent flips of a fraction rho of the n
# summands move the sum by ~u sqrt(rho) ||(a_i b_i)_i||_2, and a single flip
# by at most u max_i |a_i b_i| <= u ||(a_i b_i)_i||_2.  The absolute
# tolerance of such an output element is therefore
#     max(atol, 2 u ||(a_i b_i)_i||_2),
# with ||(a_i b_i)_i||_2 = sqrt((a*a)^T (b*b)) computed from the oracle's own
# operands (factor 2: several flips).  When the summands are not at hand
# the rms of the sum stands in for their norm (random-sign sums:
# rms(sum) ~ ||(a_i b_i)||_2 for a typical element).
RED_UNIT = {"bf16": 2.0 ** -7, "f32": 2.0 ** -23}


def term_norm(a, b):
    """sqrt((a*a)^T (b*b)): per output element, the 2-norm of the summands
    of a^T b (a [n, M], b [n, N])."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.sqrt((a * a).T @ (b * b))


def terms_tol(norm, dtype):
    """(rtol, atol array) for a sum whose summand norms are `norm`."""
    rtol, atol = TOL[dtype]
    return rtol, np.maximum(atol, 2.0 * RED_UNIT[dtype] * np.asarray(norm, np.float64))


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_f64(t) -> np.ndarray:
    """device tensor -> float64 numpy (bf16 converted exactly through its bits).

    Buffers sized for Rmax rows hold whatever memory held past the R rows
    written; signaling-NaN patterns there raise numpy's invalid-cast flag
    on conversion.  Those rows are never compared, so the flag is ignored."""
    import torch
    t = t.detach()
    with np.errstate(invalid="ignore"):
        if t.dtype == torch.bfloat16:
            return O.to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
        return t.cpu().numpy().astype(np.float64)


def to_int(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int64)


def cfg_of(M, w, route_margin=0.0, recompute=False):
    cap = O.capacity(w.T, w.k, w.E, w.cf)
    return M.make_cfg(w.T, w.d, w.E, w.k, w.f, w.dtype, capacity=cap,
                      route_margin=route_margin, aux_coeff=w.aux_coeff, recompute=recompute,
                      renorm=w.renorm, priority=w.priority, fallback=w.fallback)


def red_tol(ref, dtype):
    """(rtol, atol) for a sum over the token axis whose summands are not at
    hand: the rms of the oracle output stands in for the summand norm."""
    rtol, atol = TOL[dtype]
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return rtol, atol
    rms = float(np.sqrt(np.mean(ref * ref)))
    return rtol, max(atol, 2.0 * RED_UNIT[dtype] * rms)


def expert_grad_tols(fw, bw, dtype):
    """Per-element tolerances of dW1 and dW2 from the oracle's operands:
    dW1[e] = x_e^T dA_e, dW2[e] = H_e^T dYp_e over the expert's rows."""
    off = fw["offsets"]
    E = len(off) - 1
    n1 = np.zeros(bw["dW1"].shape)
    n2 = np.zeros(bw["dW2"].shape)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            n1[e] = term_norm(fw["x_perm"][lo:hi], bw["dA"][lo:hi])
            n2[e] = term_norm(fw["H"][lo:hi], bw["dYp"][lo:hi])
    return terms_tol(n1, dtype), terms_tol(n2, dtype)


def assert_close(name, got, ref, tol):
    rtol, atol = TOL[tol] if isinstance(tol, str) else tol
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if got.size == 0:
        return
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        at = atol if np.ndim(atol) == 0 else np.broadcast_to(atol, err.shape)[i]
        raise AssertionError(
            f"{name}: {int(bad.sum())}/{bad.size} elements outside rtol={rtol} "
            f"atol={at}; worst at {i}: gpu={got[i]!r} oracle={ref[i]!r}")


def run_layer(M, w, inp, route_margin=0.0, bwd=True, recompute=False):
    """Forward (+ backward) of the layer on the GPU through moe_layer_fwd/bwd,
    with the routing diagnostics on.  res["aux1"] is the balancing loss at
    coefficient 1 (and the drop rate) from the standalone moe_router_aux on
    the same routing, so that its sums are checked in every case."""
    import copy

    import torch
    cfg = cfg_of(M, w, route_margin, recompute)
    d = {k: to_dev(v) for k, v in inp.items()}
    layer = M.MoeLayer(cfg, d["Wr"], d["b"], d["W1"], d["W2"], diagnostics=True)
    out = layer.forward(d["x"])
    res = dict(out=out, **layer.saved)
    c1 = copy.copy(cfg)
    c1.aux_coeff = 1.0
    res["aux1"] = torch.full((2,), -1.0, dtype=torch.float32, device="cuda")
    M.moe_router_aux(c1, layer.saved["probs"], layer.saved["counts"], layer.saved["offsets"],
                     res["aux1"], layer.ws)
    if bwd:
        dX, g = layer.backward(d["x"], d["dOut"])
        res.update(dX=dX, **g)
    torch.cuda.synchronize()
    res["_layer"] = layer
    res["_cfg"] = cfg
    res["_dev"] = d
    return res


def check_routing_exact(res, fw, w):
    R = int(fw["offsets"][-1])
    np.testing.assert_array_equal(to_int(res["idx"]), fw["idx"], err_msg="idx")
    np.testing.assert_array_equal(to_int(res["counts"]), fw["counts"], err_msg="counts")
    np.testing.assert_array_equal(to_int(res["offsets"]), fw["offsets"], err_msg="offsets")
    np.testing.assert_array_equal(to_int(res["row_of"]), fw["row_of"], err_msg="row_of")
    np.testing.assert_array_equal(to_int(res["src_of"])[:R], fw["src_of"], err_msg="src_of")
    return R


def logit_error(res, fw):
    """max over tokens/experts of the error of the GPU's fast logit
    differences z_e - z_top1, recovered from log-probabilities."""
    p = to_f64(res["probs"])
    z = fw["z"]
    top = fw["idx"][:, 0]
    rows = np.arange(z.shape[0])
    ok = p > 1e-30
    lp = np.log(np.where(ok, p, 1.0))
    dg = lp - lp[rows, top][:, None]
    dz = z - z[rows, top][:, None]
    return float(np.max(np.where(ok, np.abs(dg - dz), 0.0)))


def check_gate_formula(res, fw, w):
    """gate is bitwise the probability of the chosen expert, or with
    renormalisation p_j / S with S the fp32 sum in selection order and one
    correctly rounded fp32 division -- recomputed from the GPU's own probs."""
    p = to_f64(res["probs"]).astype(np.float32)
    sel = np.take_along_axis(p, fw["idx"].astype(np.int64), axis=1)
    if w.renorm:
        S = np.zeros(sel.shape[0], np.float32)
        for j in range(sel.shape[1]):
            S = (S + sel[:, j]).astype(np.float32)
        sel = (sel / S[:, None]).astype(np.float32)
    np.testing.assert_array_equal(to_f64(res["gate"]), sel.astype(np.float64), err_msg="gate")


def check_layer_full(res, fw, bw, w, check_bwd=True):
    """Every output of the layer against the full oracle."""
    tol = w.dtype
    R = check_routing_exact(res, fw, w)
    assert_close("probs", to_f64(res["probs"]), fw["probs"], "prob")
    assert_close("gate", to_f64(res["gate"]), fw["gate"], "prob")
    check_gate_formula(res, fw, w)
    np.testing.assert_array_equal(to_f64(res["x_perm"])[:R], fw["x_perm"], err_msg="x_perm")
    if res.get("A") is not None:  # None in the recomputation mode
        assert_close("A", to_f64(res["A"])[:R], fw["A"], tol)
        assert_close("H", to_f64(res["H"])[:R], fw["H"], tol)
    assert_close("Y", to_f64(res["Y"])[:R], fw["Y"], tol)
    assert_close("out", to_f64(res["out"]), fw["out"], tol)
    if res.get("aux") is not None:
        check_aux("aux", res["aux"], res["probs"], fw, w, w.aux_coeff)
    if res.get("aux1") is not None:
        check_aux("aux1", res["aux1"], res["probs"], fw, w, 1.0)
    if check_bwd:
        assert_close("dX", to_f64(res["dX"]), bw["dX"], tol)
        dz = bw["dz"]
        x = fw["x"]
        assert_close("dWr", to_f64(res["dWr"]), bw["dWr"], terms_tol(term_norm(x, dz), tol))
        assert_close("db", to_f64(res["db"]), bw["db"],
                     terms_tol(np.sqrt((dz * dz).sum(axis=0)), tol))
        t1, t2 = expert_grad_tols(fw, bw, tol)
        assert_close("dW1", to_f64(res["dW1"]), bw["dW1"], t1)
        assert_close("dW2", to_f64(res["dW2"]), bw["dW2"], t2)
    return R


def check_aux(name, aux, probs, fw, w, coeff):
    """Balancing loss and drop rate against the oracle.

    Loss: the oracle's fp64 value on its own probabilities, within what the
    probability tolerance (1e-5 relative, 1e-6 absolute per element) allows:
    L = coeff E sum_e f_e P_e with sum_e f_e = 1 moves by at most
    1e-5 L + 1e-6 coeff E.  Against the oracle's formula on the GPU's own
    probabilities the only error left is the kernel's summation: fp32
    partial sums over at most 64 tokens (relative error <= 63 * 2^-24)
    summed in fp64, then one rounding to fp32 -- 4e-6 relative.
    Drop rate: exact integers, one rounding to fp32 (<= 2^-24 < 1e-7)."""
    a = to_f64(aux)
    ref = O.aux_loss(fw["probs"], fw["counts"], w.k, coeff)
    assert abs(a[0] - ref) <= 1e-5 * abs(ref) + 1e-6 * coeff * w.E, (name, a[0], ref)
    own = O.aux_loss(to_f64(probs), fw["counts"], w.k, coeff)
    assert abs(a[0] - own) <= 4e-6 * abs(own) + 1e-30, (name, a[0], own)
    assert abs(a[1] - O.drop_rate(fw["offsets"], w.T, w.k)) <= 1e-7, (name, a[1])


def make_case(T, d, E, k, f, dtype, cf, bias="zero", seed=0, aux_coeff=0.0, renorm=False,
              priority="token", fallback="none", **kw):
    w = W.custom(T, d, E, k, f, dtype=dtype, cf=cf, bias=bias, name=f"T{T}d{d}E{E}k{k}f{f}",
                 aux_coeff=aux_coeff, renorm=renorm, priority=priority, fallback=fallback)
    inp = W.make_inputs(w, seed=seed)
    for key, v in kw.items():
        inp[key] = v
    return w, inp
