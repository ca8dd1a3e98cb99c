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
# Four outputs are sums over the token (row) axis of products whose
# operands were rounded to the storage type upstream: dW1 = x_perm^T dA,
# dW2 = H^T dYp (per expert), dgate = <dOut, Y> and dWr = x^T dz.  Two
# correct implementations that round at the same points still flip single
# upstream roundings (fp32 versus fp64 accumulation before the rounding),
# and a flipped operand moves its summand a_i b_i by at most one unit in the
# last place, u |a_i b_i| (u = 2^-7 for bf16's 8 significant bits, 2^-23 for
# fp32), so one flip moves the sum by at most u ||(a_i b_i)_i||_2.  Where
# the sum cancels, that exceeds rtol |sum| + atol: tests/test_tolerance_needed.py
# shows on the CPU that an fp32-accumulating implementation rounding at the
# oracle's storage points exceeds the stated bound for exactly these four
# outputs (up to 4.5x, dW2 on the expert-share workload's small experts) and
# needs at most 0.76 u ||.||_2 (dW1, dW2) and 0.13 u ||.||_2 (dgate, dWr)
# beyond rtol |sum|.  Their absolute tolerance is therefore
#     max(atol, RED_C[name] u ||(a_i b_i)_i||_2)
# with ||(a_i b_i)_i||_2 = sqrt((a*a)^T (b*b)) from the oracle's own
# operands: two flips' worth for the expert weight gradients, one for dgate
# and dWr.  Every other output, db included, is held to the stated bound.
RED_UNIT = {"bf16": 2.0 ** -7, "f32": 2.0 ** -23}
RED_C = {"dW1": 2.0, "dW2": 2.0, "dgate": 1.0, "dWr": 1.0}

# max |gpu - oracle| / (atol + rtol |oracle|) at the stated tolerance, per
# (case, output): printed by the tests and written to the file named by
# $MOE_PARITY_REPORT at the end of the session (tests/conftest.py)
RATIOS = {}
CASE = ["?"]


def set_case(name):
    CASE[0] = name


def record_ratio(name, got, ref, dtype):
    rtol, atol = TOL[dtype]
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    r = float(np.max(np.abs(got - ref) / (atol + rtol * np.abs(ref))))
    RATIOS[f"{CASE[0]}:{name}"] = r
    return r


def term_norm(a, b):
    """sqrt((a*a)^T (b*b)): per output element, the 2-norm of the summands
    of a^T b (a [n, M], b [n, N])."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.sqrt((a * a).T @ (b * b))


def terms_tol(norm, dtype, name):
    """(rtol, atol array) for the sum output `name` whose summand norms are
    `norm`."""
    rtol, atol = TOL[dtype]
    return rtol, np.maximum(atol, RED_C[name] * RED_UNIT[dtype] * np.asarray(norm, np.float64))


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


def check_expert_grads(dW1, dW2, fw, bw, dtype):
    """dW1 and dW2 (device tensors [E, ...]) against the oracle expert by
    expert, each with its summand-norm tolerance; the ratio at the stated
    tolerance is recorded as the maximum over experts.  Empty experts must
    be exactly zero."""
    off = fw["offsets"]
    worst = {"dW1": 0.0, "dW2": 0.0}
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        for name, got_t, ref, a, b in (("dW1", dW1, bw["dW1"], fw["x_perm"], bw["dA"]),
                                       ("dW2", dW2, bw["dW2"], fw["H"], bw["dYp"])):
            got = to_f64(got_t[e])
            if hi == lo:
                assert np.all(got == 0), f"{name}[e={e}] of an empty expert is not zero"
                continue
            r = record_ratio(name, got, ref[e], dtype)
            worst[name] = max(worst[name], r)
            assert_close(f"{name}[e={e}]", got, ref[e],
                         terms_tol(term_norm(a[lo:hi], b[lo:hi]), dtype, name))
    for name, r in worst.items():
        RATIOS[f"{CASE[0]}:{name}"] = r


def assert_close(name, got, ref, tol):
    rtol, atol = TOL[tol] if isinstance(tol, str) else tol
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if got.size == 0:
        return
    if isinstance(tol, str) and tol in ("bf16", "f32"):
        record_ratio(name, got, ref, tol)
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        at = atol if np.ndim(atol) == 0 else np.broadcast_to(atol, err.shape)[i]
        raise AssertionError(
            f"{name}: {int(bad.sum())}/{bad.size} elements outside rtol={rtol} "
            f"atol={at}; worst at {i}: gpu={got[i]!r} oracle={ref[i]!r}")


def assert_close_sum(name, got, ref, norm, dtype):
    """A sum-over-rows output (dW1, dW2, dgate, dWr): its ratio at the stated
    tolerance is recorded, then it is checked against the summand-norm bound."""
    record_ratio(name, got, ref, dtype)
    assert_close(name, got, ref, terms_tol(norm, dtype, name.split("[")[0]))


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
        assert_close_sum("dWr", to_f64(res["dWr"]), bw["dWr"], term_norm(x, dz), tol)
        assert_close("db", to_f64(res["db"]), bw["db"], tol)
        check_expert_grads(res["dW1"], res["dW2"], fw, bw, tol)
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
