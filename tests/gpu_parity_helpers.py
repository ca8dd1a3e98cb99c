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
# Outputs that are sums over the token (row) axis -- dW1, dW2, dWr, db --
# of products whose inputs were rounded to the storage type upstream: two
# correct implementations that round at the same points still flip single
# upstream roundings (fp32 vs fp64 accumulation before the rounding), and a
# flipped input moves one summand by one unit of the storage type.  With n
# summands of rms size a, the sum has rms ~ sqrt(n) a, while the flips move
# it by ~ u sqrt(rho n) a <= u * rms(sum), u = 2^-8 (bf16) or 2^-23 (fp32),
# rho = fraction of flipped summands.  So the absolute tolerance of these
# outputs is max(atol, u * rms(oracle output)); rtol is unchanged.
RED_UNIT = {"bf16": 2.0 ** -8, "f32": 2.0 ** -23}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_f64(t) -> np.ndarray:
    """device tensor -> float64 numpy (bf16 converted exactly through its bits)."""
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return O.to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def to_int(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int64)


def cfg_of(M, w, route_margin=0.0):
    cap = O.capacity(w.T, w.k, w.E, w.cf)
    return M.make_cfg(w.T, w.d, w.E, w.k, w.f, w.dtype, capacity=cap,
                      route_margin=route_margin)


def red_tol(ref, dtype):
    """(rtol, atol) for a sum over the token axis (see RED_UNIT)."""
    rtol, atol = TOL[dtype]
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    return rtol, max(atol, RED_UNIT[dtype] * rms)


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
        raise AssertionError(
            f"{name}: {int(bad.sum())}/{bad.size} elements outside rtol={rtol} "
            f"atol={atol}; worst at {i}: gpu={got[i]!r} oracle={ref[i]!r}")


def run_layer(M, w, inp, route_margin=0.0, bwd=True):
    """Forward (+ backward) of the layer on the GPU through moe_layer_fwd/bwd."""
    import torch
    cfg = cfg_of(M, w, route_margin)
    d = {k: to_dev(v) for k, v in inp.items()}
    layer = M.MoeLayer(cfg, d["Wr"], d["b"], d["W1"], d["W2"])
    out = layer.forward(d["x"])
    res = dict(out=out, **layer.saved)
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


def check_layer_full(res, fw, bw, w, check_bwd=True):
    """Every output of the layer against the full oracle."""
    tol = w.dtype
    R = check_routing_exact(res, fw, w)
    assert_close("probs", to_f64(res["probs"]), fw["probs"], "prob")
    assert_close("gate", to_f64(res["gate"]), fw["gate"], "prob")
    # gate is bitwise the probability of the chosen expert
    p = to_f64(res["probs"])
    np.testing.assert_array_equal(
        to_f64(res["gate"]), np.take_along_axis(p, fw["idx"].astype(np.int64), axis=1))
    np.testing.assert_array_equal(to_f64(res["x_perm"])[:R], fw["x_perm"], err_msg="x_perm")
    assert_close("A", to_f64(res["A"])[:R], fw["A"], tol)
    assert_close("H", to_f64(res["H"])[:R], fw["H"], tol)
    assert_close("Y", to_f64(res["Y"])[:R], fw["Y"], tol)
    assert_close("out", to_f64(res["out"]), fw["out"], tol)
    if check_bwd:
        assert_close("dX", to_f64(res["dX"]), bw["dX"], tol)
        for key in ("dWr", "db", "dW1", "dW2"):
            assert_close(key, to_f64(res[key]), bw[key], red_tol(bw[key], tol))
    return R


def make_case(T, d, E, k, f, dtype, cf, bias="zero", seed=0, **kw):
    w = W.custom(T, d, E, k, f, dtype=dtype, cf=cf, bias=bias, name=f"T{T}d{d}E{E}k{k}f{f}")
    inp = W.make_inputs(w, seed=seed)
    for key, v in kw.items():
        inp[key] = v
    return w, inp
