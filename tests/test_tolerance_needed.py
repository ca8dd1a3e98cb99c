"""Which outputs can be held to the stated bf16 tolerance (rtol 2e-2, atol
1e-2), shown on the CPU with a second, correct implementation.

tests/fp32_emulation.py computes the layer as a GPU does -- float32
products and float32 accumulation, bf16 rounding at the oracle's storage
points.  Its distance to the fp64 oracle is what any correct fp32
implementation must be allowed:
  * every element-wise output (A, H, Y, out, dYp, dA, dXp, dXe, dX) and the
    bias gradient db stay within the stated bound, so the GPU is held to it;
  * the sums over rows dW1, dW2 (per expert), dgate and dWr exceed it where
    the sum cancels (a single flipped upstream rounding moves the sum by up
    to 2^-7 times the norm of its summands), on the named workloads c1_bf16
    and c3_epshare, so the GPU tests give exactly these four the
    summand-norm bound of gpu_parity_helpers (RED_C), which the emulation
    meets.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
import fp32_emulation as F
from gpu_parity_helpers import RED_C, RED_UNIT, term_norm

ELEMENTWISE = ("A", "H", "Y", "out", "dYp", "dA", "dXp", "dXe", "dX", "db")


def _norms(w, inp, fw, bw):
    off = fw["offsets"]
    n1 = np.zeros(bw["dW1"].shape)
    n2 = np.zeros(bw["dW2"].shape)
    for e in range(w.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            n1[e] = term_norm(fw["x_perm"][lo:hi], bw["dA"][lo:hi])
            n2[e] = term_norm(fw["H"][lo:hi], bw["dYp"][lo:hi])
    dOut = O.to_f64(inp["dOut"])
    gn = np.zeros_like(bw["dgate"])
    for j in range(w.k):
        m = fw["row_of"][:, j] >= 0
        gn[m, j] = np.sqrt(((dOut[m] * fw["Y"][fw["row_of"][m, j]]) ** 2).sum(axis=1))
    out = {"dW1": n1, "dW2": n2, "dgate": gn}
    if w.kind == "layer":
        out["dWr"] = term_norm(fw["x"], bw["dz"])
    return out


@pytest.fixture(scope="module", params=["C1", "C3"])
def case(request):
    w = W.get(request.param)
    inp = W.make_inputs(w, seed=0)
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    ref = {**{k: fw[k] for k in ("A", "H", "Y", "out")}, **bw}
    return w, ref, F.layer(inp, w, fw), _norms(w, inp, fw, bw)


def test_elementwise_outputs_meet_the_stated_tolerance(case):
    w, ref, em, _ = case
    for key in ELEMENTWISE:
        if key in em:
            r = F.ratio(em[key], ref[key])
            assert r <= 1.0, (w.name, key, r)


def test_row_sums_need_the_summand_norm_bound(case):
    """The stated bound fails for a correct implementation on these sums."""
    w, ref, em, _ = case
    exceeds = {"c1_bf16": ("dW2", "dgate", "dWr"), "c3_epshare": ("dW1", "dW2", "dgate")}
    for key in exceeds[w.name]:
        assert F.ratio(em[key], ref[key]) > 1.0, (w.name, key)


def test_row_sums_meet_the_summand_norm_bound(case):
    w, ref, em, norms = case
    for key, nrm in norms.items():
        err = np.abs(em[key] - ref[key])
        bound = 2e-2 * np.abs(ref[key]) + np.maximum(1e-2, RED_C[key] * RED_UNIT["bf16"] * nrm)
        worst = float(np.max(err / bound))
        assert worst <= 1.0, (w.name, key, worst)
