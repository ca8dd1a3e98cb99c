"""Pin of the oracle's bf16 storage rounding points (reading R10) to a
hand-worked case, tests/golden/rounding_points_bf16.json.

The fixture pushes one row through the expert FFN, the gate-weighted
combine and their backward with inputs chosen so that every storage
rounding (A, H, Y, out, dYp, dA, dXp, dW1, dW2) shows in a stored bf16
value: dropping a rounding, or moving it past the next step (for example
taking H from the unrounded A), changes at least one output bit.  The
expected bits were derived by hand (the fixture's "derivation" walks
through each), so the oracle is checked against something other than
itself.
"""
import numpy as np

import oracle as O
import oracle.moe_oracle as OM
import workloads as W
from golden_fixture import evaluate, load_raw, symbols

FIX = "rounding_points_bf16.json"


def _bf16_bits(a):
    a = np.asarray(a, np.float32)
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    # every fixture input is bf16-exact
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), a)
    return bits


def _case():
    fx = load_raw(FIX)
    c = fx["config"]
    w = W.custom(c["T"], c["d"], c["E"], c["k"], c["f"], dtype=c["dtype"], cf=None,
                 kind=c["kind"], name="rounding_points")
    inp = {k: _bf16_bits(v) for k, v in fx["inputs"].items() if k != "gate"}
    inp["gate"] = np.asarray(fx["inputs"]["gate"], np.float32)
    for k, v in fx["layout"].items():
        inp[k] = np.asarray(v, np.int32)
    env = symbols(fx)
    ev = lambda v: evaluate(v, env) if isinstance(v, str) else float(v)
    exp = {k: np.vectorize(ev, otypes=[np.float64])(np.asarray(v, dtype=object))
           for k, v in fx["expected"].items()}
    return fx, w, inp, env, exp


def _ulp(v):
    """spacing of bf16 values at v (8 significant bits)"""
    return 2.0 ** (np.floor(np.log2(abs(v))) - 7)


def test_oracle_rounds_at_the_storage_points():
    fx, w, inp, env, exp = _case()
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    got = {**{k: fw[k] for k in ("A", "H", "Y", "out")}, **bw}
    for k, v in exp.items():
        np.testing.assert_array_equal(np.asarray(got[k], np.float64), v, err_msg=k)


def test_fixture_values_are_the_nearest_bf16_to_their_exact_values():
    """The fixture against itself: each stored value is the bf16 value
    nearest to the exact (unrounded) quantity the derivation names, and
    every alternative placement of a rounding gives another value that is
    in turn nearest to its own exact quantity -- so the case tells the
    placements apart."""
    fx, _, _, env, exp = _case()
    for k, expr in fx["unrounded"].items():
        v = evaluate(expr, env)
        r = exp[k].flat[0]
        assert abs(v - r) < 0.5 * _ulp(r), (k, v, r)
        assert v != r  # the rounding does something
    for what, (k, alt) in fx["if_moved"].items():
        a = evaluate(alt, env)
        v = evaluate(fx["if_moved_exact"][what], env)
        assert abs(v - a) < 0.5 * _ulp(a), (what, v, a)
        assert a != exp[k].flat[0], what


def _run(w, inp):
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    return {**{k: fw[k] for k in ("A", "H", "Y", "out")}, **bw}


def _mismatch(got, exp):
    return [k for k, v in exp.items() if not np.array_equal(np.asarray(got[k], np.float64), v)]


def test_the_pin_catches_moved_roundings(monkeypatch):
    """Oracle variants with one storage rounding moved downstream (planted
    here, on the CPU) all fail the pin."""
    fx, w, inp, env, exp = _case()
    real_fwd, real_bwd = O.expert_ffn_fwd, O.expert_ffn_bwd

    def h_from_unrounded_a(xe, W1e, W2e, rnd):
        Ae = np.asarray(xe, np.float64) @ np.asarray(W1e, np.float64)
        H = rnd(O.gelu_tanh(Ae))
        return rnd(Ae), H, rnd(H @ np.asarray(W2e, np.float64))

    def y_from_unrounded_h(xe, W1e, W2e, rnd):
        A = rnd(np.asarray(xe, np.float64) @ np.asarray(W1e, np.float64))
        Hu = O.gelu_tanh(A)
        return A, rnd(Hu), rnd(Hu @ np.asarray(W2e, np.float64))

    def dxp_from_unrounded_da(xe, W1e, W2e, Ae, He, dYe, rnd):
        dX, dW1, dW2, dA = real_bwd(xe, W1e, W2e, Ae, He, dYe, rnd)
        dAu = (dYe @ np.asarray(W2e, np.float64).T) * O.gelu_tanh_grad(Ae)
        return rnd(dAu @ np.asarray(W1e, np.float64).T), dW1, dW2, dA

    def no_dw1_rounding(xe, W1e, W2e, Ae, He, dYe, rnd):
        dX, dW1, dW2, dA = real_bwd(xe, W1e, W2e, Ae, He, dYe, rnd)
        return dX, np.asarray(xe, np.float64).T @ dA, dW2, dA

    for name, fwd, bwd in (("H from the unrounded A", h_from_unrounded_a, real_bwd),
                           ("Y from the unrounded H", y_from_unrounded_h, real_bwd),
                           ("dXp from the unrounded dA", real_fwd, dxp_from_unrounded_da),
                           ("dW1 not rounded", real_fwd, no_dw1_rounding)):
        monkeypatch.setattr(OM, "expert_ffn_fwd", fwd)
        monkeypatch.setattr(OM, "expert_ffn_bwd", bwd)
        assert _mismatch(_run(w, inp), exp), name
    monkeypatch.setattr(OM, "expert_ffn_fwd", real_fwd)
    monkeypatch.setattr(OM, "expert_ffn_bwd", real_bwd)
    assert not _mismatch(_run(w, inp), exp)
