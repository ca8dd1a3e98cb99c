"""The CPU oracle against the hand-worked layer in tests/golden/.

The fixture's expected values were derived by hand in closed form (its
"derivation" field walks through every step), so this pins the oracle to
something other than itself: a wrong sign, index, transposed operand or
dropped term anywhere in the forward or backward changes at least one of
the 30-odd named outputs.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from golden_fixture import load

INT_KEYS = ("idx", "counts", "offsets", "row_of", "src_of")
FWD_KEYS = ("z", "probs", "gate", "x_perm", "A", "H", "Y", "out")
BWD_KEYS = ("dYp", "dgate", "dA", "dXp", "dW1", "dW2", "dXe", "dz", "db", "dWr", "dX")


def _workload(cfg):
    return W.custom(cfg["T"], cfg["d"], cfg["E"], cfg["k"], cfg["f"], dtype=cfg["dtype"],
                    cf=cfg["cf"], name="hand_worked")


@pytest.mark.parametrize("exact,tol", [(True, 1e-13), (False, 3e-7)],
                         ids=["fp64-throughout", "fp32-storage"])
def test_oracle_reproduces_the_hand_worked_layer(exact, tol):
    cfg, inp, exp = load("hand_worked_layer.json")
    w = _workload(cfg)
    fw = O.layer_fwd(inp, w, exact=exact)
    bw = O.layer_bwd(inp, w, fw, exact=exact)
    assert fw["C"] == exp["C"]
    for k in INT_KEYS:
        np.testing.assert_array_equal(np.asarray(fw[k]), exp[k], err_msg=k)
    # fp32 storage rounds each stored value once (relative 2^-24); the
    # values reaching dX pass through at most a few such roundings
    for k in FWD_KEYS:
        np.testing.assert_allclose(np.asarray(fw[k], np.float64), exp[k], rtol=tol, atol=tol,
                                   err_msg=k)
    for k in BWD_KEYS:
        np.testing.assert_allclose(np.asarray(bw[k], np.float64), exp[k], rtol=tol, atol=tol,
                                   err_msg=k)


def test_hand_worked_values_are_what_the_steps_say():
    """Internal consistency of the fixture itself (not of the oracle): the
    closed forms obey the identities the steps imply."""
    cfg, inp, exp = load("hand_worked_layer.json")
    p = exp["probs"]
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    # db is the column sum of dz; dWr = x^T dz; dX = dXe + dz Wr^T
    np.testing.assert_allclose(exp["db"], exp["dz"].sum(axis=0), atol=1e-14)
    np.testing.assert_allclose(exp["dWr"], inp["x"].T.astype(np.float64) @ exp["dz"], atol=1e-14)
    np.testing.assert_allclose(exp["dX"], exp["dXe"] + exp["dz"] @ inp["Wr"].T.astype(np.float64),
                               atol=1e-14)
    # the dropped token contributes nothing and receives no gradient
    assert exp["row_of"][2, 0] == -1
    assert not exp["out"][2].any() and not exp["dX"][2].any()
