"""GPU parity of the HIP path (through the C-ABI) against the CPU oracle.

Integer routing outputs (idx, counts, offsets, row_of, src_of) must be
bit-exact and x_perm bitwise; float outputs within the stated tolerances:
bf16 configs rtol 2e-2 / atol 1e-2, fp32 configs 1e-5 / 1e-5, router
probabilities and gates 1e-5 / 1e-6 in every config.  The four sums over
rows whose stated bound no correct fp32-accumulating implementation meets
(dW1, dW2, dgate, dWr; see tests/test_tolerance_needed.py) take a
summand-norm absolute tolerance instead (gpu_parity_helpers.RED_C).
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_parity_helpers import (TOL, assert_close, assert_close_sum, cfg_of, check_aux,
                                check_layer_full,
                                check_routing_exact, logit_error, make_case,
                                run_layer, say, to_dev, to_f64, to_int)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_router_gemm_softmax_amd as M
    return M


SMALL_CASES = [
    # T, d, E, k, f, dtype, cf, bias
    (64, 32, 4, 1, 64, "f32", 1.25, "zero"),        # the tiny fp32 workload
    (300, 36, 5, 2, 52, "f32", 0.9, "normal"),      # fp32, ragged, drops
    (1000, 264, 6, 2, 200, "bf16", 1.1, "zero"),    # ragged K and N tails, drops
    (777, 128, 16, 4, 96, "bf16", None, "normal"),  # dropless, ragged T
    (513, 64, 40, 3, 136, "bf16", 0.75, "zipf"),    # 2 router N tiles, skew + drops
    (1, 64, 8, 2, 64, "bf16", 1.0, "zero"),         # a single token
    (200, 64, 4, 4, 64, "bf16", None, "normal"),    # k == E
    (260, 48, 130, 8, 40, "bf16", None, "normal"),  # E > 128: 8 router tiles, k = 8
    (300, 64, 256, 16, 64, "bf16", None, "normal"), # E = 256 (largest), k = 16
    (100, 64, 40, 32, 64, "bf16", 1.0, "normal"),   # k = 32 (largest), drops
    (200, 64, 100, 4, 64, "f32", 1.0, "zipf"),      # fp32 router over 100 experts
    (1000, 512, 40, 3, 256, "bf16", 1.25, "normal"),  # router logits in 4 K parts, E < Epad
    (2000, 256, 128, 8, 64, "bf16", 1.0, "normal"),   # router logits in 2 K parts, 8 per lane
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: "T{}d{}E{}k{}f{}{}".format(*c))
def test_layer_matches_oracle_small(M, case):
    T, d, E, k, f, dt, cf, bias = case
    w, inp = make_case(T, d, E, k, f, dt, cf, bias, seed=T)
    say("case", case)
    res = run_layer(M, w, inp)
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    R = check_layer_full(res, fw, bw, w)
    say("  R =", R, "of", T * k, "logit err", logit_error(res, fw))


def test_tiny_workload_named(M):
    w = W.get("C0")
    inp = W.make_inputs(w, seed=0)
    res = run_layer(M, w, inp)
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    check_layer_full(res, fw, bw, w)
    assert fw["C"] == 20


def test_hand_worked_layer(M):
    """The HIP path against the hand-worked three-token layer of
    tests/golden/: expected values derived by hand in closed form, not by
    the oracle (one drop, two experts, every output checked)."""
    from golden_fixture import load
    cfg, inp, exp = load("hand_worked_layer.json")
    w = W.custom(cfg["T"], cfg["d"], cfg["E"], cfg["k"], cfg["f"], dtype=cfg["dtype"],
                 cf=cfg["cf"], name="hand_worked")
    res = run_layer(M, w, inp)
    R = int(exp["offsets"][-1])
    for k in ("idx", "counts", "offsets", "row_of"):
        np.testing.assert_array_equal(to_int(res[k]), exp[k], err_msg=k)
    np.testing.assert_array_equal(to_int(res["src_of"])[:R], exp["src_of"], err_msg="src_of")
    assert_close("probs", to_f64(res["probs"]), exp["probs"], "prob")
    assert_close("gate", to_f64(res["gate"]), exp["gate"], "prob")
    for k in ("x_perm", "A", "H", "Y"):
        assert_close(k, to_f64(res[k])[:R], exp[k], "f32")
    for k in ("out", "dX", "dWr", "db", "dW1", "dW2"):
        assert_close(k, to_f64(res[k]), exp[k], "f32")


def test_zero_capacity_drops_everything(M):
    w, inp = make_case(100, 64, 4, 2, 64, "bf16", 0.0, seed=3)
    res = run_layer(M, w, inp)
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    check_layer_full(res, fw, bw, w)
    assert int(to_int(res["offsets"])[-1]) == 0
    assert np.all(to_f64(res["out"]) == 0) and np.all(to_f64(res["dX"]) == 0)
    assert np.all(to_f64(res["dW1"]) == 0) and np.all(to_f64(res["dWr"]) == 0)


def test_router_weights_only_4_byte_aligned(M):
    """With 8 experts (bf16) the router backward computes dz Wr^T inside the
    unpermute-sum's pass, reading Wr rows as 16-byte vectors, and takes that
    pass only for a 16-byte-aligned Wr.  A Wr the ABI allows but that is only
    4-byte aligned takes the GEMM path instead; both layers match the
    oracle, and their dX agree within the bf16 tolerance."""
    import copy

    import torch
    w, inp = make_case(300, 64, 8, 2, 96, "bf16", 1.0, "normal", seed=11)
    res = run_layer(M, w, inp)
    d = res["_dev"]
    Wr = d["Wr"]
    buf = torch.zeros(Wr.numel() + 2, dtype=Wr.dtype, device="cuda")
    buf[2:].copy_(Wr.reshape(-1))
    Wr_u = buf[2:].view(Wr.shape)
    assert Wr_u.data_ptr() % 16 == 4 and torch.equal(Wr_u, Wr)
    layer = M.MoeLayer(copy.copy(res["_cfg"]), Wr_u, d["b"], d["W1"], d["W2"])
    out = layer.forward(d["x"])
    dX, g = layer.backward(d["x"], d["dOut"])
    torch.cuda.synchronize()
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    check_layer_full(res, fw, bw, w)
    res_u = dict(out=out, dX=dX, **layer.saved, **g)
    check_layer_full(res_u, fw, bw, w)
    assert torch.equal(out, res["out"])  # forward: same kernels
    assert_close("dX aligned vs unaligned Wr", to_f64(dX), to_f64(res["dX"]), "bf16")


def test_one_hot_expert_overflows_capacity(M):
    # a large bias sends every token's first choice to expert 2
    w, inp = make_case(600, 64, 8, 2, 64, "bf16", 1.0, seed=4)
    inp["b"] = np.zeros(8, np.float32)
    inp["b"][2] = 20.0
    res = run_layer(M, w, inp)
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    check_layer_full(res, fw, bw, w)
    assert fw["counts"][2] == 600 and np.diff(fw["offsets"])[2] == fw["C"]


def test_exact_ties_go_to_the_lower_expert(M):
    # duplicated router columns make logits of experts 1, 4 and 6 bitwise equal
    w, inp = make_case(400, 64, 8, 2, 64, "bf16", None, seed=5)
    inp["Wr"][:, 4] = inp["Wr"][:, 1]
    inp["Wr"][:, 6] = inp["Wr"][:, 1]
    res = run_layer(M, w, inp)
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    check_layer_full(res, fw, bw, w)
    ties = np.isin(fw["idx"], [1, 4, 6]).any(axis=1)
    assert ties.sum() > 50


WIDE_MARGIN_CASES = [  # T, d, E, k, renorm
    (512, 64, 64, 6, False),
    (256, 128, 128, 8, True),
    (256, 64, 256, 32, False),   # four 16-lane rows of 16 experts each; ranks past 16
]


@pytest.mark.parametrize("case", WIDE_MARGIN_CASES,
                         ids=lambda c: "T{}E{}k{}{}".format(c[0], c[2], c[3],
                                                            "-renorm" if c[4] else ""))
def test_wide_margin_rescoring_is_canonical(M, case):
    """A certification margin at the median gap of the top-(k+1) logits sends
    most tokens to the fp64 rescoring, with clusters of near-equal logits of
    every shape: several per token, the cluster of rank k reaching into the
    output ranks, and experts below rank k within the margin of it.  Routing
    stays bit-exact with the oracle's canonical top-k and the gates bitwise
    their formula (renormalised over the final order where asked)."""
    T, d, E, k, renorm = case
    w, inp = make_case(T, d, E, k, 64, "bf16", None, "normal", seed=11, renorm=renorm)
    fw = O.layer_fwd(inp, w)
    zs = -np.sort(-fw["z"], axis=1)
    gaps = zs[:, :k] - zs[:, 1:k + 1]
    tau = float(np.median(gaps))
    # the shapes this margin produces (on the canonical logits; the fast
    # ones differ by far less than tau)
    near = gaps < tau
    several = sum(int(np.sum(np.diff(np.concatenate(([0], near[t].astype(int), [0]))) == 1)) >= 2
                  for t in range(T))
    open_end = near[:, k - 1]
    below = np.sum((fw["z"] >= zs[:, k:k + 1] - tau) & (fw["z"] < zs[:, k:k + 1]), axis=1) > 0
    say("tau", tau, "tokens with two clusters", several, "open at rank k", int(open_end.sum()),
        "with experts below rank k in the band", int((open_end & below).sum()))
    assert several > T // 4 and (open_end & below).sum() > T // 4
    res = run_layer(M, w, inp, route_margin=tau)
    bw = O.layer_bwd(inp, w, fw)
    check_layer_full(res, fw, bw, w)


LARGE_T_ROUTER_CASES = [  # T, d, E, k
    (32700, 512, 128, 2),  # 256 row tiles of 128 (60 rows in the last), K in two parts
    (33000, 256, 160, 3),  # 258 row tiles x 2 expert tiles (Epad 256, 96 padded), one K part
]


@pytest.mark.parametrize("case", LARGE_T_ROUTER_CASES, ids=lambda c: "T{}d{}E{}".format(*c[:3]))
def test_router_at_large_token_counts(M, case):
    """The router's logit GEMM at token counts like the largest workload's,
    with a ragged last row tile: K cut into parts whose partial logits the
    select kernel sums, and padded expert columns across two expert tiles.
    Routing stays bit-exact with the oracle, the fast logits within tau/2 of
    the canonical ones, and every other output within tolerance."""
    T, d, E, k = case
    w, inp = make_case(T, d, E, k, 32, "bf16", 1.0, "normal", seed=13)
    res = run_layer(M, w, inp)
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    check_layer_full(res, fw, bw, w)
    err = logit_error(res, fw)
    say("logit error", err)
    assert err <= 1e-3 / 2


def test_zero_tokens(M):
    import torch
    w = W.custom(0, 64, 4, 2, 64, dtype="bf16", cf=None, aux_coeff=0.01)
    cfg = cfg_of(M, w)
    e = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt, device="cuda")
    layer = M.MoeLayer(cfg, e(64, 4), None, e(4, 64, 64), e(4, 64, 64))
    layer.saved["aux"].fill_(-1.0)
    x = e(0, 64)
    out = layer.forward(x)
    dX, g = layer.backward(x, e(0, 64))
    torch.cuda.synchronize()
    assert out.shape == (0, 64)
    assert to_int(layer.saved["counts"]).tolist() == [0] * 4
    assert to_int(layer.saved["offsets"]).tolist() == [0] * 5
    assert np.all(to_f64(g["dW1"]) == 0) and np.all(to_f64(g["dWr"]) == 0)
    assert to_f64(layer.saved["aux"]).tolist() == [0.0, 0.0]


def test_binding_refuses_strided_views(M):
    # refused on the host, before any launch; a contiguous slice passes
    import torch
    a = torch.zeros(8, 16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="dense row-major"):
        M.binding._ptr(a.t())
    assert M.binding._ptr(a[2:]) == a.data_ptr() + 2 * 16 * 2


BALANCE_CASES = [
    # T, d, E, k, f, dtype, cf, bias, alpha
    (513, 64, 40, 3, 136, "bf16", 0.75, "zipf", 1.0),  # skewed loads, drops
    (300, 36, 5, 2, 52, "f32", 0.9, "normal", 0.01),   # the tutorial's coefficient
    (260, 48, 130, 8, 40, "bf16", None, "normal", 0.1),  # E > 128, dropless
]


@pytest.mark.parametrize("case", BALANCE_CASES,
                         ids=lambda c: "T{}E{}k{}{}a{}".format(c[0], c[2], c[3], c[5], c[8]))
def test_layer_with_balancing_loss(M, case):
    """The layer with the load-balancing loss on: its value, the drop rate
    and every gradient (the router's now carry the loss's term) against the
    oracle."""
    T, d, E, k, f, dt, cf, bias, alpha = case
    w, inp = make_case(T, d, E, k, f, dt, cf, bias, seed=T + 1, aux_coeff=alpha)
    say("case", case)
    res = run_layer(M, w, inp)
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    check_layer_full(res, fw, bw, w)
    say("  loss", float(to_f64(res["aux"])[0]), "oracle", fw["aux_loss"],
        "drop", float(to_f64(res["aux"])[1]), "oracle", fw["drop_rate"])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_balancing_gradient_alone(M, dt):
    """dOut = 0: the whole router gradient is the balancing loss's, so a
    dropped or mis-scaled term cannot hide under the task gradient.  The
    router outputs are compared at the tolerance of their dtype after scaling
    by the output's largest magnitude; the expert gradients are exactly 0."""
    w, inp = make_case(700, 128, 16, 4, 96, dt, 1.0, "normal", seed=11, aux_coeff=1.0)
    inp["dOut"] = np.zeros_like(inp["dOut"])
    res = run_layer(M, w, inp)
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    check_aux("aux", res["aux"], res["probs"], fw, w, 1.0)
    rtol, atol = TOL[dt]
    for name in ("dX", "dWr", "db"):
        ref = bw[name]
        scale = float(np.abs(ref).max())
        assert scale > 0, name
        assert_close(name, to_f64(res[name]), ref, (rtol, atol * scale))
    assert np.all(to_f64(res["dW1"]) == 0) and np.all(to_f64(res["dW2"]) == 0)


VARIANT_CASES = [
    # T, d, E, k, f, dtype, cf, bias, renorm, priority, fallback
    (513, 64, 40, 3, 136, "bf16", 0.75, "zipf", True, "slot", "identity"),  # all three
    (1000, 264, 6, 2, 200, "bf16", 1.1, "zero", True, "token", "none"),  # renormalised top-2
    (300, 36, 5, 2, 52, "f32", 0.9, "normal", False, "slot", "identity"),  # fp32
    (260, 48, 130, 8, 40, "bf16", None, "normal", True, "token", "none"),  # E > 128, k = 8
    (100, 64, 40, 32, 64, "bf16", 1.0, "normal", True, "slot", "none"),  # k = 32
    (777, 128, 16, 4, 96, "bf16", 0.6, "normal", False, "token", "identity"),  # many drops
    (200, 64, 4, 4, 64, "bf16", 0.0, "normal", False, "token", "identity"),  # all dropped
    (1, 64, 8, 2, 64, "bf16", 1.0, "zero", True, "slot", "identity"),   # a single token
    (64, 32, 4, 1, 64, "f32", 1.25, "zero", True, "slot", "identity"),  # k = 1: gates 1
    (300, 64, 256, 16, 64, "bf16", 0.5, "normal", True, "slot", "identity"),  # E = 256
]


@pytest.mark.parametrize("case", VARIANT_CASES,
                         ids=lambda c: "T{}E{}k{}{}{}-{}{}".format(
                             c[0], c[2], c[3], c[5], "-renorm" if c[8] else "", c[9],
                             "-identity" if c[10] == "identity" else ""))
def test_routing_variants_match_oracle(M, case):
    """Renormalised gates, slot-major capacity priority and the identity
    fallback of dropped assignments: routing maps bit-exact, gates bitwise
    their formula, every output within tolerance."""
    T, d, E, k, f, dt, cf, bias, renorm, prio, fb = case
    w, inp = make_case(T, d, E, k, f, dt, cf, bias, seed=T + 3, renorm=renorm, priority=prio,
                       fallback=fb)
    say("case", case)
    res = run_layer(M, w, inp)
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    R = check_layer_full(res, fw, bw, w)
    if prio == "slot" and cf is not None:
        # the variant changes which assignments are kept
        tok = O.assign(fw["idx"], E, fw["C"], "token")[2]
        say("  R =", R, "kept sets differ from token-major:",
            bool(np.any((tok >= 0) != (fw["row_of"] >= 0))))
    if renorm and k == 1:
        np.testing.assert_array_equal(to_f64(res["gate"]), 1.0)
    if fb == "identity" and cf == 0.0 and k == E:
        # every assignment dropped, gates summing to 1: the layer returns x
        assert R == 0
        assert_close("out = x", to_f64(res["out"]), O.to_f64(inp["x"]), dt)


@pytest.mark.parametrize("mode", ["save", "recompute", "variants", "c1", "gemm_router"])
def test_step_entry_points_equal_the_layer_entry_points(M, mode):
    """The per-step entry points chained exactly as the header declares them
    (moe_route, moe_permute, moe_router_aux, moe_grouped_ffn, moe_combine;
    moe_combine_bwd, moe_grouped_ffn_bwd, moe_unpermute_bwd writing dXe,
    moe_route_bwd reading it) give bitwise the layer's results and match the
    oracle; in the recomputation mode with no A and H buffers at all; with
    every routing variant on (renormalised gates, slot priority, identity
    fallback), whose extra inputs the step entry points then take; at C1's
    size, many tiles and a split-K tail per GEMM, where the grouped GEMMs'
    M-tile schedule comes from the permute and the combine backward in the
    layer but from the schedule kernel in the steps; and with 12 experts,
    where the router's dX runs on the GEMM (the others, with 8 experts, on
    the VALU)."""
    import torch
    recompute = mode == "recompute"
    var = dict(renorm=True, priority="slot", fallback="identity") if mode == "variants" else {}
    if mode == "c1":
        w = W.get("C1")
        inp = W.make_inputs(w, seed=3)
    elif mode == "gemm_router":
        w, inp = make_case(700, 128, 12, 3, 160, "bf16", 1.0, "normal", seed=5,
                           aux_coeff=0.05)
    else:
        w, inp = make_case(700, 128, 8, 2, 160, "bf16", 1.0, "normal", seed=7,
                           aux_coeff=0.05, **var)
    res = run_layer(M, w, inp, recompute=recompute)
    cfg, d, L = res["_cfg"], res["_dev"], res["_layer"]
    T, E, k = w.T, w.E, w.k
    Rmax = M.moe_rows_max(cfg)
    z = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt, device="cuda")
    probs, idx, gate = z(T, E, dt=torch.float32), z(T, k, dt=torch.int32), z(T, k, dt=torch.float32)
    ws = torch.zeros(M.moe_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    M.moe_route(cfg, d["x"], d["Wr"], d["b"], probs, idx, gate, ws)
    counts, offsets = z(E, dt=torch.int32), z(E + 1, dt=torch.int32)
    row_of, src_of, xp = z(T, k, dt=torch.int32), z(Rmax, dt=torch.int32), z(Rmax, w.d)
    M.moe_permute(cfg, d["x"], idx, counts, offsets, row_of, src_of, xp, ws)
    aux = z(2, dt=torch.float32)
    M.moe_router_aux(cfg, probs, counts, offsets, aux, ws)
    A, H, Y = z(Rmax, w.f), z(Rmax, w.f), z(Rmax, w.d)
    if recompute:
        A = H = None
    M.moe_grouped_ffn(cfg, xp, offsets, d["W1"], d["W2"], A, H, Y, ws)
    out = z(T, w.d)
    M.moe_combine(cfg, Y, row_of, gate, out, x=d["x"])
    dYp, dg = z(Rmax, w.d), z(T, k, dt=torch.float32)
    M.moe_combine_bwd(cfg, d["dOut"], Y, row_of, gate, dYp, dg, x=d["x"])
    dXp, dW1, dW2 = z(Rmax, w.d), torch.zeros_like(d["W1"]), torch.zeros_like(d["W2"])
    M.moe_grouped_ffn_bwd(cfg, xp, offsets, d["W1"], d["W2"], A, H, dYp, dXp, dW1, dW2, ws)
    dXe = z(T, w.d, dt=torch.float32)
    M.moe_unpermute_bwd(cfg, dXp, row_of, dXe, gate=gate, dOut=d["dOut"])
    dX, dWr, db = z(T, w.d), torch.zeros_like(d["Wr"]), z(E, dt=torch.float32)
    M.moe_route_bwd(cfg, d["x"], d["Wr"], probs, idx, row_of, counts, dg, dXe, dX, dWr, db,
                    ws)
    torch.cuda.synchronize()
    R = int(to_int(offsets)[-1])
    for name, a, b in [("probs", probs, res["probs"]), ("idx", idx, res["idx"]),
                       ("gate", gate, res["gate"]), ("offsets", offsets, res["offsets"]),
                       ("row_of", row_of, res["row_of"]), ("out", out, res["out"]),
                       ("aux", aux, res["aux"]),
                       ("dX", dX, res["dX"]), ("dWr", dWr, res["dWr"]), ("db", db, res["db"]),
                       ("dW1", dW1, res["dW1"]), ("dW2", dW2, res["dW2"])]:
        assert torch.equal(a, b), name
    for name, a, b in [("x_perm", xp, res["x_perm"]), ("A", A, res["A"]),
                       ("Y", Y, res["Y"]), ("src_of", src_of, res["src_of"])]:
        if a is None:
            assert b is None, name
            continue
        assert torch.equal(a[:R], b[:R]), name
    # the chain's own outputs against the oracle
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    assert_close("dXe", to_f64(dXe), bw["dXe"], "bf16")
    assert_close("dX", to_f64(dX), bw["dX"], "bf16")
    gn = np.zeros_like(bw["dgate"])
    dOut = O.to_f64(inp["dOut"])
    for j in range(w.k):
        m = fw["row_of"][:, j] >= 0
        gn[m, j] = np.sqrt(((dOut[m] * fw["Y"][fw["row_of"][m, j]]) ** 2).sum(axis=1))
        if w.fallback == "identity":   # dropped: <dOut, x>
            gn[~m, j] = np.sqrt(((dOut[~m] * fw["x"][~m]) ** 2).sum(axis=1))
    assert_close_sum("dgate", to_f64(dg), bw["dgate"], gn, "bf16")


RECOMPUTE_CASES = [
    # T, d, E, k, f, dtype, cf, bias, alpha
    (1000, 264, 6, 2, 200, "bf16", 1.1, "zero", 0.0),   # ragged K and N tails, drops
    (300, 36, 5, 2, 52, "f32", 0.9, "normal", 0.01),    # fp32, balancing loss on
    (260, 48, 130, 8, 40, "bf16", None, "normal", 0.0),  # many experts, empty ones
]

SAME_IN_BOTH_MODES = ("probs", "idx", "gate", "counts", "offsets", "row_of", "out", "dX",
                      "dWr", "db", "dW1", "dW2", "aux", "aux1")


@pytest.mark.parametrize("case", RECOMPUTE_CASES,
                         ids=lambda c: "T{}E{}k{}{}".format(c[0], c[2], c[3], c[5]))
def test_recompute_mode_is_bitwise_the_save_mode(M, case):
    """Selective recomputation (A and H not saved, recomputed in backward)
    changes memory, not results: every output is bitwise that of the save
    mode, and so within the oracle's tolerances."""
    import torch
    T, d, E, k, f, dt, cf, bias, alpha = case
    w, inp = make_case(T, d, E, k, f, dt, cf, bias, seed=T + 2, aux_coeff=alpha)
    a = run_layer(M, w, inp)
    b = run_layer(M, w, inp, recompute=True)
    assert b["A"] is None and b["H"] is None
    for key in SAME_IN_BOTH_MODES:
        assert torch.equal(a[key], b[key]), key
    R = int(to_int(a["offsets"])[-1])
    for key in ("src_of", "x_perm", "Y"):
        assert torch.equal(a[key][:R], b[key][:R]), key
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    check_layer_full(b, fw, bw, w)


@pytest.mark.parametrize("name", ["C1", "C2"])
def test_recompute_mode_named_workloads_bitwise(M, name):
    import torch
    w = W.get(name)
    inp = W.make_inputs(w, seed=0)
    a = run_layer(M, w, inp)
    b = run_layer(M, w, inp, recompute=True)
    for key in SAME_IN_BOTH_MODES:
        assert torch.equal(a[key], b[key]), key


def test_runs_are_bitwise_deterministic(M):
    import torch
    w, inp = make_case(1500, 256, 16, 2, 384, "bf16", 1.0, "normal", seed=8, aux_coeff=0.01)
    a = run_layer(M, w, inp)
    b = run_layer(M, w, inp)
    for key in ("probs", "idx", "gate", "counts", "offsets", "row_of", "out", "dX",
                "dWr", "db", "dW1", "dW2", "aux", "aux1"):
        assert torch.equal(a[key], b[key]), key
    R = int(to_int(a["offsets"])[-1])
    for key in ("src_of", "x_perm", "A", "H", "Y"):
        assert torch.equal(a[key][:R], b[key][:R]), key


def test_c1_full_layer_matches_oracle(M):
    w = W.get("C1")
    inp = W.make_inputs(w, seed=0)
    res = run_layer(M, w, inp)
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    R = check_layer_full(res, fw, bw, w)
    err = logit_error(res, fw)
    say("C1 R", R, "logit err", err)
    assert err <= 1e-3 / 2


def test_layer_step_replays_from_a_hip_graph(M):
    """The whole forward + backward enqueues no allocation, copy or memset,
    so it can be captured once into a HIP graph and replayed: every replay
    (with the program's own eager work and synchronisations between them)
    gives bitwise the eager step's results."""
    import torch
    w, inp = make_case(700, 128, 8, 2, 160, "bf16", 1.0, "normal", seed=9, aux_coeff=0.01)
    cfg = cfg_of(M, w)
    d = {k: to_dev(v) for k, v in inp.items()}
    layer = M.MoeLayer(cfg, d["Wr"], d["b"], d["W1"], d["W2"], diagnostics=True)
    out = torch.empty_like(d["x"])
    dX = torch.empty_like(d["x"])
    grads = layer.alloc_grads()

    def step():
        layer.forward(d["x"], out)
        layer.backward(d["x"], d["dOut"], dX, grads)

    keys = ("out", "dX", "dWr", "db", "dW1", "dW2", "aux")
    snap = lambda: {"out": out.clone(), "dX": dX.clone(), "aux": layer.saved["aux"].clone(),
                    **{k: v.clone() for k, v in grads.items()}}
    step()
    torch.cuda.synchronize()
    ref = snap()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        for t in (out, dX, *grads.values()):   # clobber the outputs eagerly
            t.fill_(float("nan") if t.is_floating_point() else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snap()
        for k in keys:
            assert torch.equal(got[k], ref[k]), (r, k)


def test_kernel_probe_records_the_probed_launches_only(M):
    """A caller-owned probe in cfg times exactly the launches of its kernel
    (the split-K fixup under its own id), stops at its capacity, and leaves
    every result bitwise unchanged."""
    import torch
    w = W.get("C1")
    inp = W.make_inputs(w, seed=0)
    res = run_layer(M, w, inp)
    layer, d = res["_layer"], res["_dev"]
    probe = M.KernelProbe("GEMM_DH", 3)
    probe.attach(layer.cfg)
    outs = []
    for _ in range(4):
        out = layer.forward(d["x"])
        dX, g = layer.backward(d["x"], d["dOut"])
        outs.append((out, dX, g["dW1"]))
    torch.cuda.synchronize()
    probe.detach(layer.cfg)
    ms, n, each = probe.read()
    probe.close()
    assert n == 3 and all(t > 0 for t in each), (n, each)
    for out, dX, dW1 in outs:
        assert torch.equal(out, res["out"]) and torch.equal(dX, res["dX"])
        assert torch.equal(dW1, res["dW1"])
    fix = M.KernelProbe("GEMM_FIXUP", 64)
    fix.attach(layer.cfg)
    layer.backward(d["x"], d["dOut"])
    torch.cuda.synchronize()
    fix.detach(layer.cfg)
    _, nf, _ = fix.read()
    fix.close()
    # the dH and dX GEMMs' split-K fixups and the weight gradients' slab sums
    # (no-ops here: no expert of this layer is split)
    assert nf == 4
