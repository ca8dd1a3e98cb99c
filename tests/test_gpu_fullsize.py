"""GPU parity at the full sizes of the named workloads (c2_zipf, c3_epshare,
c4_large), in the launch configuration bench.py times.

c2_zipf and c3_epshare are compared against the full oracle.  c4_large is
too large for a full CPU backward: routing is compared in full (bit-exact),
the forward activations and the output of every expert are compared in
full by streaming the oracle expert by expert, the router gradients (dWr,
db) in full from the oracle's gate gradients, dX on sampled tokens and the
expert weight gradients on sampled experts.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_parity_helpers import (assert_close, check_aux, check_gate_formula,
                                check_layer_full, check_routing_exact,
                                expert_grad_tols, logit_error, run_layer, say, term_norm,
                                terms_tol, to_dev, to_f64, to_int)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

TAU = 1e-3  # default router certification margin of the library


@pytest.fixture(scope="module")
def M():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_router_gemm_softmax_amd as M
    return M


def test_c2_zipf_full_layer(M):
    w = W.get("C2")
    inp = W.make_inputs(w, seed=0)
    res = run_layer(M, w, inp)
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    R = check_layer_full(res, fw, bw, w)
    err = logit_error(res, fw)
    counts = fw["counts"]
    say(f"C2 R={R} empty experts={int(np.sum(counts == 0))} max count={int(counts.max())} "
        f"logit err={err:.3g}")
    assert R == w.T * w.k
    assert err <= TAU / 2


def test_c3_epshare_full(M):
    import torch
    w = W.get("C3")
    inp = W.make_inputs(w, seed=0)
    d = {k: to_dev(v) for k, v in inp.items()}
    cfg = M.make_cfg(w.T, w.d, w.E, w.k, w.f, w.dtype, capacity=None)
    Rmax = M.moe_rows_max(cfg)
    e = lambda *s, dt=torch.bfloat16: torch.empty(*s, dtype=dt, device="cuda")
    ws = torch.empty(M.moe_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    A, H, Y = e(Rmax, w.f), e(Rmax, w.f), e(Rmax, w.d)
    out, dYp, dXp = e(w.T, w.d), e(Rmax, w.d), e(Rmax, w.d)
    dg = e(w.T, 1, dt=torch.float32)
    dW1, dW2 = torch.empty_like(d["W1"]), torch.empty_like(d["W2"])
    M.moe_grouped_ffn(cfg, d["x_perm"], d["offsets"], d["W1"], d["W2"], A, H, Y, ws)
    M.moe_combine(cfg, Y, d["row_of"], d["gate"], out)
    M.moe_combine_bwd(cfg, d["dOut"], Y, d["row_of"], d["gate"], dYp, dg)
    M.moe_grouped_ffn_bwd(cfg, d["x_perm"], d["offsets"], d["W1"], d["W2"], A, H, dYp, dXp,
                          dW1, dW2, ws)
    torch.cuda.synchronize()
    fw = O.layer_fwd(inp, w)
    bw = O.layer_bwd(inp, w, fw)
    say("C3 counts", inp["counts"].tolist())
    for name, got, ref in (("A", A, fw["A"]), ("H", H, fw["H"]), ("Y", Y, fw["Y"]),
                           ("out", out, fw["out"]), ("dYp", dYp, bw["dYp"]),
                           ("dXp", dXp, bw["dXp"])):
        assert_close(name, to_f64(got), ref, "bf16")
    # dgate[t] = <dOut[t], Y[row]>: summand norm from the oracle's operands
    dOut = O.to_f64(inp["dOut"])
    rows = inp["row_of"][:, 0]
    gn = np.sqrt(((dOut * fw["Y"][rows]) ** 2).sum(axis=1))[:, None]
    assert_close("dgate", to_f64(dg), bw["dgate"], terms_tol(gn, "bf16"))
    t1, t2 = expert_grad_tols(fw, bw, "bf16")
    assert_close("dW1", to_f64(dW1), bw["dW1"], t1)
    assert_close("dW2", to_f64(dW2), bw["dW2"], t2)


def test_c4_routing_variants(M):
    """C4 with renormalised gates and slot-major capacity priority: the
    routing maps bit-exact and the gates bitwise their formula (forward)."""
    w = W.get("C4").replace(renorm=True, priority="slot")
    inp = W.make_inputs(w, seed=0)
    res = run_layer(M, w, inp, bwd=False)
    fw = O.route(inp, w)
    R = check_routing_exact(res, fw, w)
    check_gate_formula(res, fw, w)
    assert_close("gate", to_f64(res["gate"]), fw["gate"], "prob")
    tok = O.assign(fw["idx"], w.E, fw["C"], "token")[2]
    say(f"C4 slot-major: R={R}, {int(np.sum((tok >= 0) != (fw['row_of'] >= 0)))} "
        f"assignments kept differently from token-major")


def test_c4_large(M):
    w = W.get("C4")
    inp = W.make_inputs(w, seed=0)
    say("C4 inputs ready")
    res = run_layer(M, w, inp)
    say("C4 GPU layer done")
    rnd = O.rounder("bf16")
    r32 = O.rounder("f32")
    fw = O.route(inp, w)
    R = check_routing_exact(res, fw, w)
    err = logit_error(res, fw)
    say(f"C4 routing bit-exact: R={R} dropped={w.T * w.k - R} C={fw['C']} logit err={err:.3g}")
    assert err <= TAU / 2
    assert_close("probs", to_f64(res["probs"]), fw["probs"], "prob")
    assert_close("gate", to_f64(res["gate"]), fw["gate"], "prob")
    check_aux("aux1", res["aux1"], res["probs"], fw, w, 1.0)
    say(f"C4 balancing loss (coefficient 1) {float(to_f64(res['aux1'])[0]):.6f}, "
        f"drop rate {float(to_f64(res['aux1'])[1]):.6f}")

    off, src, k = fw["offsets"], fw["src_of"], w.k
    x = fw["x"]
    dOut = O.to_f64(inp["dOut"])
    gpu = {n: res[n] for n in ("A", "H", "Y", "x_perm")}
    dg = np.zeros((w.T, k))
    out_acc = np.zeros((w.T, w.d))
    keep = {}
    e_sorted = np.argsort(np.diff(off))
    sample_e = sorted({int(e_sorted[-1]), int(e_sorted[len(e_sorted) // 2]),
                       int(e_sorted[0])})
    for e in range(w.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        xe = x[src[lo:hi] // k]
        A, H, Y = O.expert_ffn_fwd(xe, O.to_f64(inp["W1"][e]), O.to_f64(inp["W2"][e]), rnd)
        for name, ref in (("A", A), ("H", H), ("Y", Y)):
            assert_close(f"{name}[e={e}]", to_f64(gpu[name][lo:hi]), ref, "bf16")
        t = src[lo:hi] // k
        j = src[lo:hi] % k
        dg[t, j] = np.einsum("rd,rd->r", dOut[t], Y)
        np.add.at(out_acc, t, fw["gate"][t, j][:, None] * Y)
        if e in sample_e:
            keep[e] = (xe, A, H, Y)
    say("C4 forward activations match for every expert")
    # out: the oracle's combine sums j in ascending order; this sum runs
    # expert by expert (fp64, one rounding), well inside the bf16 tolerance
    assert_close("out", to_f64(res["out"]), rnd(out_acc), "bf16")
    dg = r32(dg)
    dz = O.router_dz(fw["probs"], fw["idx"], fw["row_of"], dg)
    db = r32(dz.sum(axis=0))
    dWr = rnd(x.T @ dz)
    assert_close("dWr", to_f64(res["dWr"]), dWr, terms_tol(term_norm(x, dz), "bf16"))
    assert_close("db", to_f64(res["db"]), db, terms_tol(np.sqrt((dz * dz).sum(axis=0)), "bf16"))
    say("C4 router gradients match")
    # dX on sampled tokens: per-row backward of each kept assignment
    rng = np.random.default_rng(1)
    toks = np.sort(rng.choice(w.T, 48, replace=False))
    dX_ref = np.zeros((len(toks), w.d))
    for n, t in enumerate(toks):
        acc = np.zeros(w.d)
        for jj in range(k):
            r = int(fw["row_of"][t, jj])
            if r < 0:
                continue
            e = int(np.searchsorted(off, r, side="right") - 1)
            W1e, W2e = O.to_f64(inp["W1"][e]), O.to_f64(inp["W2"][e])
            A_r, _, _ = O.expert_ffn_fwd(x[t][None], W1e, W2e, rnd)
            dYp_r = rnd(fw["gate"][t, jj] * dOut[t][None])
            dA_r = rnd((dYp_r @ W2e.T) * O.gelu_tanh_grad(A_r))
            acc += rnd(dA_r @ W1e.T)[0]
        dX_ref[n] = rnd(r32(acc) + dz[t] @ O.to_f64(inp["Wr"]).T)
    assert_close("dX[sampled]", to_f64(res["dX"])[toks], dX_ref, "bf16")
    # expert weight gradients on the sampled experts (full expert backward)
    for e, (xe, A, H, Y) in keep.items():
        lo, hi = int(off[e]), int(off[e + 1])
        t = src[lo:hi] // k
        j = src[lo:hi] % k
        dYe = rnd(fw["gate"][t, j][:, None] * dOut[t])
        _, dW1, dW2, dA = O.expert_ffn_bwd(xe, O.to_f64(inp["W1"][e]),
                                           O.to_f64(inp["W2"][e]), A, H, dYe, rnd)
        assert_close(f"dW1[e={e}]", to_f64(res["dW1"][e]), dW1,
                     terms_tol(term_norm(xe, dA), "bf16"))
        assert_close(f"dW2[e={e}]", to_f64(res["dW2"][e]), dW2,
                     terms_tol(term_norm(H, dYe), "bf16"))
    say(f"C4 dX (sampled) and dW1/dW2 of experts {sorted(keep)} match")
    empty = np.nonzero(np.diff(off) == 0)[0]
    for e in empty[:4]:
        assert np.all(to_f64(res["dW1"][int(e)]) == 0)


def test_c4_recompute_mode_is_bitwise_the_save_mode(M):
    """At C4's size (256 x 256 tiles, split-K tails) the recomputation mode
    still reproduces every output of the save mode bitwise."""
    import torch
    w = W.get("C4")
    inp = W.make_inputs(w, seed=0)
    a = run_layer(M, w, inp)
    keys = ("out", "dX", "dWr", "db", "dW1", "dW2")
    ref = {k: a[k].clone() for k in keys}
    del a
    torch.cuda.empty_cache()
    b = run_layer(M, w, inp, recompute=True)
    assert b["A"] is None and b["H"] is None
    for k in keys:
        assert torch.equal(b[k], ref[k]), k
    say("C4 recompute mode bitwise equal to the save mode")
