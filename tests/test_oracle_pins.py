"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test ties one oracle function to a closed form, an invariant the pages
state, a brute-force recomputation by a different route, a reduction to a
textbook case, or finite differences.  A dropped term, a wrong sign or
index, or a transposed operand in the oracle fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as W


# ------------------------------------------------------------------ helpers
def _exact_inputs(T, d, E, k, f, seed=0, wstd=0.3, bias=None):
    """Small float64 inputs for exact-mode (no storage rounding) checks."""
    rng = np.random.default_rng(seed)
    inp = dict(x=rng.standard_normal((T, d)),
               Wr=rng.standard_normal((d, E)) * wstd,
               b=(rng.standard_normal(E) if bias is None else bias),
               W1=rng.standard_normal((E, d, f)) * wstd,
               W2=rng.standard_normal((E, f, d)) * wstd,
               dOut=rng.standard_normal((T, d)))
    return inp


def _rational_to_f32(q: Fraction) -> float:
    """Round a rational to float32, ties to even, by exact arithmetic."""
    if q == 0:
        return 0.0
    s = -1 if q < 0 else 1
    a = abs(q)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** max(e - 23, -149)
    n = round(a / quantum)          # Fraction.__round__: half to even
    return s * float(n * quantum)


# ------------------------------------------------------------------ formats
def test_bf16_rne_closed_forms():
    two = 2.0
    cases = [
        (1 + two ** -8, 1.0),                         # tie -> even (down)
        (1 + 3 * two ** -8, 1 + two ** -6),           # tie -> even (up)
        (1 + two ** -8 + two ** -40, 1 + two ** -7),  # above tie: one rounding
        (-(1 + two ** -8 + two ** -40), -(1 + two ** -7)),
        (1 + two ** -8 - two ** -40, 1.0),
        (255.5, 256.0),                               # 8 significant bits
        (two ** -130, two ** -130),                   # bf16 subnormal, exact
        (3 * two ** -134, two ** -132),               # subnormal tie -> even
        (0.0, 0.0),
    ]
    got = O.bf16_rne(np.array([c[0] for c in cases]))
    np.testing.assert_array_equal(got, np.array([c[1] for c in cases]))


def test_bf16_rne_matches_torch_cast_on_fp32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(200000) * np.exp2(rng.integers(-60, 60, 200000))
         ).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_rne(v.astype(np.float64)), ref)


def test_fp32_rne_closed_forms():
    two = 2.0
    xs = np.array([1 + two ** -24, 1 + 3 * two ** -24, 1 + two ** -24 + two ** -40])
    np.testing.assert_array_equal(
        O.fp32_rne(xs), [1.0, 1 + two ** -22, 1 + two ** -23])


def test_storage_bits_roundtrip():
    x = W.make_inputs(W.custom(8, 16, 4, 2, 8, dtype="bf16"))["x"]
    np.testing.assert_array_equal(O.bf16_bits(O.to_f64(x)), x)


# ------------------------------------------------------------------ F1 router
def test_router_logits_equal_exact_rational_sum():
    w = W.custom(T=6, d=24, E=5, k=2, f=8, dtype="bf16", bias="normal")
    inp = W.make_inputs(w, seed=3)
    x, Wr, b = O.to_f64(inp["x"]), O.to_f64(inp["Wr"]), O.to_f64(inp["b"])
    z = O.router_logits(x, Wr, b)
    for t in range(w.T):
        for e in range(w.E):
            q = sum(Fraction(x[t, i]) * Fraction(Wr[i, e]) for i in range(w.d))
            q += Fraction(b[e])
            assert z[t, e] == _rational_to_f32(q), (t, e)


def test_softmax_normalised_shift_invariant_and_two_expert_sigmoid():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((50, 7)) * 4
    p = O.softmax(z)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.softmax(z + 123.25), p, rtol=1e-12, atol=0)
    z2 = rng.standard_normal((50, 2))
    sig = 1.0 / (1.0 + np.exp(z2[:, 1] - z2[:, 0]))
    np.testing.assert_allclose(O.softmax(z2)[:, 0], sig, rtol=1e-13)
    np.testing.assert_array_equal(np.argsort(-z, axis=1, kind="stable"),
                                  np.argsort(-p, axis=1, kind="stable"))  # monotone


@pytest.mark.parametrize("E,k", [(4, 1), (8, 2), (7, 3), (5, 5), (16, 8)])
def test_topk_matches_sorted_brute_force(E, k):
    rng = np.random.default_rng(E * 10 + k)
    # a coarse grid makes exact ties frequent
    z = rng.integers(-3, 4, size=(300, E)).astype(np.float64) * 0.5
    idx = O.topk_select(z, k)
    for t in range(z.shape[0]):
        order = sorted(range(E), key=lambda e: (-z[t, e], e))
        assert list(idx[t]) == order[:k]


def test_topk_ties_from_duplicated_router_columns_go_to_lower_index():
    w = W.custom(T=32, d=16, E=6, k=2, f=8, dtype="bf16")
    inp = W.make_inputs(w, seed=5)
    Wr = inp["Wr"].copy()
    Wr[:, 4] = Wr[:, 1]                      # experts 1 and 4 always tie
    Wr[:, 5] = Wr[:, 1]
    z = O.router_logits(O.to_f64(inp["x"]), O.to_f64(Wr), np.zeros(6))
    assert np.all(z[:, 1] == z[:, 4]) and np.all(z[:, 1] == z[:, 5])
    idx = O.topk_select(z, 2)
    for t in range(w.T):
        if 1 in idx[t] or 4 in idx[t] or 5 in idx[t]:
            # among the tied trio the lower index always comes first
            picked = [e for e in idx[t] if e in (1, 4, 5)]
            assert picked == sorted(picked) and picked[0] == 1


def test_negative_zero_equals_positive_zero_in_selection():
    z = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]])
    np.testing.assert_array_equal(O.topk_select(z, 2), [[0, 1], [0, 1]])


# ------------------------------------------------------------------ F2 capacity / maps
def test_capacity_closed_forms():
    assert O.capacity(64, 1, 4, 1.25) == 20
    assert O.capacity(4096, 2, 8, 1.25) == 1280
    assert O.capacity(32768, 8, 128, 1.0) == 2048
    assert O.capacity(80, 1, 8, 1.1) == 11          # 1.1*10 is exactly 11
    assert O.capacity(81, 1, 8, 1.1) == 12          # 11.1375 -> 12
    assert O.capacity(10, 2, 4, None) is None
    assert O.capacity(10, 2, 4, 0.0) == 0


def _brute_force_maps(idx, E, C, priority="token"):
    """pos of (t,j) = number of (t',j') before it with the same expert, by
    direct pairwise comparison (no running counters).  'token': before
    means t' < t (a token's experts are distinct); 'slot': j' < j, or
    j' = j and t' < t."""
    T, k = idx.shape
    flat_e = idx.reshape(-1)
    flat_t = np.repeat(np.arange(T), k)
    flat_j = np.tile(np.arange(k), T)
    if priority == "token":
        before = lambda a: flat_t < flat_t[a]
    else:
        before = lambda a: (flat_j < flat_j[a]) | ((flat_j == flat_j[a]) & (flat_t < flat_t[a]))
    pos = np.array([np.sum((flat_e == flat_e[a]) & before(a))
                    for a in range(T * k)]).reshape(T, k)
    counts = np.bincount(flat_e, minlength=E)
    kept_mask = pos < (C if C is not None else T * k + 1)
    kept = np.array([np.sum(kept_mask[idx == e]) for e in range(E)])
    offsets = np.concatenate([[0], np.cumsum(kept)])
    row_of = np.where(kept_mask, offsets[idx] + pos, -1)
    return counts, offsets, row_of


@pytest.mark.parametrize("T,E,k,C", [(50, 4, 1, 10), (64, 8, 2, 12),
                                     (40, 5, 3, None), (30, 6, 2, 0),
                                     (1, 3, 2, 1), (33, 16, 8, 5)])
def test_assign_matches_pairwise_brute_force_and_invariants(T, E, k, C):
    rng = np.random.default_rng(T + E + k)
    z = rng.standard_normal((T, E)) + np.linspace(2, 0, E)   # skewed load
    idx = O.topk_select(z, k)
    counts, offsets, row_of, src_of = O.assign(idx, E, C)
    bc, bo, br = _brute_force_maps(idx, E, C)
    np.testing.assert_array_equal(counts, bc)
    np.testing.assert_array_equal(offsets, bo)
    np.testing.assert_array_equal(row_of, br)
    assert counts.sum() == T * k                              # sum counts = T*k
    kept = np.diff(offsets)
    cap = C if C is not None else T * k
    np.testing.assert_array_equal(kept, np.minimum(counts, cap))
    R = offsets[-1]
    assert sorted(row_of[row_of >= 0].tolist()) == list(range(R))
    for r in range(R):                                        # src_of inverts row_of
        t, j = divmod(int(src_of[r]), k)
        assert row_of[t, j] == r
    for e in range(E):                                        # token order per expert
        toks = src_of[offsets[e]:offsets[e + 1]] // k
        assert np.all(np.diff(toks) > 0)
        assert np.all(idx.reshape(-1)[src_of[offsets[e]:offsets[e + 1]]] == e)


@pytest.mark.parametrize("T,E,k,C", [(64, 8, 2, 12), (40, 5, 3, None), (30, 6, 2, 0),
                                     (1, 3, 2, 1), (33, 16, 8, 5), (80, 4, 3, 30)])
def test_slot_priority_matches_pairwise_brute_force(T, E, k, C):
    rng = np.random.default_rng(T * 7 + k)
    z = rng.standard_normal((T, E)) + np.linspace(2, 0, E)
    idx = O.topk_select(z, k)
    counts, offsets, row_of, src_of = O.assign(idx, E, C, "slot")
    bc, bo, br = _brute_force_maps(idx, E, C, "slot")
    np.testing.assert_array_equal(counts, bc)
    np.testing.assert_array_equal(offsets, bo)
    np.testing.assert_array_equal(row_of, br)
    cap = C if C is not None else T * k
    np.testing.assert_array_equal(np.diff(offsets), np.minimum(counts, cap))
    for e in range(E):   # rows of an expert in slot-major order (j, then t)
        a = src_of[offsets[e]:offsets[e + 1]]
        key = (a % k) * T + a // k
        assert np.all(np.diff(key) > 0)


def test_slot_priority_hand_example():
    # token 0 picks (0, 1), token 1 picks (1, 0); C = 1.  Token-major keeps
    # both choices of token 0; slot-major keeps both first choices.
    idx = np.array([[0, 1], [1, 0]])
    _, off_t, row_t, _ = O.assign(idx, 2, 1, "token")
    _, off_s, row_s, _ = O.assign(idx, 2, 1, "slot")
    assert row_t.tolist() == [[0, 1], [-1, -1]]
    assert row_s.tolist() == [[0, -1], [1, -1]]
    assert off_t.tolist() == off_s.tolist() == [0, 1, 2]


def test_slot_priority_with_one_expert_per_token_is_token_priority():
    rng = np.random.default_rng(5)
    idx = O.topk_select(rng.standard_normal((50, 6)), 1)
    for C in (None, 3, 0):
        a = O.assign(idx, 6, C, "token")
        b = O.assign(idx, 6, C, "slot")
        for u, v in zip(a, b):
            np.testing.assert_array_equal(u, v)


def test_identity_fallback_closed_forms():
    """With every assignment dropped the identity fallback returns
    (sum_j gate_j) x: exactly x when k = E (the probabilities sum to 1) or
    when the gates are renormalised; without drops it changes nothing."""
    T, d, E, f = 9, 5, 4, 6
    inp = _exact_inputs(T, d, E, 2, f, seed=21)
    for k, renorm in ((E, False), (2, True)):
        w = W.custom(T, d, E, k, f, cf=0.0, renorm=renorm, fallback="identity")
        fw = O.layer_fwd(inp, w, exact=True)
        assert fw["R"] == 0
        np.testing.assert_allclose(fw["out"], inp["x"], rtol=1e-14, atol=1e-15)
        bw = O.layer_bwd(inp, w, fw, exact=True)
        # no expert ran: the expert weights get no gradient
        assert np.all(bw["dW1"] == 0) and np.all(bw["dW2"] == 0)
    w0 = W.custom(T, d, E, 2, f, cf=None)
    w1 = W.custom(T, d, E, 2, f, cf=None, fallback="identity")
    np.testing.assert_array_equal(O.layer_fwd(inp, w0, exact=True)["out"],
                                  O.layer_fwd(inp, w1, exact=True)["out"])
    with pytest.raises(ValueError):
        O.layer_fwd(inp, W.custom(T, d, E, 2, f, cf=None, fallback="skip"), exact=True)


def test_renormalised_gates_closed_forms():
    rng = np.random.default_rng(6)
    z = rng.standard_normal((20, 7))
    p = O.softmax(z)
    for k in (1, 2, 4):
        idx = O.topk_select(z, k)
        g = O.renorm_gates(p, idx)
        np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-15)
        if k == 1:
            np.testing.assert_array_equal(g, 1.0)
        # only ratios of the selected probabilities matter
        np.testing.assert_allclose(O.renorm_gates(3.0 * p, idx), g, rtol=1e-15)
        # ordered like the selection (z descending)
        assert np.all(np.diff(g, axis=1) <= 0)
    # all experts selected: the probabilities themselves
    idx = O.topk_select(z, 7)
    np.testing.assert_allclose(O.renorm_gates(p, idx),
                               np.take_along_axis(p, idx.astype(np.int64), axis=1),
                               rtol=1e-14)


def test_permute_then_inverse_permute_is_identity_on_kept_tokens():
    T, d, E, k = 40, 6, 5, 1
    rng = np.random.default_rng(9)
    x = rng.standard_normal((T, d))
    idx = O.topk_select(rng.standard_normal((T, E)), k)
    for C in (None, 4):
        counts, offsets, row_of, src_of = O.assign(idx, E, C)
        xp = O.permute(x, src_of, k)
        back = O.combine(xp, row_of, np.ones((T, k)), O.rounder("f32", exact=True))
        kept = row_of[:, 0] >= 0
        np.testing.assert_array_equal(back[kept], x[kept])
        np.testing.assert_array_equal(back[~kept], 0.0)
        if C is None:
            assert kept.all()


# ------------------------------------------------------------------ GELU
def test_gelu_tanh_close_to_erf_gelu_and_limits():
    a = np.linspace(-6, 6, 2401)
    erf_gelu = 0.5 * a * (1 + np.vectorize(math.erf)(a / math.sqrt(2)))
    # the tanh form approximates the erf form to ~5e-4; dropping the cubic
    # term or the sqrt(2/pi) factor breaks this by more than 5e-3
    assert np.max(np.abs(O.gelu_tanh(a) - erf_gelu)) < 5e-4
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(O.gelu_tanh(np.array([30.0, -30.0])), [30.0, 0.0],
                               atol=1e-12)


def test_gelu_tanh_grad_matches_central_difference():
    a = np.linspace(-5, 5, 1001)
    h = 1e-6
    fd = (O.gelu_tanh(a + h) - O.gelu_tanh(a - h)) / (2 * h)
    np.testing.assert_allclose(O.gelu_tanh_grad(a), fd, rtol=1e-7, atol=1e-8)


# ------------------------------------------------------------------ layer fwd
def _dense_masked_reference(inp, w):
    """Every expert on every token, then mask to the top-k and weight by the
    softmax probability (unlimited capacity)."""
    x = inp["x"]
    z = x @ inp["Wr"] + inp["b"]
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    out = np.zeros_like(x)
    for t in range(w.T):
        order = sorted(range(w.E), key=lambda e: (-z[t, e], e))[:w.k]
        for e in range(w.E):
            a = x[t] @ inp["W1"][e]
            h = 0.5 * a * (1 + np.tanh(math.sqrt(2 / math.pi) * (a + 0.044715 * a ** 3)))
            y = h @ inp["W2"][e]
            out[t] += (1.0 if e in order else 0.0) * p[t, e] * y
    return out


@pytest.mark.parametrize("T,d,E,k,f", [(12, 5, 4, 2, 7), (9, 3, 6, 3, 4),
                                       (20, 8, 3, 1, 5)])
def test_unlimited_capacity_equals_dense_masked_mixture(T, d, E, k, f):
    w = W.custom(T, d, E, k, f, cf=None)
    inp = _exact_inputs(T, d, E, k, f, seed=T)
    fw = O.layer_fwd(inp, w, exact=True)
    np.testing.assert_allclose(fw["out"], _dense_masked_reference(inp, w),
                               rtol=1e-12, atol=1e-14)
    assert fw["R"] == T * k


def test_single_expert_top1_is_a_plain_mlp():
    T, d, f = 10, 6, 9
    w = W.custom(T, d, 1, 1, f, cf=None)
    inp = _exact_inputs(T, d, 1, 1, f, seed=4)
    fw = O.layer_fwd(inp, w, exact=True)
    a = inp["x"] @ inp["W1"][0]
    ref = (0.5 * a * (1 + np.tanh(math.sqrt(2 / math.pi) * (a + 0.044715 * a ** 3)))
           ) @ inp["W2"][0]
    np.testing.assert_allclose(fw["out"], ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(fw["gate"], 1.0)


def test_k_equals_E_is_the_softmax_weighted_mixture():
    T, d, E, f = 8, 4, 3, 5
    w = W.custom(T, d, E, E, f, cf=None)
    inp = _exact_inputs(T, d, E, E, f, seed=6)
    fw = O.layer_fwd(inp, w, exact=True)
    np.testing.assert_allclose(fw["gate"].sum(1), 1.0, atol=1e-15)
    np.testing.assert_allclose(fw["out"], _dense_masked_reference(inp, w),
                               rtol=1e-12, atol=1e-14)


def test_zero_capacity_drops_everything():
    T, d, E, k, f = 10, 4, 3, 2, 5
    w = W.custom(T, d, E, k, f, cf=0.0)
    inp = _exact_inputs(T, d, E, k, f, seed=7)
    fw = O.layer_fwd(inp, w, exact=True)
    bw = O.layer_bwd(inp, w, fw, exact=True)
    assert fw["R"] == 0 and np.all(fw["row_of"] == -1)
    assert fw["counts"].sum() == T * k
    np.testing.assert_array_equal(fw["out"], 0.0)
    for key in ("dX", "dWr", "db", "dW1", "dW2"):
        np.testing.assert_array_equal(bw[key], 0.0)


# ------------------------------------------------------------------ layer bwd
def _loss(inp, w):
    """L = <out, dOut> + the load-balancing loss (zero when w.aux_coeff = 0)."""
    fw = O.layer_fwd(inp, w, exact=True)
    return float(np.sum(fw["out"] * inp["dOut"])) + fw["aux_loss"], fw


def _min_topk_gap(z, k):
    zs = -np.sort(-z, axis=1)
    kk = min(k + 1, z.shape[1])
    return np.min(zs[:, :kk - 1] - zs[:, 1:kk]) if kk > 1 else np.inf


@pytest.mark.parametrize("T,d,E,k,f,cf,aux,renorm,prio,fb", [
    (10, 4, 3, 2, 5, None, 0.0, False, "token", "none"),
    (12, 5, 4, 2, 6, 0.75, 0.0, False, "token", "none"),
    (7, 3, 4, 1, 4, 1.0, 0.0, False, "token", "none"),
    (6, 4, 5, 3, 3, None, 0.0, False, "token", "none"),
    (12, 5, 4, 2, 6, 0.75, 0.3, False, "token", "none"),
    (9, 4, 5, 1, 3, None, 2.0, False, "token", "none"),
    (12, 5, 4, 2, 6, 0.75, 0.0, True, "token", "none"),   # renormalised gates, drops
    (6, 4, 5, 3, 3, None, 0.3, True, "token", "none"),    # renormalised, balancing loss
    (12, 5, 4, 2, 6, 0.75, 0.0, False, "slot", "none"),   # slot-major priority, drops
    (10, 4, 4, 3, 5, 0.8, 0.0, True, "slot", "none"),
    (12, 5, 4, 2, 6, 0.75, 0.0, False, "token", "identity"),  # identity fallback
    (10, 4, 4, 3, 5, 0.8, 0.2, True, "slot", "identity"),     # everything at once
])
def test_backward_matches_central_finite_differences(T, d, E, k, f, cf, aux, renorm, prio,
                                                     fb):
    w = W.custom(T, d, E, k, f, cf=cf, aux_coeff=aux, renorm=renorm, priority=prio,
                 fallback=fb)
    seed = 0
    while True:      # pick a seed whose routing margins exceed the step by far
        inp = _exact_inputs(T, d, E, k, f, seed=seed)
        L0, fw = _loss(inp, w)
        if _min_topk_gap(fw["z"], k) > 1e-3:
            break
        seed += 1
    if cf is not None:
        assert fw["R"] < T * k          # the case really drops assignments
    bw = O.layer_bwd(inp, w, fw, exact=True)
    h = 1e-6
    for name, grad in (("x", "dX"), ("Wr", "dWr"), ("b", "db"),
                       ("W1", "dW1"), ("W2", "dW2")):
        base = inp[name]
        fd = np.zeros_like(base)
        for i in np.ndindex(base.shape):
            pert = dict(inp)
            for sgn in (+1, -1):
                arr = base.copy()
                arr[i] += sgn * h
                pert[name] = arr
                Lp, fwp = _loss(pert, w)
                np.testing.assert_array_equal(fwp["idx"], fw["idx"])
                fd[i] += sgn * Lp / (2 * h)
        np.testing.assert_allclose(bw[grad], fd, rtol=1e-5, atol=1e-7,
                                   err_msg=name)


@pytest.mark.parametrize("renorm,fb", [(False, "none"), (True, "none"),
                                       (False, "identity"), (True, "identity")])
def test_backward_matches_torch_autograd_in_fp64(renorm, fb):
    """Independent library cross-check: the same layer written with torch
    autograd (routing and drops taken from the oracle, then held fixed)."""
    torch = pytest.importorskip("torch")
    T, d, E, k, f = 16, 6, 5, 2, 7
    w = W.custom(T, d, E, k, f, cf=1.0, renorm=renorm, fallback=fb)
    inp = _exact_inputs(T, d, E, k, f, seed=11)
    fw = O.layer_fwd(inp, w, exact=True)
    bw = O.layer_bwd(inp, w, fw, exact=True)
    tt = {n: torch.tensor(inp[n], dtype=torch.float64, requires_grad=True)
          for n in ("x", "Wr", "b", "W1", "W2")}
    p = torch.softmax(tt["x"] @ tt["Wr"] + tt["b"], dim=1)
    out = torch.zeros(T, d, dtype=torch.float64)
    for t in range(T):
        sel = p[t, torch.as_tensor(fw["idx"][t].astype(np.int64))]
        gates = sel / sel.sum() if renorm else sel
        for j in range(k):
            if fw["row_of"][t, j] < 0:
                if fb == "identity":     # the token passes the expert unchanged
                    out[t] = out[t] + gates[j] * tt["x"][t]
                continue
            e = int(fw["idx"][t, j])
            hdn = torch.nn.functional.gelu(tt["x"][t] @ tt["W1"][e], approximate="tanh")
            out[t] = out[t] + gates[j] * (hdn @ tt["W2"][e])
    (out * torch.tensor(inp["dOut"])).sum().backward()
    np.testing.assert_allclose(fw["out"], out.detach().numpy(), rtol=1e-12, atol=1e-15)
    for n, g in (("x", "dX"), ("Wr", "dWr"), ("b", "db"), ("W1", "dW1"), ("W2", "dW2")):
        np.testing.assert_allclose(bw[g], tt[n].grad.numpy(), rtol=1e-11, atol=1e-14,
                                   err_msg=n)


def test_empty_expert_weight_grads_are_zero():
    T, d, E, k, f = 12, 4, 4, 1, 5
    w = W.custom(T, d, E, k, f, cf=None)
    inp = _exact_inputs(T, d, E, k, f, seed=12, bias=np.array([5.0, 5.0, -50, -50]))
    fw = O.layer_fwd(inp, w, exact=True)
    assert fw["counts"][2] == 0 and fw["counts"][3] == 0
    bw = O.layer_bwd(inp, w, fw, exact=True)
    np.testing.assert_array_equal(bw["dW1"][2:], 0.0)
    np.testing.assert_array_equal(bw["dW2"][2:], 0.0)


# ------------------------------------------------------------------ ep share
def test_ep_share_combine_is_the_gate_scaled_inverse_permutation():
    w = W.custom(T=40, d=8, E=4, k=1, f=6, dtype="f32", kind="ep_share")
    inp = W.make_inputs(w.replace(dirichlet_alpha=0.5), seed=2)
    fw = O.layer_fwd(inp, w)
    Y = fw["Y"]
    for r in range(w.T):
        t = int(inp["src_of"][r])
        np.testing.assert_array_equal(
            fw["out"][t], O.fp32_rne(inp["gate"][t, 0] * Y[r]))
    assert int(np.sum(inp["counts"])) == w.T
    np.testing.assert_array_equal(np.diff(inp["offsets"]), inp["counts"])


# ------------------------------------------------------------------ workload recipes
def test_zipf_bias_softmax_is_the_zipf_pmf():
    w = W.get("C2")
    b = W.make_inputs(w.replace(T=4, d=8, f=8))["b"].astype(np.float64)
    pmf = np.arange(1, w.E + 1) ** -1.2
    pmf /= pmf.sum()
    np.testing.assert_allclose(O.softmax(b[None])[0], pmf, rtol=1e-6)


def test_named_workload_capacities():
    for name, C in (("C0", 20), ("C1", 1280), ("C4", 2048)):
        w = W.get(name)
        assert O.capacity(w.T, w.k, w.E, w.cf) == C
    assert O.capacity(W.get("C2").T, 2, 64, W.get("C2").cf) is None


# ------------------------------------------------------- load-balancing loss
def test_aux_loss_uniform_routing_is_the_coefficient():
    # every expert gets T k / E assignments and probability 1/E: E * sum 1/E^2 = 1
    T, E, k = 12, 4, 2
    probs = np.full((T, E), 1.0 / E)
    counts = np.full(E, T * k // E)
    assert abs(O.aux_loss(probs, counts, k, 0.01) - 0.01) < 1e-15


def test_aux_loss_collapsed_routing_is_E_times_the_coefficient():
    # top-1, every token on expert 0 with probability 1: f_0 = P_0 = 1
    T, E = 9, 6
    probs = np.zeros((T, E))
    probs[:, 0] = 1.0
    counts = np.zeros(E)
    counts[0] = T
    assert abs(O.aux_loss(probs, counts, 1, 0.5) - 0.5 * E) < 1e-12


def test_aux_gradient_matches_finite_differences_through_the_softmax():
    rng = np.random.default_rng(3)
    T, E, k = 5, 6, 2
    z = rng.standard_normal((T, E))
    counts = rng.integers(0, 4, size=E)
    coeff = 0.7
    no_route = -np.ones((T, k), dtype=np.int32)       # no gate gradient
    idx = np.zeros((T, k), dtype=np.int32)
    dz = O.router_dz(O.softmax(z), idx, no_route, np.zeros((T, k)),
                     O.aux_dp(counts, T, k, coeff))
    h = 1e-6
    fd = np.zeros_like(z)
    for i in np.ndindex(z.shape):
        for sgn in (+1, -1):
            zz = z.copy()
            zz[i] += sgn * h
            fd[i] += sgn * O.aux_loss(O.softmax(zz), counts, k, coeff) / (2 * h)
    np.testing.assert_allclose(dz, fd, rtol=1e-6, atol=1e-9)


def test_drop_rate_closed_forms():
    idx = np.array([[0, 1], [0, 1], [0, 2], [0, 3]], dtype=np.int32)
    _, off_inf, _, _ = O.assign(idx, 4, None)
    assert O.drop_rate(off_inf, 4, 2) == 0.0
    _, off_1, _, _ = O.assign(idx, 4, 1)      # expert 0 keeps 1 of 4, expert 1 1 of 2
    assert O.drop_rate(off_1, 4, 2) == 1.0 - 4 / 8
    _, off_0, _, _ = O.assign(idx, 4, 0)
    assert O.drop_rate(off_0, 4, 2) == 1.0
