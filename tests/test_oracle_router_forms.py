"""Pins of the oracle's general router (sigmoid / biased / group-limited).

* hand-derived fixtures (tests/golden/router_cases.json);
* the selection against an independent brute force: group and expert ranks
  by a full sort with explicit keys, on small random cases with ties;
* softmax scores against float64 softmax, the butterfly sum against the
  exact (fsum) sum, exactly on integer data;
* special cases that reduce to the ungrouped router: one group, or one
  expert per group with K groups kept.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle as O

F32 = np.float32
GOLD = os.path.join(os.path.dirname(__file__), "golden", "router_cases.json")


def _cases():
    return json.load(open(GOLD))


@pytest.mark.parametrize("form", ["max", "top2"])
def test_golden_selection(form):
    for case in _cases()["selection_cases"]:
        s = np.array(case["scores"], F32)
        got = O.select_scored(s, case["K"], None, case["n_group"], case["topk_group"], form)
        assert got.tolist() == case["expected"][form], case["name"]


@pytest.mark.parametrize("renorm", [True, False])
def test_golden_route(renorm):
    for case in _cases()["route_cases"]:
        l = np.array(case["logits"], F32)
        b = None if case["bias"] is None else np.array(case["bias"], F32)
        ids, w, off, sp = O.route_scored(l, case["K"], case["score"], b, case["n_group"],
                                         case["topk_group"], case["group_score"], renorm)
        assert ids.tolist() == case["expected_ids"], case["name"]
        key = "renormalize" if renorm else "raw"
        assert w.tolist() == case["expected_w"][key], case["name"]


def _brute_select(c, K, n_group, topk_group, form):
    """Independent selection: rank by full sorts with explicit keys."""
    c = [(-math.inf if math.isnan(v) else float(v)) for v in c]
    E = len(c)
    allowed = list(range(E))
    if n_group > 1:
        gs = E // n_group
        scores = []
        for g in range(n_group):
            vals = sorted(c[g * gs:(g + 1) * gs], reverse=True)
            if form == "max" or gs == 1:
                sc = vals[0]
            else:
                sc = float(F32(vals[0]) + F32(vals[1]))
            if math.isnan(sc):
                sc = -math.inf
            scores.append((-sc, g))
        keep = [g for _, g in sorted(scores)[:topk_group]]
        allowed = [e for e in range(E) if e // gs in keep]
    ranked = sorted(allowed, key=lambda e: (-c[e], e))
    return ranked[:K]


@pytest.mark.parametrize("seed", range(6))
def test_selection_equals_brute_force(seed):
    g = np.random.Generator(np.random.PCG64(100 + seed))
    for E, n_group in [(8, 4), (12, 3), (16, 8), (16, 1), (24, 6), (6, 6)]:
        for _ in range(30):
            s = g.integers(-3, 4, size=(1, E)).astype(F32) * F32(0.25)   # many ties
            if g.random() < 0.3:
                s[0, g.integers(0, E)] = np.nan
            gs = E // n_group
            topk_group = int(g.integers(1, n_group + 1))
            K = int(g.integers(1, topk_group * gs + 1))
            bias = g.integers(-2, 3, size=E).astype(F32) * F32(0.125) if g.random() < 0.5 else None
            c = s[0] if bias is None else (s[0] + bias).astype(F32)
            for form in ("max", "top2"):
                got = O.select_scored(s, K, bias, n_group, topk_group, form)[0].tolist()
                assert got == _brute_select(c.tolist(), K, n_group, topk_group, form), \
                    (E, n_group, topk_group, K, form, s, bias)


def test_tree_sum_exact_on_integers_and_close_to_fsum():
    g = np.random.Generator(np.random.PCG64(5))
    z = g.integers(0, 1000, size=(50, 1000)).astype(F32)        # every partial sum exact
    assert np.array_equal(O.tree_sum64(z), z.astype(np.float64).sum(axis=1).astype(F32))
    for E in (1, 7, 64, 65, 160, 256, 1024):
        z = g.random((40, E)).astype(F32)
        exact = np.array([math.fsum(r) for r in z.astype(np.float64)])
        got = O.tree_sum64(z).astype(np.float64)
        bound = (math.ceil(E / 64) + 6) * 2.0 ** -24 * np.abs(z).astype(np.float64).sum(axis=1)
        assert np.all(np.abs(got - exact) <= bound), E


@pytest.mark.parametrize("E", [8, 64, 160, 256])
def test_softmax_scores_close_to_float64(E):
    g = np.random.Generator(np.random.PCG64(E))
    l = (g.standard_normal((64, E)) * 3).astype(F32)
    s = O.router_scores(l, "softmax").astype(np.float64)
    l64 = l.astype(np.float64)
    ref = np.exp(l64 - l64.max(axis=1, keepdims=True))
    ref /= ref.sum(axis=1, keepdims=True)
    # the f32 difference d = l - m (a relative error of exp(d) up to |d| ulp),
    # pexp (~1.2 ulp), the sum (E adds) and the divide
    d = np.abs(l64 - l64.max(axis=1, keepdims=True))
    assert np.all(np.abs(s - ref) <= (d + E / 32 + 8) * 2.0 ** -24 * ref + 1e-45)
    assert np.all(np.abs(s.sum(axis=1) - 1.0) < 1e-5)


def test_sigmoid_scores_are_the_sigmoid():
    l = np.linspace(-30, 30, 601, dtype=F32)[None, :]
    s = O.router_scores(l, "sigmoid").astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-l.astype(np.float64)))
    assert np.all(np.abs(s - ref) <= 4 * 2.0 ** -24 * ref + 1e-45)


def test_one_group_softmax_renormalised_matches_ungrouped_router():
    g = np.random.Generator(np.random.PCG64(9))
    l = g.standard_normal((300, 128)).astype(F32)              # no ties
    ids0, w0, off0, sp0 = O.route(l, 8)
    ids, w, off, sp = O.route_scored(l, 8, "softmax", None, 1, 1, "max", True)
    assert np.array_equal(ids, ids0) and np.array_equal(off, off0) and np.array_equal(sp, sp0)
    assert np.all(np.abs(w - w0) <= 6 * 2.0 ** -24 * w0)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_one_expert_per_group_reduces_to_plain_topk(score):
    g = np.random.Generator(np.random.PCG64(11))
    l = g.standard_normal((200, 32)).astype(F32)
    b = (g.standard_normal(32) * 0.1).astype(F32)
    for form in ("max", "top2"):
        a = O.route_scored(l, 4, score, b, 32, 4, form, True)
        z = O.route_scored(l, 4, score, b, 1, 1, "max", True)
        assert np.array_equal(a[0], z[0]) and np.array_equal(a[1], z[1])


def test_raw_weights_are_the_unbiased_scores_and_renormalised_sum_to_one():
    g = np.random.Generator(np.random.PCG64(13))
    l = g.standard_normal((100, 64)).astype(F32)
    b = (g.standard_normal(64) * 0.5).astype(F32)
    s = O.router_scores(l, "sigmoid")
    ids, w, _, _ = O.route_scored(l, 6, "sigmoid", b, 8, 3, "top2", False)
    assert np.array_equal(w, np.take_along_axis(s, ids.astype(np.int64), axis=1))
    ids2, w2, _, _ = O.route_scored(l, 6, "sigmoid", b, 8, 3, "top2", True)
    assert np.array_equal(ids, ids2)
    assert np.all(np.abs(w2.astype(np.float64).sum(axis=1) - 1.0) < 4e-7)
    # the chosen experts lie in 3 groups of 8
    assert np.all(np.array([len(set((r // 8).tolist())) for r in ids]) <= 3)


def test_planted_mistakes_are_caught():
    """Weights taken from the biased values, or groups scored by max instead
    of the top-2 sum, change a golden case."""
    case = _cases()["route_cases"][0]
    l = np.array(case["logits"], F32)
    b = np.array(case["bias"], F32)
    s = O.router_scores(l, "sigmoid")
    ids = O.select_scored(s, 2, b)
    wrong = np.take_along_axis((s + b).astype(F32), ids.astype(np.int64), axis=1)
    wrong = wrong / wrong.sum(axis=1, keepdims=True)
    assert wrong.tolist() != case["expected_w"]["renormalize"]
    sel = _cases()["selection_cases"][0]
    s2 = np.array(sel["scores"], F32)
    assert O.select_scored(s2, 2, None, 4, 2, "max").tolist() != sel["expected"]["top2"]


def test_refusals():
    s = np.zeros((1, 8), F32)
    with pytest.raises(ValueError):
        O.select_scored(s, 2, None, 3, 1)          # 8 experts do not split into 3 groups
    with pytest.raises(ValueError):
        O.select_scored(s, 5, None, 4, 2)          # 2 groups of 2 hold only 4 experts
    with pytest.raises(ValueError):
        O.router_scores(s, "relu")


# --- the butterfly order of the full-softmax sum and the bias rounding point ---
def _vec(case):
    z = np.zeros((1, case["E"]), F32)
    for e, h in case["nonzero"].items():
        z[0, int(e)] = F32(float.fromhex(h))
    return z


def _butterfly_reversed(z):
    """Planted mistake: lane sums as in the reading, butterfly m = 1 .. 32."""
    T, E = z.shape
    p = np.zeros((T, 64), F32)
    for e in range(E):
        p[:, e % 64] = (p[:, e % 64] + z[:, e]).astype(F32)
    for m in (1, 2, 4, 8, 16, 32):
        p = (p + p[:, np.arange(64) ^ m]).astype(F32)
    return p[:, 0]


def _contiguous_chunks(z):
    """Planted mistake: lane l sums the contiguous chunk [l*c, (l+1)*c)."""
    T, E = z.shape
    c = -(-E // 64)
    p = np.zeros((T, 64), F32)
    for lane in range(64):
        for e in range(lane * c, min(E, (lane + 1) * c)):
            p[:, lane] = (p[:, lane] + z[:, e]).astype(F32)
    for m in (32, 16, 8, 4, 2, 1):
        p = (p + p[:, np.arange(64) ^ m]).astype(F32)
    return p[:, 0]


def _sequential(z):
    acc = np.zeros(z.shape[0], F32)
    for e in range(z.shape[1]):
        acc = (acc + z[:, e]).astype(F32)
    return acc


def _lane_decreasing(z):
    """Planted mistake: each lane adds its elements in decreasing e."""
    T, E = z.shape
    p = np.zeros((T, 64), F32)
    for e in reversed(range(E)):
        p[:, e % 64] = (p[:, e % 64] + z[:, e]).astype(F32)
    for m in (32, 16, 8, 4, 2, 1):
        p = (p + p[:, np.arange(64) ^ m]).astype(F32)
    return p[:, 0]


_MUTANT_SUMS = {"reversed_butterfly": _butterfly_reversed, "contiguous_chunks": _contiguous_chunks,
                "sequential": _sequential, "lane_decreasing_e": _lane_decreasing}


@pytest.mark.parametrize("case", _cases()["sum_order_cases"], ids=lambda c: c["name"])
def test_golden_butterfly_sum_order(case):
    got = O.tree_sum64(_vec(case))
    assert got.tolist() == [float.fromhex(case["expected_hex"])], (case["name"], got)


@pytest.mark.parametrize("case", _cases()["sum_order_cases"], ids=lambda c: c["name"])
def test_planted_sum_orders_fail_golden(case):
    exp = float.fromhex(case["expected_hex"])
    for name, h in case["mutants_hex"].items():
        got = _MUTANT_SUMS[name](_vec(case))
        assert got.tolist() == [float.fromhex(h)], name     # the fixture separates them
        assert got[0] != exp, name


def _softmax_logits(case):
    l = np.full((1, case["E"]), F32(case["other_logit"]), F32)
    for e, h in case["logits_hex"].items():
        l[0, int(e)] = F32(float.fromhex(h))
    return l


@pytest.mark.parametrize("case", _cases()["softmax_sum_order_cases"], ids=lambda c: c["name"])
def test_golden_softmax_denominator_order(case):
    l = _softmax_logits(case)
    s = O.router_scores(l, "softmax")
    assert float(s[0, 0]) == float.fromhex(case["expected_s0_hex"])
    # the route through the softmax router carries the same first weight
    ids, w, _, _ = O.route_scored(l, 2, "softmax", None, 1, 1, "max", False)
    assert ids[0, 0] == 0 and float(w[0, 0]) == float.fromhex(case["expected_s0_hex"])
    # the fixture's premise: the two small terms are each under half an ulp of 1
    z = O.pexp((l - l.max()).astype(F32))
    assert 2.0 ** -25 < float(z[0, 1]) < 2.0 ** -24 and z[0, 1] == z[0, 3]


@pytest.mark.parametrize("case", _cases()["softmax_sum_order_cases"], ids=lambda c: c["name"])
def test_planted_softmax_sum_orders_fail_golden(case):
    l = _softmax_logits(case)
    z = O.pexp((l - l.max()).astype(F32))
    exp = float.fromhex(case["expected_s0_hex"])
    for S in (_sequential(z), np.sum(z, axis=1, dtype=F32), _butterfly_reversed(z),
              _contiguous_chunks(z)):
        s0 = float((z[0, 0] / S[0]).astype(F32))
        assert s0 == float.fromhex(case["mutants_s0_hex"]["sequential_or_pairwise_sum"])
        assert s0 != exp


def _bias_inputs(case):
    x = O.bf16_from_f32(np.array(case["x"], F32))
    w = np.array([[float.fromhex(h) for h in row] for row in case["w_r_hex"]], F32)
    wb = O.bf16_from_f32(w)
    assert np.array_equal(O.f32_from_bf16(wb), w), "fixture not bf16-exact"
    return x, wb, np.array(case["bias"], F32)


@pytest.mark.parametrize("case", _cases()["logit_bias_cases"], ids=lambda c: c["name"])
def test_golden_logit_bias_rounding(case):
    x, wb, b = _bias_inputs(case)
    got = O.router_logits(x, wb, b)
    exp = np.array([[float.fromhex(h) for h in row] for row in case["expected_hex"]], F32)
    assert np.array_equal(got, exp), got


@pytest.mark.parametrize("case", _cases()["logit_bias_cases"], ids=lambda c: c["name"])
def test_planted_float64_bias_add_fails_golden(case):
    x, wb, b = _bias_inputs(case)
    xf = O.f32_from_bf16(x).astype(np.float64)
    wf = O.f32_from_bf16(wb).astype(np.float64)
    bad = (xf @ wf.T + b.astype(np.float64)[None, :]).astype(F32)   # one rounding, after the bias
    mut = np.array([[float.fromhex(h) for h in row]
                    for row in case["mutants_hex"]["bias_added_in_float64"]], F32)
    exp = np.array([[float.fromhex(h) for h in row] for row in case["expected_hex"]], F32)
    assert np.array_equal(bad, mut) and not np.array_equal(bad, exp)
