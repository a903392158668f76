"""Pins of the oracle's GEMM steps, weight placement and combine.

* A dense brute force (every token against every expert, masked by the
  selection, no grouping or permutation; dot products as exact Python
  ``math.fsum`` loops) must reproduce the oracle's layer bit for bit.
* Special cases: identical experts make the routed part a single dense SwiGLU
  FFN (the weights sum to 1), so applying the weights twice or never shows.
* Combine closed forms: gate logit 0 gives factor 0.5 exactly, +-inf gives 1/0,
  K = 1 without a shared term is the identity, routed_scale 1 changes nothing.
* Hand-derived fixtures in ``tests/golden`` fix the k order, the absence of
  FMA contraction and the bf16 rounding of the shared term.
* Planted mistakes (in a copy of the oracle, on the CPU) must fail a pin.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
import workloads as W

F32 = np.float32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f(b):
    return O.f32_from_bf16(b).astype(np.float64)


def _fsum_dot(a_row, b_row):
    return math.fsum(float(p) for p in a_row * b_row)


def _dense_brute_force(d, ids, w):
    """Every (token, expert) pair evaluated directly; unselected ones masked."""
    cfg = d["cfg"]
    T, H, E, K, I = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I
    x = _f(d["x"])
    wgu = _f(d["w_gu"])
    wd = _f(d["w_d"])
    eo = np.zeros((T, K, H), dtype=np.uint16)
    for t in range(T):
        for e in range(E):
            sel = np.nonzero(ids[t] == e)[0]
            gu = np.array([_fsum_dot(x[t], wgu[e, j]) for j in range(2 * I)], dtype=F32)
            gu = O.f32_from_bf16(O.bf16_from_f32(gu))
            act = O.bf16_from_f32((O.silu(gu[:I]) * gu[I:]).astype(F32))
            a = _f(act)
            y = np.array([_fsum_dot(a, wd[e, h]) for h in range(H)], dtype=F32)
            for k in sel:                       # mask: only selected experts land
                eo[t, k] = O.bf16_from_f32((y * w[t, k]).astype(F32))
    sd = gl = None
    if "w_gu_s" in d:
        ws_gu, ws_d = _f(d["w_gu_s"]), _f(d["w_d_s"])
        Is = cfg.I_s
        sd = np.zeros((T, H), dtype=np.uint16)
        for t in range(T):
            gu = np.array([_fsum_dot(x[t], ws_gu[j]) for j in range(2 * Is)], dtype=F32)
            gu = O.f32_from_bf16(O.bf16_from_f32(gu))
            a = _f(O.bf16_from_f32((O.silu(gu[:Is]) * gu[Is:]).astype(F32)))
            sd[t] = O.bf16_from_f32(np.array([_fsum_dot(a, ws_d[h]) for h in range(H)], F32))
        wg = _f(d["w_g"])[0]
        gl = np.array([_fsum_dot(x[t], wg) for t in range(T)], dtype=F32)
    return eo, sd, gl


def test_dense_brute_force_equals_grouped_oracle_bitwise():
    d = W.make_inputs(1)
    cfg = d["cfg"]
    x, wr = _f(d["x"]), _f(d["w_r"])
    logits = np.array([[_fsum_dot(x[t], wr[e]) for e in range(cfg.E)]
                       for t in range(cfg.T)], dtype=F32)
    res = O.moe_layer(d, keep=True)
    assert np.array_equal(res["logits"], logits)
    ids = np.array([sorted(range(cfg.E), key=lambda e: (-logits[t, e], e))[:cfg.K]
                    for t in range(cfg.T)], dtype=np.int32)
    assert np.array_equal(res["ids"], ids)
    eo, sd, gl = _dense_brute_force(d, ids, res["w"])
    assert np.array_equal(res["expert_out"].reshape(cfg.T, cfg.K, cfg.H), eo)
    assert np.array_equal(res["sd"], sd)
    assert np.array_equal(res["gl"], gl)
    out = O.combine_gate(eo, cfg.T, cfg.K, cfg.H, None, 1.0, sd, gl)
    assert np.array_equal(res["out"], out)


def test_dense_brute_force_skewed_small_layer():
    """A small layer with the skewed router bias, K=4, uneven per-expert counts."""
    cfg = W.MoeConfig("small_skewed", 24, 32, 6, 4, 16, skew_bias=True)
    d = W.make_inputs(cfg, seed=21)
    res = O.moe_layer(d, keep=True)
    eo, _, _ = _dense_brute_force(d, res["ids"], res["w"])
    assert np.array_equal(res["expert_out"].reshape(cfg.T, cfg.K, cfg.H), eo)
    assert len(set(np.diff(res["offsets"]).tolist())) > 1


def test_dense_brute_force_grouped_sigmoid_small_layer():
    """The grouped sigmoid router in a small layer: selection within the 4 kept
    groups of 2, unbiased renormalised weights, routed scale 2.5."""
    cfg = W.MoeConfig("small_grouped", 24, 32, 16, 4, 16, I_s=16, router="grouped_sigmoid")
    d = W.make_inputs(cfg, seed=22)
    res = O.moe_layer(d, keep=True)
    s = O.router_scores(res["logits"], "sigmoid").astype(np.float64)
    c = s + d["selection_bias"].astype(np.float64)
    for t in range(cfg.T):
        groups = sorted(range(8), key=lambda g: (-(np.sort(c[t, 2 * g:2 * g + 2])[::-1].sum()), g))
        allowed = [e for e in range(16) if e // 2 in groups[:4]]
        want = sorted(allowed, key=lambda e: (-c[t, e], e))[:4]
        assert res["ids"][t].tolist() == want
        ws = s[t, res["ids"][t]]
        assert np.allclose(res["w"][t], ws / ws.sum(), rtol=1e-6, atol=0)
    eo, sd, gl = _dense_brute_force(d, res["ids"], res["w"])
    assert np.array_equal(res["expert_out"].reshape(cfg.T, cfg.K, cfg.H), eo)
    out = O.combine_gate(eo, cfg.T, cfg.K, cfg.H, None, 2.5, sd, gl)
    assert np.array_equal(res["out"], out)


def _identical_experts(seed=3):
    cfg = W.MoeConfig("identical", 20, 64, 8, 3, 32)
    d = W.make_inputs(cfg, seed=seed)
    d["w_gu"][:] = d["w_gu"][0]
    d["w_d"][:] = d["w_d"][0]
    return cfg, d


def _dense_ffn(d):
    x = _f(d["x"])
    I = d["cfg"].I
    gu = (x @ _f(d["w_gu"][0]).T)
    g, u = gu[:, :I], gu[:, I:]
    a = g / (1 + np.exp(-g)) * u
    return a @ _f(d["w_d"][0]).T


def test_identical_experts_reduce_to_one_dense_ffn():
    cfg, d = _identical_experts()
    res = O.moe_layer(d)
    ref = _dense_ffn(d)
    out = _f(res["out"])
    err = np.abs(out - ref) / (np.sqrt(np.mean(ref ** 2)))
    assert err.max() < 0.05                  # bf16 storage at three points
    # weights once: sum_k w = 1 keeps the scale; twice or never does not
    assert abs(np.sum(out * ref) / np.sum(ref * ref) - 1.0) < 0.01


def test_combine_gate_zero_logit_is_half():
    g = np.random.Generator(np.random.PCG64(5))
    T, K, H = 7, 3, 16
    eo = O.bf16_from_f32(g.standard_normal((T * K, H)).astype(F32))
    sd = O.bf16_from_f32(g.standard_normal((T, H)).astype(F32))
    out0 = O.combine_gate(eo, T, K, H, None, 1.0, sd, np.zeros(T, F32), out_bf16=False)
    half = O.f32_from_bf16(sd) * F32(0.5)     # exact: a power-of-two scale
    acc = np.zeros((T, H), F32)
    for k in range(K):
        acc = (acc + O.f32_from_bf16(eo).reshape(T, K, H)[:, k]).astype(F32)
    assert np.array_equal(out0, (acc + half).astype(F32))
    outp = O.combine_gate(eo, T, K, H, None, 1.0, sd, np.full(T, np.inf, F32), out_bf16=False)
    assert np.array_equal(outp, (acc + O.f32_from_bf16(sd)).astype(F32))
    outn = O.combine_gate(eo, T, K, H, None, 1.0, sd, np.full(T, -np.inf, F32), out_bf16=False)
    assert np.array_equal(outn, acc + F32(0))


def test_combine_identity_and_scale():
    g = np.random.Generator(np.random.PCG64(6))
    T, H = 9, 24
    v = g.standard_normal((T, H)).astype(F32)
    v[0, 0] = -0.0
    eo = O.bf16_from_f32(v)
    out = O.combine_gate(eo, T, 1, H)
    ref = eo.copy()
    ref[0, 0] = 0                             # -0 + (+0) = +0
    assert np.array_equal(out, ref)
    w = g.random((T, 2)).astype(F32)
    eo2 = O.bf16_from_f32(g.standard_normal((T * 2, H)).astype(F32))
    a = O.combine_gate(eo2, T, 2, H, w, 1.0, out_bf16=False)
    b = O.combine_gate(eo2, T, 2, H, w, 0.7, out_bf16=False)
    assert np.array_equal(b, (a * F32(0.7)).astype(F32))


def _golden_cases():
    with open(os.path.join(GOLDEN, "combine_cases.json")) as fh:
        return json.load(fh)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_combine_golden_fixtures(case):
    T, K, H = case["T"], case["K"], case["H"]
    eo = np.array(case["expert_out"], F32).reshape(T * K, H)
    w = None if case["topk_w"] is None else np.array(case["topk_w"], F32)
    sh = None if case["shared"] is None else np.array(case["shared"], F32).reshape(T, H)
    gl = None if case["gate_logit"] is None else np.array(case["gate_logit"], F32)
    out = O.combine_gate(eo, T, K, H, w, case["routed_scale"], sh, gl,
                         eo_bf16=False, sh_bf16=False, out_bf16=False)
    exp = np.array([float.fromhex(s) for s in case["expected_hex"]], F32).reshape(T, H)
    assert np.array_equal(out, exp), (out, exp)


# --- planted mistakes: each must turn a pin red ------------------------------
def _combine_fma(expert_out, T, K, H, topk_w, *a, **kw):
    eo = expert_out.astype(np.float64).reshape(T, K, H)
    acc = np.zeros((T, H), np.float64)
    for k in range(K):
        acc = (np.asarray(topk_w, np.float64).reshape(T, K)[:, k:k + 1] * eo[:, k] + acc
               ).astype(F32).astype(np.float64)
    return acc.astype(F32)


def test_planted_fma_contraction_fails_golden():
    case = next(c for c in _golden_cases() if c["name"] == "no_fma_contraction")
    eo = np.array(case["expert_out"], F32)
    exp = np.array([float.fromhex(s) for s in case["expected_hex"]], F32)
    got = _combine_fma(eo, case["T"], case["K"], case["H"], np.array(case["topk_w"], F32))
    assert not np.array_equal(got.reshape(-1), exp)


def test_planted_reversed_k_order_fails_golden():
    case = next(c for c in _golden_cases() if c["name"] == "sequential_k_order")
    T, K, H = case["T"], case["K"], case["H"]
    eo = np.array(case["expert_out"], F32).reshape(T, K, H)[:, ::-1].reshape(T * K, H)
    out = O.combine_gate(eo, T, K, H, None, 1.0, None, None,
                         eo_bf16=False, sh_bf16=False, out_bf16=False)
    exp = np.array([float.fromhex(s) for s in case["expected_hex"]], F32).reshape(T, H)
    assert not np.array_equal(out, exp)


def test_planted_weights_twice_or_never_fail_identical_expert_pin():
    cfg, d = _identical_experts()
    ref = _dense_ffn(d)
    res = O.moe_layer(d, keep=True)
    eo = res["expert_out"]
    twice = _f(O.combine_gate(eo, cfg.T, cfg.K, cfg.H, res["w"]))
    ratio_twice = np.sum(twice * ref) / np.sum(ref * ref)
    assert abs(ratio_twice - 1.0) > 0.1
    unweighted = O.down_proj(res["act"], d["w_d"], res["sorted_pairs"], res["offsets"], None)
    never = _f(O.combine_gate(unweighted, cfg.T, cfg.K, cfg.H))
    assert abs(np.sum(never * ref) / np.sum(ref * ref) - cfg.K) < 0.05


def test_planted_missing_narrowing_fails_gateup_golden():
    """SiLU-mul on the f32 accumulator (N1 dropped) misses the hand-derived act."""
    case = next(c for c in _gemm_cases()["gateup"] if c["name"] == "narrowing_before_activation")
    acc = O.moe_oracle._dot_f32(_bf(case["x"]), _bf(case["w_gu"])[0])
    I = case["I"]
    bad = O.bf16_from_f32((O.silu(acc[:, :I]) * acc[:, I:]).astype(F32))
    assert not np.array_equal(O.f32_from_bf16(bad), np.array(case["expected_act"], F32))


def test_planted_unstable_grouping_fails_argsort_pin():
    ids = O.topk_ids(O.router_logits(W.make_inputs(2, experts=False)["x"],
                                     W.make_inputs(2, experts=False)["w_r"]), 8)
    flat = ids.reshape(-1)
    bad = np.argsort(flat, kind="quicksort")[::-1]
    bad = bad[np.argsort(flat[bad], kind="stable")]       # grouped, but reversed within
    assert not np.array_equal(bad, O.group_pairs(ids, 128)[1])


def _gemm_cases():
    with open(os.path.join(GOLDEN, "gemm_cases.json")) as fh:
        return json.load(fh)


def _bf(v):
    b = O.bf16_from_f32(np.array(v, F32))
    assert np.array_equal(O.f32_from_bf16(b), np.array(v, F32)), "fixture not bf16-exact"
    return b


@pytest.mark.parametrize("case", _gemm_cases()["gateup"], ids=lambda c: c["name"])
def test_gateup_golden_fixtures(case):
    act = O.gateup_silu(_bf(case["x"]), _bf(case["w_gu"]),
                        np.array(case["sorted_pairs"]), np.array(case["offsets"]), case["K"])
    assert np.array_equal(O.f32_from_bf16(act), np.array(case["expected_act"], F32))


@pytest.mark.parametrize("case", _gemm_cases()["down"], ids=lambda c: c["name"])
def test_down_golden_fixtures(case):
    out = O.down_proj(_bf(case["act"]), _bf(case["w_d"]), np.array(case["sorted_pairs"]),
                      np.array(case["offsets"]), np.array(case["pair_w"], F32))
    assert np.array_equal(O.f32_from_bf16(out), np.array(case["expected_out"], F32))


def test_planted_double_rounding_fails_down_golden():
    case = _gemm_cases()["down"][0]
    acc = O.moe_oracle._dot_f32(_bf(case["act"]), _bf(case["w_d"])[0])
    twice_rounded = O.bf16_from_f32((O.f32_from_bf16(O.bf16_from_f32(acc)) * F32(1.5)).astype(F32))
    assert not np.array_equal(O.f32_from_bf16(twice_rounded),
                              np.array(case["expected_out"], F32))
