"""Pins of the oracle's routing: top-k selection, renormalised weights, grouping.

Top-k is checked against a full stable sort (numpy), the weights against the
literal float64 chain softmax -> top-k -> renormalise and against closed forms
(K = 1, K = E), the grouping against numpy's stable argsort and invariants.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W

F32 = np.float32


def _sort_topk(l, K):
    key = np.where(np.isnan(l), -np.inf, l.astype(np.float64))
    return np.argsort(-key, axis=1, kind="stable")[:, :K].astype(np.int32)


def _cfg_logits(n, T=None):
    d = W.make_inputs(n, T=T, experts=False)
    return O.router_logits(d["x"], d["w_r"], d.get("router_bias")), d["cfg"]


@pytest.mark.parametrize("n,T", [(1, None), (2, None), (3, 512), (4, None), (5, 512)])
def test_topk_equals_full_stable_sort(n, T):
    l, cfg = _cfg_logits(n, T)
    assert np.array_equal(O.topk_ids(l, cfg.K), _sort_topk(l, cfg.K))


def test_topk_ties_nan_and_infinities():
    g = np.random.Generator(np.random.PCG64(7))
    l = g.integers(-3, 3, size=(400, 37)).astype(F32)        # many exact ties
    l[g.random(l.shape) < 0.05] = np.nan
    l[g.random(l.shape) < 0.05] = -np.inf
    l[g.random(l.shape) < 0.01] = np.inf
    l[0, :] = np.nan                                          # all NaN
    l[1, :] = -np.inf
    for K in (1, 2, 5, 37):
        ids = O.topk_ids(l, K)
        assert np.array_equal(ids, _sort_topk(l, K))
        s = np.sort(ids, axis=1)
        assert np.all(np.diff(s, axis=1) > 0)                 # distinct ids
        assert ids.min() >= 0 and ids.max() < 37


def test_topk_rejects_bad_k():
    l = np.zeros((2, 4), F32)
    for K in (0, 5):
        with pytest.raises(ValueError):
            O.topk_ids(l, K)


def _f64_chain(l, K):
    """softmax over all experts in f64, take the top K, renormalise."""
    l64 = l.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ids = _sort_topk(l, K)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("n,T", [(1, None), (2, None), (4, None), (5, 512)])
def test_weights_match_f64_chain_and_sum_to_one(n, T):
    l, cfg = _cfg_logits(n, T)
    ids = O.topk_ids(l, cfg.K)
    w = O.topk_weights(l, ids)
    ref = _f64_chain(l, cfg.K)
    rel = np.abs(w.astype(np.float64) - ref) / ref
    assert rel.max() <= 2.0 ** -20, rel.max()
    s = w.astype(np.float64).sum(axis=1)
    assert np.max(np.abs(s - 1.0)) <= (cfg.K + 2) * 2.0 ** -24
    assert np.all(np.diff(w, axis=1) <= 0)                     # ordered like the logits


def test_weights_k1_is_exactly_one_and_k_eq_e_is_softmax():
    l, cfg = _cfg_logits(1)
    w1 = O.topk_weights(l, O.topk_ids(l, 1))
    assert np.all(w1 == F32(1.0))
    ids = O.topk_ids(l, cfg.E)
    w = O.topk_weights(l, ids)
    l64 = l.astype(np.float64)
    sm = np.exp(l64 - l64.max(axis=1, keepdims=True))
    sm /= sm.sum(axis=1, keepdims=True)
    full = np.take_along_axis(sm, ids.astype(np.int64), axis=1)
    assert np.max(np.abs(w - full) / full) <= 2.0 ** -20


def test_weights_equal_logits_are_uniform():
    l = np.zeros((3, 16), F32)
    for K in (1, 2, 4, 8, 16):
        w = O.topk_weights(l, O.topk_ids(l, K))
        assert np.all(w == F32(1.0) / F32(K))


@pytest.mark.parametrize("n,T", [(1, None), (2, None), (3, 1024), (5, 1024)])
def test_grouping_is_stable_argsort(n, T):
    l, cfg = _cfg_logits(n, T)
    ids = O.topk_ids(l, cfg.K)
    off, sp = O.group_pairs(ids, cfg.E)
    flat = ids.reshape(-1)
    assert np.array_equal(sp, np.argsort(flat, kind="stable"))
    assert off[0] == 0 and off[-1] == flat.size
    assert np.all(np.diff(off) >= 0)
    assert np.array_equal(np.diff(off), np.bincount(flat, minlength=cfg.E))
    for e in range(cfg.E):
        seg = sp[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def test_grouping_edge_cases():
    off, sp = O.group_pairs(np.zeros((0, 2), np.int32), 4)
    assert off.tolist() == [0, 0, 0, 0, 0] and sp.size == 0
    off, sp = O.group_pairs(np.array([[3, 3], [3, 0]], np.int32), 4)
    assert off.tolist() == [0, 1, 1, 1, 4] and sp.tolist() == [3, 0, 1, 2]
    with pytest.raises(ValueError):
        O.group_pairs(np.array([[4]], np.int32), 4)


def test_skewed_router_is_skewed():
    l, cfg = _cfg_logits(5, 1024)
    cnt = np.bincount(O.topk_ids(l, cfg.K).reshape(-1), minlength=cfg.E)
    assert cnt.max() > 10 * cnt.mean()
