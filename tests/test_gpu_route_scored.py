"""GPU parity of moe_route_scored (sigmoid / full-softmax scores, selection
bias, group-limited selection): ids, weights, expert offsets and the stable
permutation are bit-exact against the oracle's route_scored on the same f32
logits -- DeepSeek-V3-like (sigmoid, bias, 8 groups keep 4 by top-2 sums) and
DeepSeek-V2-like (softmax, 8 groups keep 3 by max, raw weights) router shapes,
E up to 1024 / K up to 32, one expert per group, the multi-segment grouping,
and tie-heavy / NaN / inf logits."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import DEV, assert_bits_equal, bits, to_dev

pytestmark = pytest.mark.gpu
F32 = np.float32

# (T, E, K, score, bias, n_group, topk_group, group_score, renormalize)
CASES = [
    (512, 256, 8, "sigmoid", True, 8, 4, "top2", True),     # DeepSeek-V3-like
    (32, 256, 8, "sigmoid", True, 8, 4, "top2", True),      # the same at decode size
    (512, 160, 6, "softmax", False, 8, 3, "max", False),    # DeepSeek-V2-like
    (300, 128, 8, "sigmoid", False, 1, 1, "max", True),     # plain sigmoid top-k
    (300, 128, 8, "softmax", False, 1, 1, "max", True),
    (200, 64, 4, "softmax", True, 64, 8, "top2", True),     # one expert per group
    (100, 1024, 32, "softmax", True, 32, 4, "top2", False), # largest E and K
    (77, 96, 5, "sigmoid", True, 6, 2, "max", False),       # E not a multiple of 64
    (8192, 256, 8, "sigmoid", True, 8, 4, "top2", True),    # 65536 pairs: segmented grouping
]


def _check(gpu_lib, logits, K, score, bias, n_group, topk_group, gscore, renorm, what):
    T, E = logits.shape
    got = gpu_lib.moe_route_scored(to_dev(logits), K, score,
                                   None if bias is None else to_dev(bias), n_group, topk_group,
                                   gscore, renorm)
    torch.cuda.synchronize()
    ref = O.route_scored(logits, K, score, bias, n_group, topk_group, gscore, renorm)
    names = ("ids", "weights", "offsets", "sorted_pairs")
    n = 0
    for g_, r_, nm in zip(got, ref, names):
        n += assert_bits_equal(bits(g_), r_, f"{what} {nm}")
    assert n == 2 * T * K + (E + 1) + T * K


@pytest.mark.parametrize("T,E,K,score,use_bias,n_group,topk_group,gscore,renorm", CASES)
def test_route_scored_bit_exact(gpu_lib, T, E, K, score, use_bias, n_group, topk_group, gscore,
                                renorm):
    g = np.random.Generator(np.random.PCG64(T * 7 + E * 3 + K))
    logits = (g.standard_normal((T, E)) * 2.0).astype(F32)
    bias = (g.standard_normal(E) * 0.05).astype(F32) if use_bias else None
    what = f"T={T} E={E} K={K} {score} bias={use_bias} groups={n_group}/{topk_group} {gscore}"
    print(what, flush=True)
    _check(gpu_lib, logits, K, score, bias, n_group, topk_group, gscore, renorm, what)


@pytest.mark.parametrize("score,gscore", [("sigmoid", "top2"), ("softmax", "max"),
                                          ("softmax", "top2"), ("sigmoid", "max")])
def test_route_scored_ties_nan_inf(gpu_lib, score, gscore):
    T, E, K = 600, 64, 6
    g = np.random.Generator(np.random.PCG64(17))
    l = g.integers(-3, 3, size=(T, E)).astype(F32)
    l[g.random(l.shape) < 0.05] = np.nan
    l[g.random(l.shape) < 0.05] = -np.inf
    l[g.random(l.shape) < 0.01] = np.inf
    l[0, :] = np.nan
    l[1, :] = -np.inf
    l[2, :] = np.inf
    bias = g.integers(-2, 3, size=E).astype(F32) * F32(0.25)
    for n_group, topk_group in [(1, 1), (8, 2), (16, 5), (64, 6)]:
        _check(gpu_lib, l, K, score, bias, n_group, topk_group, gscore, True,
               f"ties {score} {gscore} groups={n_group}/{topk_group}")
        _check(gpu_lib, l, K, score, None, n_group, topk_group, gscore, False,
               f"ties nobias {score} {gscore} groups={n_group}/{topk_group}")


def test_route_scored_selection_respects_groups(gpu_lib):
    T, E, K = 256, 256, 8
    g = np.random.Generator(np.random.PCG64(23))
    logits = g.standard_normal((T, E)).astype(F32)
    ids, w, off, sp = gpu_lib.moe_route_scored(to_dev(logits), K, "sigmoid", None, 8, 4, "top2",
                                               True)
    torch.cuda.synchronize()
    groups = bits(ids) // 32
    assert all(len(set(r.tolist())) <= 4 for r in groups)
    assert np.all(np.abs(bits(w).astype(np.float64).sum(axis=1) - 1.0) < 1e-6)


def test_route_scored_zero_tokens(gpu_lib):
    logits = torch.empty((0, 64), dtype=torch.float32, device=DEV)
    ids, w, off, sp = gpu_lib.moe_route_scored(logits, 4, "sigmoid", None, 8, 2, "top2", True)
    assert ids.shape == (0, 4) and sp.numel() == 0
