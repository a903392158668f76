"""GPU parity of moe_route: top-k ids, renormalised weights, expert offsets
and the stable permutation are bit-exact against the oracle, fed the same f32
logits (every workload at full size, extra seeds, tie-heavy / NaN / inf
logits, E not a multiple of 64, K up to 32, E = 1024)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_helpers import DEV, assert_bits_equal, bits, to_dev

pytestmark = pytest.mark.gpu
F32 = np.float32


def _check(gpu_lib, logits, K, what):
    T, E = logits.shape
    ids, w, off, sp = gpu_lib.moe_route(to_dev(logits), K)
    torch.cuda.synchronize()
    r_ids, r_w, r_off, r_sp = O.route(logits, K)
    n = assert_bits_equal(bits(ids), r_ids, what + " ids")
    n += assert_bits_equal(bits(w), r_w, what + " weights")
    n += assert_bits_equal(bits(off), r_off, what + " offsets")
    n += assert_bits_equal(bits(sp), r_sp, what + " sorted_pairs")
    assert n == 2 * T * K + (E + 1) + T * K
    return bits(ids), bits(sp)


@pytest.mark.parametrize("n,seed", [(1, None), (2, None), (3, None), (4, None), (5, None),
                                    (1, 11), (1, 12), (2, 11), (2, 12), (2, 13), (4, 11), (4, 12)])
def test_route_workloads_bit_exact(gpu_lib, n, seed):
    d = W.make_inputs(n, seed, experts=False)
    print(f"route cfg={n} seed={d['seed']} T={d['cfg'].T}", flush=True)
    logits = O.router_logits(d["x"], d["w_r"], d.get("router_bias"))
    _check(gpu_lib, logits, d["cfg"].K, f"cfg{n}")


@pytest.mark.parametrize("T,E,K", [(777, 37, 1), (777, 37, 5), (300, 37, 32), (129, 1024, 32),
                                   (64, 1024, 32), (65, 37, 5), (64, 64, 64 // 2),
                                   (64, 1, 1), (1, 8, 8), (5000, 256, 8)])
def test_route_ties_nan_inf(gpu_lib, T, E, K):
    g = np.random.Generator(np.random.PCG64(T * 1000 + E + K))
    l = g.integers(-3, 3, size=(T, E)).astype(F32)
    l[g.random(l.shape) < 0.05] = np.nan
    l[g.random(l.shape) < 0.05] = -np.inf
    l[g.random(l.shape) < 0.01] = np.inf
    l[0, :] = np.nan
    if T > 1:
        l[1, :] = -np.inf
    _check(gpu_lib, l, K, f"ties T={T} E={E} K={K}")


def test_route_is_deterministic(gpu_lib):
    d = W.make_inputs(5, experts=False)
    logits = to_dev(O.router_logits(d["x"], d["w_r"], d["router_bias"]))
    a = [bits(t).copy() for t in gpu_lib.moe_route(logits, 8)]
    b = [bits(t).copy() for t in gpu_lib.moe_route(logits, 8)]
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("T,E,K", [(513, 128, 8), (512, 128, 8), (3000, 1024, 32), (8192, 256, 8),
                                   (8200, 256, 8), (4100, 128, 8), (640, 64, 7), (2048, 1024, 8)])
def test_route_multi_segment_grouping_with_dirty_workspace(gpu_lib, T, E, K):
    """Pair counts around the single-workgroup limit (4096 pairs) and far above
    it (1024-pair segments, a partial last one), on both sides of the largest
    count table (segments x experts = 16,384) whose scan runs inside the
    scatter launch: 8192 x 256 x 8 and 2048 x 1024 x 8 (more experts than
    threads) at it, 8200 x 256 x 8 just past it; the caller's
    workspace starts full of garbage and the result must not depend on it."""
    g = np.random.Generator(np.random.PCG64(T + E + K))
    l = g.standard_normal((T, E)).astype(F32)
    l[:, :3] += 4.0                        # a few hot experts: long, uneven segments
    need = gpu_lib.moe_route_workspace_bytes(T, E, K)
    ws = torch.full((max(need, 16),), 0xA5, dtype=torch.uint8, device=DEV)
    out = [bits(t).copy() for t in gpu_lib.moe_route(to_dev(l), K, workspace=ws)]
    torch.cuda.synchronize()
    r_ids, r_w, r_off, r_sp = O.route(l, K)
    assert_bits_equal(out[0], r_ids, "ids")
    assert_bits_equal(out[1], r_w, "weights")
    assert_bits_equal(out[2], r_off, "offsets")
    assert_bits_equal(out[3], r_sp, "sorted_pairs")
