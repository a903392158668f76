"""GPU parity of the grouped GEMMs at one GPU's share of an expert-parallel
layer: the experts are split into contiguous blocks, and the owner of a
block receives only its own pairs, their x rows already grouped by expert
(as an all-to-all would deliver them). It runs the same grouped calls on
them with K = 1, identity pair order, offsets rebased to its first pair and
the packed weights of its experts only (``PackedWeights.experts``).

* Exact-arithmetic inputs: every shard's act and expert_out rows equal the
  oracle's rows of the whole layer bit for bit (so the split changes no
  arithmetic), with skewed routing that leaves experts empty.
* Random bf16 inputs at the prefill and skewed workloads' full shapes: the
  hottest and the coldest non-empty block of E/8 experts, as the benchmark
  times them, against the oracle on sampled rows (2 bf16 ulp / 1e-2 rms,
  NMSE <= 1e-5).
"""
import numpy as np
import pytest
import torch

import oracle as O
from conftest import cached_inputs
from gpu_helpers import (DEV, assert_bits_equal, assert_gemm_close, bits, packed_d, packed_gu,
                         sample_rows, sub_down, sub_gateup, to_dev, to_dev_bf16)
from test_gpu_gemm import _exact_bf16, _routing_for

pytestmark = pytest.mark.gpu


def run_shard(lib, x_dev, wgu_p, wd_p, sp, off, w_flat, K, e0, e1, act_in=None):
    """The owner of experts [e0, e1): its received x rows, act and expert_out
    (rows in the owner's order, i.e. global sorted positions off[e0]..off[e1])."""
    q0, q1 = int(off[e0]), int(off[e1])
    pairs = np.asarray(sp[q0:q1], np.int64)
    xs = x_dev.index_select(0, torch.from_numpy(pairs // K).to(DEV)).contiguous()
    offs = (np.asarray(off[e0:e1 + 1], np.int64) - q0).astype(np.int32)
    idn = np.arange(q1 - q0, dtype=np.int32)
    act = lib.moe_grouped_gemm_gateup_silu(xs, wgu_p.experts(e0, e1), to_dev(idn), to_dev(offs), 1)
    a = act if act_in is None else to_dev_bf16(act_in)
    eo = lib.moe_grouped_gemm_down(a, wd_p.experts(e0, e1), to_dev(idn), to_dev(offs),
                                   to_dev(np.ascontiguousarray(w_flat[pairs])))
    torch.cuda.synchronize()
    return act, eo


@pytest.mark.parametrize("skew", [False, True])
def test_shards_bit_exact_on_exact_arithmetic(gpu_lib, skew):
    T, H, E, K, I = 4096, 520, 16, 4, 1000
    print(f"expert shards exact T={T} H={H} E={E} K={K} I={I} skew={skew}", flush=True)
    seed = 91 + int(skew)
    x = _exact_bf16(seed, (T, H), -4, 4, 1.0)
    wgu = _exact_bf16(seed + 1, (E, 2 * I, H), -4, 4, 2.0 ** -6)
    wd = _exact_bf16(seed + 4, (E, H, I), -4, 4, 2.0 ** -5)
    a2 = _exact_bf16(seed + 3, (T * K, I), -8, 8, 2.0 ** -4)
    ids, w, off, sp = _routing_for(T, E, K, seed + 2, skew)
    w_flat = w.reshape(-1)
    ref_act = O.gateup_silu(x, wgu, sp, off, K)
    ref_eo = O.down_proj(a2, wd, sp, off, w_flat)
    x_d, wgu_p, wd_p = to_dev_bf16(x), packed_gu(wgu), packed_d(wd)
    if skew:
        assert np.any(np.diff(off) == 0), "expected empty experts"
    nb = 4
    for e0 in range(0, E, nb):
        q0, q1 = int(off[e0]), int(off[e0 + nb])
        if q0 == q1:
            continue
        # down runs on the exact act rows a2 takes in sorted order
        act, eo = run_shard(gpu_lib, x_d, wgu_p, wd_p, sp, off, w_flat, K, e0, e0 + nb,
                            act_in=a2[q0:q1])
        assert_bits_equal(bits(act), ref_act[q0:q1], f"act experts {e0}..{e0 + nb}")
        assert_bits_equal(bits(eo), ref_eo[sp[q0:q1]], f"expert_out experts {e0}..{e0 + nb}")


@pytest.mark.parametrize("n", [3, 5])
def test_hot_and_cold_shards_full_size_sampled(gpu_lib, n):
    d = cached_inputs(n)
    cfg = d["cfg"]
    K, E = cfg.K, cfg.E
    logits = O.router_logits(d["x"], d["w_r"], d.get("router_bias"))
    ids, w, off, sp = O.route(logits, K)
    w_flat = w.reshape(-1)
    nb = E // 8
    sizes = [int(off[b + nb] - off[b]) for b in range(0, E, nb)]
    nonempty = [i for i, s in enumerate(sizes) if s > 0]
    hot = int(np.argmax(sizes))
    cold = min(nonempty, key=lambda i: sizes[i])
    x_d, wgu_p, wd_p = to_dev_bf16(d["x"]), packed_gu(d["w_gu"]), packed_d(d["w_d"])
    for b in sorted({hot, cold}):
        e0, e1 = b * nb, (b + 1) * nb
        q0, q1 = int(off[e0]), int(off[e1])
        print(f"cfg{n} shard experts {e0}..{e1} pairs {q1 - q0}", flush=True)
        act, eo = run_shard(gpu_lib, x_d, wgu_p, wd_p, sp, off, w_flat, K, e0, e1)
        qs = sample_rows(off[e0:e1 + 1], 4, seed=b)       # global sorted positions
        ref_act = sub_gateup(d["x"], d["w_gu"], sp, off, K, qs)
        act_h = bits(act)
        assert_gemm_close(act_h[qs - q0], ref_act, f"cfg{n} shard {b} act (sampled)")
        ref_eo = sub_down(act_h[qs - q0], d["w_d"], off, qs, w_flat[sp[qs]])
        assert_gemm_close(bits(eo)[qs - q0], ref_eo, f"cfg{n} shard {b} expert_out (sampled)")
