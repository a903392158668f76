"""GPU parity of the grouped GEMMs and the logits helper.

* Exact-arithmetic inputs (small integers times powers of two, every partial
  sum exact in f32) make the GEMMs independent of summation order, so the GPU
  must match the oracle bit for bit, through both kernel shapes (weight
  streaming for few rows per expert, LDS tiles for many), ragged row counts,
  empty experts and column / k tails; the hand-derived golden fixtures (N1,
  N2, gather, scatter) run bit-exact too.
* Random bf16 inputs at the workload shapes: stage-wise (the GPU stage gets
  the oracle's routing) within 2 bf16 ulp / 1e-2 rms and NMSE <= 1e-5; the
  8192-token skewed workload is checked on sampled rows, the launch
  configuration being the one the benchmark times.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from conftest import cached_inputs
from gpu_helpers import (DEV, assert_bits_equal, assert_gemm_close, bits, packed_d, packed_gu,
                         sample_rows, sub_down, sub_gateup, to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu
F32 = np.float32


def _exact_bf16(seed, shape, lo, hi, scale):
    g = np.random.Generator(np.random.PCG64(seed))
    v = (g.integers(lo, hi + 1, size=shape).astype(np.float64) * scale).astype(F32)
    b = O.bf16_from_f32(v)
    assert np.array_equal(O.f32_from_bf16(b), v)
    return b


def _routing_for(T, E, K, seed, skew=False):
    g = np.random.Generator(np.random.PCG64(seed))
    l = g.standard_normal((T, E)).astype(F32)
    if skew:
        l += (3.0 * np.log(1.0 / (1.0 + np.arange(E)))).astype(F32)
    ids, w, off, sp = O.route(l, K)
    return ids, w, off, sp


# (T, H, E, K, I): avg rows/expert T*K/E spans the streaming (<= 8, <= 24) and
# tiled kernels; H, I not multiples of the tile sizes to exercise tails.
EXACT_SHAPES = [
    (16, 64, 8, 2, 32),       # 4 rows/expert, tiny
    (40, 136, 16, 3, 40),     # 7.5 rows/expert, k tail, column tail
    (96, 256, 16, 4, 72),     # 24 rows/expert -> 32-row streaming tiles
    (300, 328, 8, 2, 200),    # 75 rows/expert -> LDS tiles, ragged
    (700, 512, 12, 3, 136),   # 175 rows/expert, several m tiles per expert
]


@pytest.mark.parametrize("T,H,E,K,I", EXACT_SHAPES)
@pytest.mark.parametrize("skew", [False, True])
def test_gemms_bit_exact_on_exact_arithmetic(gpu_lib, T, H, E, K, I, skew):
    print(f"exact gemm T={T} H={H} E={E} K={K} I={I} skew={skew}", flush=True)
    seed = T * 7 + H + E * 3 + K + I + int(skew)
    x = _exact_bf16(seed, (T, H), -4, 4, 1.0)
    wgu = _exact_bf16(seed + 1, (E, 2 * I, H), -4, 4, 2.0 ** -6)
    ids, w, off, sp = _routing_for(T, E, K, seed + 2, skew)
    if skew:
        assert np.any(np.diff(off) == 0), "expected empty experts"
    act = gpu_lib.moe_grouped_gemm_gateup_silu(to_dev_bf16(x), packed_gu(wgu), to_dev(sp),
                                               to_dev(off), K)
    torch.cuda.synchronize()
    ref_act = O.gateup_silu(x, wgu, sp, off, K)
    assert_bits_equal(bits(act), ref_act, "act")
    # down on an exact act (its own values) so the sums stay exact
    a2 = _exact_bf16(seed + 3, (T * K, I), -8, 8, 2.0 ** -4)
    wd = _exact_bf16(seed + 4, (E, H, I), -4, 4, 2.0 ** -5)
    eo = gpu_lib.moe_grouped_gemm_down(to_dev_bf16(a2), packed_d(wd), to_dev(sp), to_dev(off),
                                       to_dev(w.reshape(-1)))
    torch.cuda.synchronize()
    assert_bits_equal(bits(eo), O.down_proj(a2, wd, sp, off, w.reshape(-1)), "expert_out")
    eo0 = gpu_lib.moe_grouped_gemm_down(to_dev_bf16(a2), packed_d(wd), to_dev(sp), to_dev(off),
                                        None)
    torch.cuda.synchronize()
    assert_bits_equal(bits(eo0), O.down_proj(a2, wd, sp, off, None), "expert_out unweighted")


@pytest.mark.parametrize("skew", [False, True])
def test_tiled_gemms_bit_exact_on_exact_arithmetic(gpu_lib, skew):
    """Large enough for the LDS-tiled kernels (128-row gate-up tiles with the
    direct-to-LDS ring at this size, 128-row down tiles): 16384 pairs over 16
    experts, with k tails (H = 520, I = 1000 are not multiples of 64) and a
    column tail."""
    T, H, E, K, I = 4096, 520, 16, 4, 1000
    print(f"exact tiled gemm T={T} H={H} E={E} K={K} I={I} skew={skew}", flush=True)
    seed = 77 + int(skew)
    x = _exact_bf16(seed, (T, H), -4, 4, 1.0)
    wgu = _exact_bf16(seed + 1, (E, 2 * I, H), -4, 4, 2.0 ** -6)
    ids, w, off, sp = _routing_for(T, E, K, seed + 2, skew)
    act = gpu_lib.moe_grouped_gemm_gateup_silu(to_dev_bf16(x), packed_gu(wgu), to_dev(sp),
                                               to_dev(off), K)
    torch.cuda.synchronize()
    assert_bits_equal(bits(act), O.gateup_silu(x, wgu, sp, off, K), "act")
    a2 = _exact_bf16(seed + 3, (T * K, I), -8, 8, 2.0 ** -4)
    wd = _exact_bf16(seed + 4, (E, H, I), -4, 4, 2.0 ** -5)
    eo = gpu_lib.moe_grouped_gemm_down(to_dev_bf16(a2), packed_d(wd), to_dev(sp), to_dev(off),
                                       to_dev(w.reshape(-1)))
    torch.cuda.synchronize()
    assert_bits_equal(bits(eo), O.down_proj(a2, wd, sp, off, w.reshape(-1)), "expert_out")


@pytest.mark.parametrize("T,H,I", [(16, 64, 32), (512, 264, 72), (40, 128, 512),
                                   (16384, 136, 2560), (16384, 2816, 72)])
def test_identity_rows_bit_exact(gpu_lib, T, H, I):
    """NULL sorted_pairs/offsets: a dense expert (the shared expert). The two
    16384-row cases take the tile kernels' one-expert block order: the first
    the 320 x 256 direct-load gate-up and the register-staged 128 x 128 down,
    the second the 128 x 128 direct-load gate-up and the 320 x 256 down."""
    print(f"identity rows T={T} H={H} I={I}", flush=True)
    x = _exact_bf16(T + H, (T, H), -4, 4, 1.0)
    wgu = _exact_bf16(I + 1, (1, 2 * I, H), -4, 4, 2.0 ** -6)
    act = gpu_lib.moe_grouped_gemm_gateup_silu(to_dev_bf16(x), packed_gu(wgu), None, None, 1)
    a2 = _exact_bf16(I + 2, (T, I), -8, 8, 2.0 ** -4)
    wd = _exact_bf16(I + 3, (1, H, I), -4, 4, 2.0 ** -5)
    sd = gpu_lib.moe_grouped_gemm_down(to_dev_bf16(a2), packed_d(wd), None, None, None)
    torch.cuda.synchronize()
    assert_bits_equal(bits(act), O.gateup_silu(x, wgu, None, None, 1), "shared act")
    assert_bits_equal(bits(sd), O.down_proj(a2, wd, None, None, None), "shared down")


def _golden():
    return json.load(open(os.path.join(os.path.dirname(__file__), "golden", "gemm_cases.json")))


def _pad(a, axis_sizes):
    out = np.zeros(axis_sizes, np.float32)
    out[tuple(slice(0, s) for s in np.shape(a))] = a
    return out


@pytest.mark.parametrize("case", _golden()["gateup"], ids=lambda c: c["name"])
def test_gateup_golden_on_gpu(gpu_lib, case):
    T, H, E, K, I = case["T"], case["H"], case["E"], case["K"], case["I"]
    Hp, Ip = 8, 8                       # zero padding keeps every value
    x = O.bf16_from_f32(_pad(np.array(case["x"], F32), (T, Hp)))
    wg = np.array(case["w_gu"], F32)
    wgu = np.zeros((E, 2 * Ip, Hp), F32)
    wgu[:, :I, :H] = wg[:, :I]
    wgu[:, Ip:Ip + I, :H] = wg[:, I:]
    act = gpu_lib.moe_grouped_gemm_gateup_silu(to_dev_bf16(x), packed_gu(O.bf16_from_f32(wgu)),
                                               to_dev(np.array(case["sorted_pairs"], np.int32)),
                                               to_dev(np.array(case["offsets"], np.int32)), K)
    torch.cuda.synchronize()
    got = O.f32_from_bf16(bits(act))[:, :I]
    assert np.array_equal(got, np.array(case["expected_act"], F32))


@pytest.mark.parametrize("case", _golden()["down"], ids=lambda c: c["name"])
def test_down_golden_on_gpu(gpu_lib, case):
    P, I, E, H = case["P"], case["I"], case["E"], case["H"]
    Ip, Hp = 8, 8
    act = O.bf16_from_f32(_pad(np.array(case["act"], F32), (P, Ip)))
    wd = O.bf16_from_f32(_pad(np.array(case["w_d"], F32), (E, Hp, Ip)))
    eo = gpu_lib.moe_grouped_gemm_down(to_dev_bf16(act), packed_d(wd),
                                       to_dev(np.array(case["sorted_pairs"], np.int32)),
                                       to_dev(np.array(case["offsets"], np.int32)),
                                       to_dev(np.array(case["pair_w"], F32)))
    torch.cuda.synchronize()
    got = O.f32_from_bf16(bits(eo))[:, :H]
    assert np.array_equal(got, np.array(case["expected_out"], F32))


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_gemms_stagewise_workloads(gpu_lib, n):
    d = cached_inputs(n)
    cfg = d["cfg"]
    print(f"stagewise gemm cfg={n} T={cfg.T}", flush=True)
    logits = O.router_logits(d["x"], d["w_r"], d.get("router_bias"))
    ids, w, off, sp = O.route(logits, cfg.K)
    x_d, wgu_d, wd_d = to_dev_bf16(d["x"]), packed_gu(d["w_gu"]), packed_d(d["w_d"])
    act = gpu_lib.moe_grouped_gemm_gateup_silu(x_d, wgu_d, to_dev(sp), to_dev(off), cfg.K)
    torch.cuda.synchronize()
    ref_act = O.gateup_silu(d["x"], d["w_gu"], sp, off, cfg.K)
    assert_gemm_close(bits(act), ref_act, f"cfg{n} act")
    # down from the oracle's act
    eo = gpu_lib.moe_grouped_gemm_down(to_dev_bf16(ref_act), wd_d, to_dev(sp), to_dev(off),
                                       to_dev(w.reshape(-1)))
    torch.cuda.synchronize()
    assert_gemm_close(bits(eo), O.down_proj(ref_act, d["w_d"], sp, off, w.reshape(-1)),
                      f"cfg{n} expert_out")
    if "w_gu_s" in d:
        sa = gpu_lib.moe_grouped_gemm_gateup_silu(x_d, packed_gu(d["w_gu_s"][None]), None, None, 1)
        torch.cuda.synchronize()
        ref_sa = O.gateup_silu(d["x"], d["w_gu_s"][None], None, None, 1)
        assert_gemm_close(bits(sa), ref_sa, f"cfg{n} shared act")
        sd = gpu_lib.moe_grouped_gemm_down(to_dev_bf16(ref_sa), packed_d(d["w_d_s"][None]),
                                           None, None, None)
        torch.cuda.synchronize()
        assert_gemm_close(bits(sd), O.down_proj(ref_sa, d["w_d_s"][None], None, None, None),
                          f"cfg{n} shared out")


def test_gemms_skewed_full_size_sampled(gpu_lib):
    d = cached_inputs(5)
    cfg = d["cfg"]
    print(f"skewed full-size gemm T={cfg.T} H={cfg.H} I={cfg.I}", flush=True)
    logits = O.router_logits(d["x"], d["w_r"], d["router_bias"])
    ids, w, off, sp = O.route(logits, cfg.K)
    assert np.count_nonzero(np.diff(off) == 0) > 0, "skewed routing leaves experts empty"
    act = gpu_lib.moe_grouped_gemm_gateup_silu(to_dev_bf16(d["x"]), packed_gu(d["w_gu"]),
                                               to_dev(sp), to_dev(off), cfg.K)
    eo = gpu_lib.moe_grouped_gemm_down(act, packed_d(d["w_d"]), to_dev(sp), to_dev(off),
                                       to_dev(w.reshape(-1)))
    torch.cuda.synchronize()
    qs = sample_rows(off, 3, seed=5)
    act_h = bits(act)
    ref_act = sub_gateup(d["x"], d["w_gu"], sp, off, cfg.K, qs)
    assert_gemm_close(act_h[qs], ref_act, "cfg5 act (sampled)")
    ref_eo = sub_down(act_h[qs], d["w_d"], off, qs, w.reshape(-1)[sp[qs]])
    assert_gemm_close(bits(eo)[sp[qs]], ref_eo, "cfg5 expert_out (sampled)")


@pytest.mark.parametrize("T,H,N,bias", [(16, 64, 8, False), (32, 2048, 128, False),
                                        (512, 2048, 1, False), (1000, 4096, 128, True),
                                        (1030, 520, 40, True), (4096, 2048, 128, False),
                                        (8192, 4096, 128, True), (8200, 520, 40, False)])
def test_router_logits_within_f32_bound(gpu_lib, T, H, N, bias):
    x = W.random_bf16(T + 1, (T, H))
    w = W.random_bf16(N + 2, (N, H), 1.0 / np.sqrt(H))
    b = W.random_f32(3, (N,)) if bias else None
    out = gpu_lib.moe_router_logits(to_dev_bf16(x), to_dev_bf16(w), None if b is None else to_dev(b))
    torch.cuda.synchronize()
    ref = O.router_logits(x, w, b).astype(np.float64)
    xf = O.f32_from_bf16(x).astype(np.float64)
    wf = O.f32_from_bf16(w).astype(np.float64)
    mag = np.abs(xf) @ np.abs(wf).T + (0 if b is None else np.abs(b)[None, :])
    err = np.abs(bits(out).astype(np.float64) - ref)
    # f32 accumulation: about H/16 rounded adds -> error well under 2^-14 of sum of abs terms
    assert np.all(err <= 2.0 ** -14 * mag + 1e-30), float(np.max(err / (mag + 1e-30)))


def test_gemm_output_canaries(gpu_lib):
    T, H, E, K, I = 40, 136, 16, 3, 40
    x = _exact_bf16(1, (T, H), -4, 4, 1.0)
    wgu = _exact_bf16(2, (E, 2 * I, H), -4, 4, 2.0 ** -6)
    ids, w, off, sp = _routing_for(T, E, K, 3)
    full = torch.full((T * K * I + 256,), 0x7BCD, dtype=torch.int16, device=DEV)
    act = full[: T * K * I].view(torch.bfloat16).view(T * K, I)
    gpu_lib.moe_grouped_gemm_gateup_silu(to_dev_bf16(x), packed_gu(wgu), to_dev(sp), to_dev(off),
                                         K, act=act)
    torch.cuda.synchronize()
    assert torch.all(full[T * K * I:] == 0x7BCD).item(), "gate-up wrote past act"
    assert_bits_equal(bits(act), O.gateup_silu(x, wgu, sp, off, K), "act")


def test_timed_gemm_launch_matches_untimed(gpu_lib):
    """moe_time_next_gemm: the timed launch computes the same bits, the events
    hold a positive kernel duration, and the arming covers one call only."""
    T, H, E, K, I = 32, 2048, 128, 8, 768
    x = W.random_bf16(11, (T, H))
    wgu = W.random_bf16(12, (E, 2 * I, H), 1.0 / np.sqrt(H))
    wd = W.random_bf16(13, (E, H, I), 1.0 / np.sqrt(I))
    ids, w, off, sp = _routing_for(T, E, K, 14)
    x_d, wgu_d, wd_d, sp_d, off_d = (to_dev_bf16(x), packed_gu(wgu), packed_d(wd),
                                     to_dev(sp), to_dev(off))
    pw = to_dev(w.reshape(-1))
    ref_act = gpu_lib.moe_grouped_gemm_gateup_silu(x_d, wgu_d, sp_d, off_d, K)
    ref_eo = gpu_lib.moe_grouped_gemm_down(ref_act, wd_d, sp_d, off_d, pw)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    gpu_lib.moe_time_next_gemm(evs[0], evs[1])
    act = gpu_lib.moe_grouped_gemm_gateup_silu(x_d, wgu_d, sp_d, off_d, K)
    gpu_lib.moe_time_next_gemm(evs[2], evs[3])
    eo = gpu_lib.moe_grouped_gemm_down(act, wd_d, sp_d, off_d, pw)
    # not armed any more: a plain launch
    eo2 = gpu_lib.moe_grouped_gemm_down(act, wd_d, sp_d, off_d, pw)
    torch.cuda.synchronize()
    assert torch.equal(act.view(torch.int16), ref_act.view(torch.int16))
    assert torch.equal(eo.view(torch.int16), ref_eo.view(torch.int16))
    assert torch.equal(eo2.view(torch.int16), ref_eo.view(torch.int16))
    t_gu = evs[0].elapsed_time(evs[1])
    t_dn = evs[2].elapsed_time(evs[3])
    assert 0.0 < t_gu < 100.0 and 0.0 < t_dn < 100.0, (t_gu, t_dn)


TAILS_320 = [1, 31, 32, 33, 63, 64, 65, 96, 129, 160, 200, 255, 288, 319, 320, 0]
TAILS_128 = [1, 31, 32, 33, 63, 64, 65, 96, 127, 128, 0]


@pytest.mark.parametrize("bm,tails,full,I", [(320, TAILS_320, 3, 2000), (128, TAILS_128, 2, 1000)],
                         ids=["tiles320", "tiles128"])
def test_tiled_gateup_tail_tiles_bit_exact(gpu_lib, bm, tails, full, I):
    """Every kind of partial row tile of the LDS-tiled gate-up, in both of its
    tile shapes: 320-row tiles (32-row fragments dealt to two row waves) once
    there are at least 512 of them nominally (P / 320 times 128-column
    blocks), else 128-row tiles (one fragment per row wave). Experts whose
    last tile holds from 1 row to a full tile, one empty expert, and several
    full tiles per expert; the fragments past a tile's last row are skipped.
    Exact arithmetic, so bit for bit."""
    E, K, H = len(tails), 4, 264
    counts = np.array([(full if t else 0) * bm + t for t in tails], dtype=np.int64)
    counts[0] += (-int(counts.sum())) % K  # whole tokens
    P = int(counts.sum())
    T = P // K
    nominal = (P // 320) * ((I + 127) // 128)
    assert (nominal >= 512) == (bm == 320), nominal
    assert (P // 256) * ((I + 127) // 128) >= 32 and P / E > 24    # tiled, not streamed
    print(f"tiled gate-up tail tiles bm={bm} T={T} H={H} E={E} K={K} I={I}", flush=True)
    g = np.random.Generator(np.random.PCG64(4242))
    ids = g.permutation(np.repeat(np.arange(E), counts)).reshape(T, K).astype(np.int32)
    off, sp = O.group_pairs(ids, E)
    assert np.array_equal(np.diff(off), counts)
    x = _exact_bf16(91, (T, H), -4, 4, 1.0)
    wgu = _exact_bf16(92, (E, 2 * I, H), -4, 4, 2.0 ** -6)
    act = gpu_lib.moe_grouped_gemm_gateup_silu(to_dev_bf16(x), packed_gu(wgu), to_dev(sp),
                                               to_dev(off), K)
    torch.cuda.synchronize()
    assert_bits_equal(bits(act), O.gateup_silu(x, wgu, sp, off, K), "act")


def _bf16_nan(b):
    b = np.asarray(b, np.uint16)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)


def test_tiled_gateup_silu_every_bf16_gate(gpu_lib):
    """SiLU-mul of the 320 x 256 tile kernel for every bf16 gate value.

    One-hot activation rows (row p has 1 at k = p mod 32) pick gate value
    W_g[c, p mod 32] and up value 1, so the 32 distinct rows x 2,048 columns
    hold all 65,536 bf16 bit patterns as the gate (the 65,280 finite ones in
    columns 0..2039; the infinities and NaNs in 2040..2047, where 0 * inf
    makes every gate NaN). 10,240 rows put the call on the 320-row tiles.
    Bit-exact against the oracle, NaNs by position.
    """
    P, H, I = 10240, 32, 2048
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    special = ((pats & 0x7F80) == 0x7F80)
    order = np.concatenate([pats[~special], pats[special]])
    assert order.size == I * H and int((~special).sum()) == (I - 8) * H
    wgu = np.empty((1, 2 * I, H), np.uint16)
    wgu[0, :I] = order.reshape(I, H)
    wgu[0, I:] = O.bf16_from_f32(np.ones((I, H), F32))
    x = np.zeros((P, H), np.uint16)
    x[np.arange(P), np.arange(P) % H] = O.bf16_from_f32(np.ones(1, F32))[0]
    act = gpu_lib.moe_grouped_gemm_gateup_silu(to_dev_bf16(x), packed_gu(wgu), None, None, 1)
    torch.cuda.synchronize()
    got = bits(act)
    ref = O.gateup_silu(x[:H], wgu, None, None, 1)
    gn, rn = _bf16_nan(got[:H]), _bf16_nan(ref)
    assert np.array_equal(gn, rn), f"NaN positions differ: {int((gn != rn).sum())}"
    assert rn[:, I - 8:].all() and not rn[:, :I - 8].all()
    diff = int(np.count_nonzero(np.where(gn, 0, got[:H]) != np.where(rn, 0, ref)))
    assert diff == 0, f"{diff} of {ref.size} act values differ"
    # every row repeats the row of its one-hot position
    rep = got.reshape(P // H, H, I)
    assert np.array_equal(rep, np.broadcast_to(got[:H], rep.shape))
