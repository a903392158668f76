"""GPU parity of the fused decode expert FFN (gate-up -> SiLU -> down in one
launch, moe_fused_expert_ffn).

* Exact-arithmetic inputs (small integers times powers of two, so the gate and
  up sums are exact in f32 whatever their order): act bit-exact against the
  oracle; expert_out (whose act operand is no longer on a coarse grid) at the
  GEMM bar against the oracle's down of the GPU's act; over ragged and empty
  experts, k and column tails, several row tiles per expert, identity rows.
* The decode workload: act bit-identical to the two-call path (the same tile
  arithmetic), expert_out at the GEMM bar against the oracle fed the GPU's
  act and against the two-call path; the workspace counters back at zero and
  the status word 0 after every launch.
* Three launches in a row on one workspace, then a captured HIP graph replayed
  three times with eager work between the replays: every result identical.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import (DEV, assert_bits_equal, assert_gemm_close, bits, packed_d, packed_gu,
                         to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu
F32 = np.float32


def _exact_bf16(seed, shape, lo, hi, scale):
    g = np.random.Generator(np.random.PCG64(seed))
    v = (g.integers(lo, hi + 1, size=shape).astype(np.float64) * scale).astype(F32)
    b = O.bf16_from_f32(v)
    assert np.array_equal(O.f32_from_bf16(b), v)
    return b


def _routing(T, E, K, seed, empty=()):
    g = np.random.Generator(np.random.PCG64(seed))
    l = g.standard_normal((T, E)).astype(F32)
    for e in empty:
        l[:, e] = -50.0
    return O.route(l, K)


def _ws(gpu_lib, T, E, K, grouped=True):
    n = gpu_lib.moe_fused_expert_ffn_workspace_bytes(T, E, K, grouped) // 4
    return torch.zeros((n,), dtype=torch.int32, device=DEV)


# (T, H, E, K, I, empty experts)
SHAPES = [
    (16, 64, 8, 2, 32, ()),           # 4 rows per expert
    (40, 136, 16, 3, 40, (3,)),       # k tail, column tail, an empty expert
    (32, 512, 128, 8, 96, ()),        # decode-like: 2 rows per expert, many experts
    (96, 256, 16, 4, 72, (0, 15)),    # 24 rows per expert: two 16-row tiles
    (300, 328, 8, 2, 200, ()),        # 75 rows per expert, ragged
]


@pytest.mark.parametrize("T,H,E,K,I,empty", SHAPES)
def test_fused_bit_exact_on_exact_arithmetic(gpu_lib, T, H, E, K, I, empty):
    print(f"fused exact T={T} H={H} E={E} K={K} I={I}", flush=True)
    seed = T + 3 * H + E + K + I
    x = _exact_bf16(seed, (T, H), -4, 4, 1.0)
    wgu = _exact_bf16(seed + 1, (E, 2 * I, H), -4, 4, 2.0 ** -6)
    wd = _exact_bf16(seed + 2, (E, H, I), -4, 4, 2.0 ** -5)
    ids, w, off, sp = _routing(T, E, K, seed + 3, empty)
    ws = _ws(gpu_lib, T, E, K)
    act, eo = gpu_lib.moe_fused_expert_ffn(to_dev_bf16(x), packed_gu(wgu), packed_d(wd),
                                           to_dev(sp), to_dev(off), K, to_dev(w.reshape(-1)), ws)
    torch.cuda.synchronize()
    assert_bits_equal(bits(act), O.gateup_silu(x, wgu, sp, off, K), "fused act")
    ref_eo = O.down_proj(bits(act), wd, sp, off, w.reshape(-1))
    assert_gemm_close(bits(eo), ref_eo, "fused expert_out")
    assert gpu_lib.fused_ffn_status(ws) == 0
    assert not ws.any().item(), "counters not back at zero"


def test_fused_identity_rows(gpu_lib):
    T, H, I = 40, 192, 48
    x = _exact_bf16(11, (T, H), -4, 4, 1.0)
    wgu = _exact_bf16(12, (1, 2 * I, H), -4, 4, 2.0 ** -6)
    wd = _exact_bf16(13, (1, H, I), -4, 4, 2.0 ** -5)
    ws = _ws(gpu_lib, T, 1, 1, grouped=False)
    act, eo = gpu_lib.moe_fused_expert_ffn(to_dev_bf16(x), packed_gu(wgu), packed_d(wd), None,
                                           None, 1, None, ws)
    torch.cuda.synchronize()
    assert_bits_equal(bits(act), O.gateup_silu(x, wgu, None, None, 1), "identity act")
    assert_gemm_close(bits(eo), O.down_proj(bits(act), wd, None, None, None), "identity down")
    assert gpu_lib.fused_ffn_status(ws) == 0 and not ws.any().item()


def test_fused_decode_workload_against_two_calls_and_oracle(gpu_lib):
    from conftest import cached_inputs
    d = cached_inputs(2)
    cfg = d["cfg"]
    T, H, E, K, I = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I
    x_d = to_dev_bf16(d["x"])
    logits = gpu_lib.moe_router_logits(x_d, to_dev_bf16(d["w_r"]))
    ids, w, off, sp = gpu_lib.moe_route(logits, K)
    wgu, wd = packed_gu(d["w_gu"]), packed_d(d["w_d"])
    ws = _ws(gpu_lib, T, E, K)
    act, eo = gpu_lib.moe_fused_expert_ffn(x_d, wgu, wd, sp, off, K, w.view(-1), ws)
    act2 = gpu_lib.moe_grouped_gemm_gateup_silu(x_d, wgu, sp, off, K)
    eo2 = gpu_lib.moe_grouped_gemm_down(act2, wd, sp, off, w.view(-1))
    torch.cuda.synchronize()
    assert gpu_lib.fused_ffn_status(ws) == 0 and not ws.any().item()
    assert_bits_equal(bits(act), bits(act2), "act against the two-call path")
    r_sp, r_off, r_w = bits(sp), bits(off), bits(w)
    assert_gemm_close(bits(eo), O.down_proj(bits(act), d["w_d"], r_sp, r_off, r_w.reshape(-1)),
                      "expert_out against the oracle")
    assert_gemm_close(bits(eo), bits(eo2), "expert_out against the two-call path")
    ref_act = O.gateup_silu(d["x"], d["w_gu"], r_sp, r_off, K)
    assert_gemm_close(bits(act), ref_act, "act against the oracle")


def test_fused_repeated_and_graph_replays(gpu_lib):
    from conftest import cached_inputs
    d = cached_inputs(2)
    cfg = d["cfg"]
    T, H, E, K, I = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I
    x_d = to_dev_bf16(d["x"])
    logits = gpu_lib.moe_router_logits(x_d, to_dev_bf16(d["w_r"]))
    ids, w, off, sp = gpu_lib.moe_route(logits, K)
    wgu, wd = packed_gu(d["w_gu"]), packed_d(d["w_d"])
    ws = _ws(gpu_lib, T, E, K)
    act = torch.empty((T * K, I), dtype=torch.bfloat16, device=DEV)
    eo = torch.empty((T * K, H), dtype=torch.bfloat16, device=DEV)
    gpu_lib.moe_fused_expert_ffn(x_d, wgu, wd, sp, off, K, w.view(-1), ws, act, eo)
    torch.cuda.synchronize()
    ref_act, ref_eo = bits(act).copy(), bits(eo).copy()
    for i in range(3):
        act.zero_()
        eo.zero_()
        gpu_lib.moe_fused_expert_ffn(x_d, wgu, wd, sp, off, K, w.view(-1), ws, act, eo)
        torch.cuda.synchronize()
        assert gpu_lib.fused_ffn_status(ws) == 0 and not ws.any().item()
        assert_bits_equal(bits(act), ref_act, f"act, launch {i}")
        assert_bits_equal(bits(eo), ref_eo, f"expert_out, launch {i}")
    gpu_lib.moe_init()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm-up on the capture stream
        gpu_lib.moe_fused_expert_ffn(x_d, wgu, wd, sp, off, K, w.view(-1), ws, act, eo, stream=s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        gpu_lib.moe_fused_expert_ffn(x_d, wgu, wd, sp, off, K, w.view(-1), ws, act, eo, stream=s)
    torch.cuda.synchronize()
    for i in range(3):
        act.zero_()
        eo.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert gpu_lib.fused_ffn_status(ws) == 0 and not ws.any().item()
        assert_bits_equal(bits(act), ref_act, f"act, replay {i}")
        assert_bits_equal(bits(eo), ref_eo, f"expert_out, replay {i}")
