"""GPU parity of the keep-quant path (Q4_K, Q5_K, Q6_K weights with Q8_K
activations; Q8_0 weights with Q8_0 activations).

* The Q8_K and Q8_0 quantizers are bit-exact against the oracle (quants,
  scales, sums of 16) on random rows, all-zero blocks, magnitude ties and
  exact halves.
* The grouped gate-up (SiLU, N1) and down (routing weight, N2) GEMMs of every
  weight format match the oracle's exactly summed keep-quant dots within 2
  bf16 ulp (or 1e-2 rms near cancellation) per element and NMSE <= 1e-5 per
  tensor (the pages' bar is NMSE <= 5e-4), stage-wise (each stage fed the
  oracle's input), over 1, 3, 8 and 16 units of 256, ragged experts, empty
  experts, column tails and identity rows; and the four keep-quant decode
  workloads through the whole GPU chain.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_helpers import DEV, assert_bits_equal, assert_gemm_close, bits, to_dev, to_dev_bf16

import mixture_experts_ffn_expert_amd as moe

pytestmark = pytest.mark.gpu
F32 = np.float32


def _sections(R, K):
    a = lambda v: (v + 255) // 256 * 256
    d = a(R * K)
    bs = a(d + R * (K // 256) * 4)
    return d, bs


def _q8k_from_gpu(buf, R, K):
    raw = buf.data.cpu().numpy()
    d_off, bs_off = _sections(R, K)
    qs = raw[:R * K].view(np.int8).reshape(R, K)
    d = raw[d_off:d_off + R * (K // 256) * 4].view(np.float32).reshape(R, K // 256)
    bs = raw[bs_off:bs_off + R * (K // 16) * 4].view(np.int32).reshape(R, K // 16)
    return qs, d, bs


@pytest.mark.parametrize("R,K", [(5, 256), (33, 2048), (7, 768)])
def test_quantize_q8k_bit_exact(gpu_lib, R, K):
    g = np.random.Generator(np.random.PCG64(R * K))
    x = g.standard_normal((R, K)).astype(F32) * F32(3)
    x[0, :256] = 0.0                                        # all-zero block
    x[1, 5], x[1, 9] = F32(-7.0), F32(7.0)                  # magnitude tie: first wins
    x[2, :256] = g.integers(-6, 7, 256).astype(F32) * F32(0.5)
    xb = O.bf16_from_f32(x)
    buf = gpu_lib.moe_quantize_q8k(to_dev_bf16(xb))
    torch.cuda.synchronize()
    qs, d, bs = _q8k_from_gpu(buf, R, K)
    rq, rd, rbs = O.quantize_q8k(O.f32_from_bf16(xb))
    assert_bits_equal(qs, rq, "quants")
    assert_bits_equal(d, rd, "scales")
    assert_bits_equal(bs, rbs, "sums of 16")


@pytest.mark.parametrize("R,K", [(5, 256), (33, 2048), (7, 96)])
def test_quantize_q8_0_bit_exact(gpu_lib, R, K):
    g = np.random.Generator(np.random.PCG64(R + K))
    x = g.standard_normal((R, K)).astype(F32) * F32(2)
    x[0, :32] = 0.0                                         # all-zero block
    x[1, :32] = 0.0
    x[1, 0] = F32(127.0)                                    # d = 1: exact halves below
    x[1, 1:5] = [2.5, -2.5, 0.5, -3.5]
    x[2, 32:64] = g.integers(-6, 7, 32).astype(F32) * F32(0.25)
    xb = O.bf16_from_f32(x)
    buf = gpu_lib.moe_quantize_q8_0(to_dev_bf16(xb))
    torch.cuda.synchronize()
    raw = buf.data.cpu().numpy()
    d_off = (R * K + 255) // 256 * 256
    qs = raw[:R * K].view(np.int8).reshape(R, K)
    d16 = raw[d_off:d_off + R * (K // 32) * 2].view(np.float16).reshape(R, K // 32)
    rq, rd = O.quantize_q8_0(O.f32_from_bf16(xb))
    assert_bits_equal(qs, rq, "quants")
    assert_bits_equal(d16.view(np.uint16), rd.view(np.uint16), "f16 scales")
    assert qs[1, 1:5].tolist() == [3, -3, 1, -4]


def _routing(T, E, K, seed, empty=()):
    g = np.random.Generator(np.random.PCG64(seed))
    l = g.standard_normal((T, E)).astype(F32)
    if empty == "skew":
        l += (2.0 * np.log(1.0 / (1.0 + np.arange(E)))).astype(F32)
        empty = ()
    for e in empty:
        l[:, e] = -50.0
    return O.route(l, K)


# (T, H, E, K, I, empty experts)
SHAPES = [
    (32, 2048, 16, 4, 512, ()),          # decode-like, 8 super-blocks
    (40, 768, 8, 3, 256, (2, 5)),        # 3 super-blocks, empty experts
    (24, 256, 6, 2, 264, ()),            # 1 super-block, column tail (I = 264)
    (200, 512, 4, 2, 768, ()),           # several 16-row tiles per expert
    # at most 4 rows per expert on average (Q4_K: the lane-per-row kernel)
    (16, 2048, 64, 4, 512, ()),          # 1 row per expert
    (24, 768, 32, 4, 264, (3, 7)),       # 3 super-blocks, column tail, empty experts
    (8, 256, 16, 2, 256, ()),            # 1 super-block
    (48, 1024, 64, 5, 512, "skew"),      # skewed: some experts past 8 rows (two tiles)
    (12, 4096, 8, 2, 1536, ()),          # 16 units per gate-up row, 6 per down row
]


FORMATS = ["q4_k", "q5_k", "q6_k", "q8_0"]


@pytest.mark.parametrize("wtype", FORMATS)
@pytest.mark.parametrize("T,H,E,K,I,empty", SHAPES)
def test_keepquant_gemms_stagewise(gpu_lib, T, H, E, K, I, empty, wtype):
    print(f"keep-quant {wtype} T={T} H={H} E={E} K={K} I={I}", flush=True)
    g = np.random.Generator(np.random.PCG64(T + H + E + I))
    x = O.bf16_from_f32(g.standard_normal((T, H)).astype(F32))
    wgu = W.random_kq_blocks(wtype, g.integers(1 << 30), (E, 2 * I), H, 1 / math.sqrt(H))
    ids, w, off, sp = _routing(T, E, K, T * 7 + E, empty)
    xq = gpu_lib.moe_quantize_act(wtype, to_dev_bf16(x))
    act = gpu_lib.moe_grouped_qgemm_gateup_silu(xq, torch.from_numpy(wgu).to(DEV), to_dev(sp),
                                                to_dev(off), K, wtype=wtype)
    torch.cuda.synchronize()
    ref_act, _ = O.kq_gateup_silu(x, wgu, sp, off, K, wtype)
    assert_gemm_close(bits(act), ref_act, "keep-quant act")
    if I % 256 == 0:
        wd = W.random_kq_blocks(wtype, g.integers(1 << 30), (E, H), I, 1 / math.sqrt(I))
        aq = gpu_lib.moe_quantize_act(wtype, to_dev_bf16(ref_act))
        eo = gpu_lib.moe_grouped_qgemm_down(aq, torch.from_numpy(wd).to(DEV), to_dev(sp),
                                            to_dev(off), to_dev(w.reshape(-1)), wtype=wtype)
        torch.cuda.synchronize()
        ref_eo, _ = O.kq_down(ref_act, wd, sp, off, w.reshape(-1), wtype)
        assert_gemm_close(bits(eo), ref_eo, "keep-quant expert_out")


@pytest.mark.parametrize("wtype", FORMATS)
@pytest.mark.parametrize("T", [48, 3])
def test_keepquant_identity_rows(gpu_lib, wtype, T):
    H, I = 512, 256
    g = np.random.Generator(np.random.PCG64(3))
    x = O.bf16_from_f32(g.standard_normal((T, H)).astype(F32))
    wgu = W.random_kq_blocks(wtype, g.integers(1 << 30), (1, 2 * I), H, 1 / math.sqrt(H))
    wd = W.random_kq_blocks(wtype, g.integers(1 << 30), (1, H), I, 1 / math.sqrt(I))
    ident = np.arange(T, dtype=np.int32)
    off = np.array([0, T], np.int32)
    act = gpu_lib.moe_grouped_qgemm_gateup_silu(gpu_lib.moe_quantize_act(wtype, to_dev_bf16(x)),
                                                torch.from_numpy(wgu).to(DEV), None, None, 1,
                                                wtype=wtype)
    torch.cuda.synchronize()
    ref_act, _ = O.kq_gateup_silu(x, wgu, ident, off, 1, wtype)
    assert_gemm_close(bits(act), ref_act, "identity act")
    sd = gpu_lib.moe_grouped_qgemm_down(gpu_lib.moe_quantize_act(wtype, to_dev_bf16(ref_act)),
                                        torch.from_numpy(wd).to(DEV), None, None, None,
                                        wtype=wtype)
    torch.cuda.synchronize()
    ref_sd, _ = O.kq_down(ref_act, wd, ident, off, None, wtype)
    assert_gemm_close(bits(sd), ref_sd, "identity down")


@pytest.mark.parametrize("n", [7, 8, 9, 10])
def test_keepquant_decode_layer(gpu_lib, n):
    """A keep-quant decode workload through the GPU chain: routing on the
    GPU's logits bit-exact, each GEMM stage against the oracle fed the same
    input, the combine bit-exact."""
    from conftest import cached_inputs
    d = cached_inputs(n)
    cfg = d["cfg"]
    wtype = cfg.weights
    T, H, E, K, I = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I
    print(f"keep-quant decode layer {wtype}", flush=True)
    x_d = to_dev_bf16(d["x"])
    logits = gpu_lib.moe_router_logits(x_d, to_dev_bf16(d["w_r"]))
    ids, w, off, sp = gpu_lib.moe_route(logits, K)
    xq = gpu_lib.moe_quantize_act(wtype, x_d)
    wgu = torch.from_numpy(d["w_gu_kq"]).to(DEV)
    wd = torch.from_numpy(d["w_d_kq"]).to(DEV)
    act = gpu_lib.moe_grouped_qgemm_gateup_silu(xq, wgu, sp, off, K, wtype=wtype)
    eo = gpu_lib.moe_grouped_qgemm_down(gpu_lib.moe_quantize_act(wtype, act), wd, sp, off,
                                        w.view(-1), wtype=wtype)
    out = gpu_lib.moe_combine_gate(eo, T, K)
    torch.cuda.synchronize()
    r_ids, r_w, r_off, r_sp = O.route(bits(logits), K)
    assert_bits_equal(bits(ids), r_ids, "ids")
    assert_bits_equal(bits(w), r_w, "weights")
    assert_bits_equal(bits(sp), r_sp, "sorted_pairs")
    ref_act, _ = O.kq_gateup_silu(d["x"], d["w_gu_kq"], r_sp, r_off, K, wtype)
    assert_gemm_close(bits(act), ref_act, "act")
    ref_eo, _ = O.kq_down(bits(act), d["w_d_kq"], r_sp, r_off, r_w.reshape(-1), wtype)
    assert_gemm_close(bits(eo), ref_eo, "expert_out")
    assert_bits_equal(bits(out), O.combine_gate(bits(eo), T, K, H, None, 1.0, None, None),
                      "combine")
