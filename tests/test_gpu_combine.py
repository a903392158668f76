"""GPU parity of moe_combine_gate: bit-exact against the oracle on every
dtype arm, weighted and unweighted, routed_scale 1.0 and 0.7, with no /
ungated / gated shared term, ragged sizes, the hand-derived golden cases and
the layer shapes of the 256-expert and the skewed 8192-token workloads."""
import itertools
import json
import os
import zlib

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_helpers import DEV, assert_bits_equal, bits, to_dev

pytestmark = pytest.mark.gpu
F32 = np.float32


def _as(arr_f32, bf16):
    """Host f32 -> (device tensor in the arm's dtype, host copy the oracle reads)."""
    if bf16:
        b = O.bf16_from_f32(arr_f32)
        return torch.from_numpy(b).view(torch.bfloat16).to(DEV), b
    return to_dev(arr_f32.astype(F32)), arr_f32.astype(F32)


ARMS = list(itertools.product([True, False], repeat=3))


@pytest.mark.parametrize("eo_bf16,sh_bf16,out_bf16", ARMS)
@pytest.mark.parametrize("mode", ["none", "ungated", "gated"])
@pytest.mark.parametrize("weighted,scale", [(False, 1.0), (True, 1.0), (True, 0.7), (False, 0.7)])
def test_combine_arms_bit_exact(gpu_lib, eo_bf16, sh_bf16, out_bf16, mode, weighted, scale):
    T, K, H = 37, 3, 136            # T*H/8 = 629 threads: a ragged last block
    seed = zlib.crc32(repr((eo_bf16, sh_bf16, out_bf16, mode, weighted, scale)).encode()) % 10000
    eo_d, eo_h = _as(W.random_f32(seed, (T * K, H)), eo_bf16)
    w = W.random_f32(seed + 1, (T, K)) if weighted else None
    sh_d = sh_h = gl = None
    if mode != "none":
        sh_d, sh_h = _as(W.random_f32(seed + 2, (T, H)), sh_bf16)
    if mode == "gated":
        gl = W.random_f32(seed + 3, (T,), 3.0)
        gl[:4] = [0.0, np.inf, -np.inf, -100.0]
    out = gpu_lib.moe_combine_gate(eo_d, T, K, None if w is None else to_dev(w), scale, sh_d,
                                   None if gl is None else to_dev(gl),
                                   out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    ref = O.combine_gate(eo_h, T, K, H, w, scale, sh_h, gl, eo_bf16=eo_bf16,
                         sh_bf16=sh_bf16, out_bf16=out_bf16)
    assert assert_bits_equal(bits(out), ref, "combine") == T * H


def _golden():
    p = os.path.join(os.path.dirname(__file__), "golden", "combine_cases.json")
    return json.load(open(p))["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_combine_golden_cases_on_gpu(gpu_lib, case):
    T, K, H = case["T"], case["K"], case["H"]
    Hp = 8                          # the ABI needs H % 8 == 0: pad with zero columns
    eo = np.zeros((T * K, Hp), F32)
    eo[:, :H] = np.array(case["expert_out"], F32).reshape(T * K, H)
    sh = None
    if case["shared"] is not None:
        sh = np.zeros((T, Hp), F32)
        sh[:, :H] = np.array(case["shared"], F32).reshape(T, H)
    w = None if case["topk_w"] is None else np.array(case["topk_w"], F32)
    gl = None if case["gate_logit"] is None else np.array(case["gate_logit"], F32)
    out = gpu_lib.moe_combine_gate(to_dev(eo), T, K, None if w is None else to_dev(w),
                                   case["routed_scale"], None if sh is None else to_dev(sh),
                                   None if gl is None else to_dev(gl), out_dtype=torch.float32)
    torch.cuda.synchronize()
    exp = np.array([float.fromhex(s) for s in case["expected_hex"]], F32).reshape(T, H)
    assert np.array_equal(bits(out)[:, :H].view(np.uint32), exp.view(np.uint32))


@pytest.mark.parametrize("T,K,H,shared", [(512, 8, 2048, True), (8192, 8, 4096, False), (1, 1, 8, True)])
def test_combine_layer_shapes_bit_exact(gpu_lib, T, K, H, shared):
    print(f"combine layer shape T={T} K={K} H={H}", flush=True)
    eo = W.random_bf16(101, (T * K, H), 0.05)
    sd = W.random_bf16(102, (T, H), 0.05) if shared else None
    gl = W.random_f32(103, (T,), 2.0) if shared else None
    out = gpu_lib.moe_combine_gate(torch.from_numpy(eo).view(torch.bfloat16).to(DEV), T, K, None,
                                   1.0, None if sd is None else torch.from_numpy(sd).view(torch.bfloat16).to(DEV),
                                   None if gl is None else to_dev(gl))
    torch.cuda.synchronize()
    ref = O.combine_gate(eo, T, K, H, None, 1.0, sd, gl)
    assert_bits_equal(bits(out), ref, "combine")


def test_combine_gate_zero_gives_half_and_canary(gpu_lib):
    T, K, H = 5, 2, 64
    eo = W.random_bf16(7, (T * K, H))
    sd = W.random_bf16(8, (T, H))
    out_full = torch.full((T * H + 64,), 12345.0, dtype=torch.float32, device=DEV)
    out = out_full[: T * H].view(T, H)
    gpu_lib.moe_combine_gate(torch.from_numpy(eo).view(torch.bfloat16).to(DEV), T, K, None, 1.0,
                             torch.from_numpy(sd).view(torch.bfloat16).to(DEV),
                             torch.zeros(T, device=DEV), out=out)
    torch.cuda.synchronize()
    acc = np.zeros((T, H), F32)
    for k in range(K):
        acc = (acc + O.f32_from_bf16(eo).reshape(T, K, H)[:, k]).astype(F32)
    exp = (acc + O.f32_from_bf16(sd) * F32(0.5)).astype(F32)
    assert np.array_equal(bits(out), exp)
    assert torch.all(out_full[T * H:] == 12345.0).item(), "write past the output"


def test_bf16_store_rounding_sweep(gpu_lib):
    """The combine's f32 -> bf16 store against the oracle's round-to-nearest-
    even on every bf16 high half with eight low-half classes (exact, smallest
    step up, just below / at / just above the tie, the largest, and two
    random), which covers ties to even, subnormals, the carry into the
    exponent, overflow to infinity and NaN. K = 1, unweighted, scale 1, no
    shared term: out = bf16(+0 + v). Every output bit is compared, NaNs
    included: the add keeps a quiet NaN's payload, and the conversion keeps
    sign and top payload bits and sets the quiet bit, as the oracle does."""
    g = np.random.Generator(np.random.PCG64(77))
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = [0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF]
    cols = [hi | lo for lo in lows] + [hi | g.integers(0, 1 << 16, hi.size, dtype=np.uint32)
                                       for _ in range(2)]
    u = np.stack(cols, axis=1).reshape(-1)                 # 524,288 patterns
    T, H = 512, 1024
    v = u.view(np.float32).reshape(T, H)
    out = gpu_lib.moe_combine_gate(to_dev(v), T, 1, None, 1.0, None, None,
                                   out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got = bits(out).astype(np.uint32)
    ref = O.combine_gate(v, T, 1, H, None, 1.0, None, None, eo_bf16=False, out_bf16=True)
    ref = ref.astype(np.uint32)
    nan_r = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0)
    diff = int(np.count_nonzero(got != ref))
    assert diff == 0, f"{diff} of {got.size} stores differ"
    assert int(nan_r.sum()) > 2000 and int((~nan_r).sum()) > 500000
