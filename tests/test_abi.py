"""Host-only checks of the C ABI: the library loads, exports every declared
symbol, and refuses bad arguments before touching the device.

No call here reaches a kernel launch: every argument set is rejected by host
validation (or, on a machine without a GPU, by the device check).
"""
import ctypes
import math
import os
import re
import subprocess

import pytest

import mixture_experts_ffn_expert_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

A = ctypes.c_void_p(0x10000)      # aligned, never dereferenced (refused first)
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)    # 8-byte aligned only


def _desc(kind, E, R, K, data=0x40000, layout=None, expert_bytes=None):
    """A weight descriptor as moe_pack_weights fills it (host memory only)."""
    d = moe.MoeWeights()
    d.layout = moe.MOE_WEIGHTS_PACKED_V1 if layout is None else layout
    d.kind, d.E, d.R, d.K = kind, E, R, K
    d.data = data
    nkb = (K + 31) // 32
    per = ((R // 2 + 15) // 16) * nkb * 2 * 1024 if kind == 1 else ((R + 15) // 16) * nkb * 1024
    d.expert_bytes = per if expert_bytes is None else expert_bytes
    return ctypes.byref(d)


GU = _desc(1, 8, 32, 16)          # W_gu [8, 2*16, 16] packed
DN = _desc(0, 8, 16, 16)          # W_d [8, 16, 16] packed


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    return moe.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(moe.SYMBOLS), (names, sorted(moe.SYMBOLS))
    out = subprocess.run(["nm", "-D", "--defined-only", moe.lib_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (moe_[a-z_0-9]+)$", out, flags=re.M))
    for n in names:
        assert n in exported, n
        getattr(lib, n)


def test_no_torch_types_in_the_abi():
    txt = open(HEADER).read()
    assert "torch" not in txt.lower().replace("torch types", "")
    assert "extern \"C\"" in txt


def _err(lib):
    return lib.moe_last_error().decode()


def test_f16_refused_by_name(lib):
    for args, arg in [
        ((A, moe.MOE_F16, 2, 2, 8, None, 1.0, None, moe.MOE_BF16, None, A2, moe.MOE_BF16), "expert_out"),
        ((A, moe.MOE_BF16, 2, 2, 8, None, 1.0, A, moe.MOE_F16, None, A2, moe.MOE_BF16), "shared"),
        ((A, moe.MOE_BF16, 2, 2, 8, None, 1.0, None, moe.MOE_BF16, None, A2, moe.MOE_F16), "out"),
    ]:
        st = lib.moe_combine_gate(*args, None)
        assert st == 2
        m = _err(lib)
        assert "moe_combine_gate" in m and arg in m and "f16" in m


def test_unknown_dtype_refused(lib):
    st = lib.moe_combine_gate(A, 7, 2, 2, 8, None, 1.0, None, 1, None, A2, 1, None)
    assert st == 2 and "unknown" in _err(lib)


@pytest.mark.parametrize("T,E,K", [(4, 8, 0), (4, 8, 9), (4, 2000, 2), (4, 64, 33), (-1, 8, 2)])
def test_route_shape_refusals(lib, T, E, K):
    st = lib.moe_route(A, T, E, K, A, A, A, A, None, 0, None)
    assert st == 3
    assert "moe_route" in _err(lib)


def test_route_null_outputs_refused(lib):
    st = lib.moe_route(A, 4, 8, 2, None, A, A, A, None, 0, None)
    assert st == 1 and "topk_ids" in _err(lib)
    st = lib.moe_route(A, 4, 8, 2, A, A, None, A, None, 0, None)
    assert st == 1 and "expert_offsets" in _err(lib)


def test_gemm_refusals(lib):
    f = lib.moe_grouped_gemm_gateup_silu
    assert f(A, 4, 12, GU, 8, 16, A, A, 2, A, None) == 3 and "H=12" in _err(lib)
    assert f(A, 4, 16, GU, 8, 12, A, A, 2, A, None) == 3 and "I=12" in _err(lib)
    assert f(A, 4, 16, GU, 8, 16, A, None, 2, A, None) == 1 and "both" in _err(lib)
    assert f(A, 4, 16, GU, 8, 16, None, None, 2, A, None) == 1 and "identity" in _err(lib)
    assert f(MIS, 4, 16, GU, 8, 16, A, A, 2, A, None) == 1 and "aligned" in _err(lib)
    assert f(A, 4, 16, None, 8, 16, A, A, 2, A, None) == 1 and "w_gu" in _err(lib)
    d = lib.moe_grouped_gemm_down
    assert d(A, 8, 16, DN, 8, 20, A, A, None, A, None) == 3 and "H=20" in _err(lib)
    assert d(A, 8, 16, DN, 8, 16, None, None, None, A, None) == 1 and "identity" in _err(lib)
    dn1 = _desc(0, 1, 16, 16)
    assert d(A, 8, 16, dn1, 1, 16, None, None, None, MIS, None) == 1 and "expert_out" in _err(lib)


def test_unpacked_weights_refused_by_name(lib):
    """The GEMM calls take a descriptor that moe_pack_weights fills; the
    pages' row-major weights (a descriptor without the packed layout tag),
    the other kind, other dimensions or a wrong expert size are refused
    before any launch, naming the argument."""
    f = lib.moe_grouped_gemm_gateup_silu
    d = lib.moe_grouped_gemm_down
    row_major = _desc(1, 8, 32, 16, layout=0)
    assert f(A, 4, 16, row_major, 8, 16, A, A, 2, A, None) == 1
    m = _err(lib)
    assert "w_gu" in m and "not a packed weight descriptor" in m and "moe_pack_weights" in m
    assert d(A, 8, 16, _desc(0, 8, 16, 16, layout=0x12345678), 8, 16, A, A, None, A, None) == 1
    assert "w_d" in _err(lib) and "0x12345678" in _err(lib)
    assert f(A, 4, 16, DN, 8, 16, A, A, 2, A, None) == 1 and "MOE_PACK_GATEUP" in _err(lib)
    assert d(A, 8, 16, GU, 8, 16, A, A, None, A, None) == 1 and "MOE_PACK_PLAIN" in _err(lib)
    assert f(A, 4, 16, GU, 4, 16, A, A, 2, A, None) == 1 and "8 experts" in _err(lib)
    assert f(A, 4, 32, GU, 8, 16, A, A, 2, A, None) == 1 and "[32, 16]" in _err(lib)
    assert d(A, 8, 16, DN, 8, 24, A, A, None, A, None) == 1 and "w_d" in _err(lib)
    bad_size = _desc(1, 8, 32, 16, expert_bytes=1024)
    assert f(A, 4, 16, bad_size, 8, 16, A, A, 2, A, None) == 1 and "expert size" in _err(lib)
    assert f(A, 4, 16, _desc(1, 8, 32, 16, data=0x40008), 8, 16, A, A, 2, A, None) == 1
    assert "data" in _err(lib)
    assert f(A, 4, 16, _desc(1, 8, 32, 16, data=0), 8, 16, A, A, 2, A, None) == 1
    # the fused FFN checks both
    need = lib.moe_fused_expert_ffn_workspace_bytes(4, 8, 2, 1)
    assert lib.moe_fused_expert_ffn(A, 4, 16, row_major, DN, 8, 16, A, A, 2, A, A, A, A, need,
                                    None) == 1 and "w_gu" in _err(lib)
    assert lib.moe_fused_expert_ffn(A, 4, 16, GU, GU, 8, 16, A, A, 2, A, A, A, A, need,
                                    None) == 1 and "w_d" in _err(lib)


def test_weights_slice(lib):
    W = _desc(1, 8, 32, 16, data=0x100000)
    per = W._obj.expert_bytes
    out = moe.MoeWeights()
    assert lib.moe_weights_slice(W, 2, 5, ctypes.byref(out)) == 0
    assert (out.E, out.R, out.K, out.kind) == (3, 32, 16, 1)
    assert out.data == 0x100000 + 2 * per and out.layout == moe.MOE_WEIGHTS_PACKED_V1
    for e0, e1 in [(-1, 2), (3, 3), (5, 2), (0, 9)]:
        assert lib.moe_weights_slice(W, e0, e1, ctypes.byref(out)) == 3 and "range" in _err(lib)
    assert lib.moe_weights_slice(_desc(1, 8, 32, 16, layout=0), 0, 1, ctypes.byref(out)) == 1
    r = lib.moe_router_logits
    assert r(A, 4, 10, A, 8, None, A, None) == 3
    assert r(A, 4, 16, A, 0, None, A, None) == 3


def test_combine_scale_and_gate_refusals(lib):
    c = lib.moe_combine_gate
    assert c(A, 1, 2, 2, 8, None, math.inf, None, 1, None, A2, 1, None) == 1
    assert "routed_scale" in _err(lib)
    assert c(A, 1, 2, 2, 8, None, math.nan, None, 1, None, A2, 1, None) == 1
    assert c(A, 1, 2, 2, 8, None, 1.0, None, 1, A, A2, 1, None) == 1
    assert "gate_logit" in _err(lib)
    assert c(A, 1, 2, 0, 8, None, 1.0, None, 1, None, A2, 1, None) == 3
    assert c(A, 1, 2, 2, 12, None, 1.0, None, 1, None, A2, 1, None) == 3
    assert c(A, 1, 2, 2, 8, None, 1.0, MIS, 1, None, A2, 1, None) == 1


def test_zero_tokens_is_a_no_op(lib):
    assert lib.moe_combine_gate(None, 1, 0, 2, 8, None, 1.0, None, 1, None, None, 1, None) == 0
    assert lib.moe_route(None, 0, 8, 2, None, None, A, None, None, 0, None) == 0
    assert lib.moe_grouped_gemm_gateup_silu(None, 0, 16, GU, 8, 16, A, A, 2, None, None) == 0
    assert lib.moe_grouped_gemm_down(None, 0, 16, DN, 8, 16, A, A, None, None, None) == 0
    assert lib.moe_router_logits(None, 0, 16, None, 8, None, None, None) == 0
    assert _err(lib) == ""


def test_route_noalloc_limits(lib):
    """The library-held grouping scratch is 1 MiB: 4 bytes per (1024-pair
    segment, expert). Sizes past it are refused before any launch, naming the
    sizes; the other checks are moe_route's."""
    f = lib.moe_route_noalloc
    # E = 128: 2048 segments fit (2,097,152 pairs); one more pair does not
    assert lib.moe_route_workspace_bytes(262144, 128, 8) == 1 << 20
    assert f(A, 262145, 128, 8, A, A, A, A, None) == 4
    m = _err(lib)
    assert "moe_route_noalloc" in m and "2097160 pairs" in m and "1048576" in m
    assert f(A, 4, 8, 9, A, A, A, A, None) == 3 and "K=9" in _err(lib)
    assert f(A, 4, 8, 2, A, A, None, A, None) == 1 and "expert_offsets" in _err(lib)
    assert f(None, 0, 8, 2, None, None, A, None, None) == 0 and _err(lib) == ""


def test_route_workspace_query(lib):
    assert lib.moe_route_workspace_bytes(8192, 128, 8) == 64 * 128 * 4  # 1024-pair segments
    assert lib.moe_route_workspace_bytes(512, 128, 8) == 0
    assert lib.moe_route(A, 1000, 8, 8, A, A, A, A, None, 0, None) == 4
    assert "workspace" in _err(lib)


def test_error_is_cleared_by_next_call(lib):
    lib.moe_combine_gate(A, moe.MOE_F16, 2, 2, 8, None, 1.0, None, 1, None, A2, 1, None)
    assert _err(lib) != ""
    lib.moe_route_workspace_bytes(1, 1, 1)
    lib.moe_combine_gate(None, 1, 0, 2, 8, None, 1.0, None, 1, None, None, 1, None)
    assert _err(lib) == ""


def test_valid_call_without_gpu_fails_at_device_check(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this case is for hosts without one")
    st = lib.moe_combine_gate(A, 1, 2, 2, 8, None, 1.0, None, 1, None, A2, 1, None)
    assert st == 5 and "moe_combine_gate" in _err(lib)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(moe, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        moe.load()


def test_product_code_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "mixture_experts_ffn_expert_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, fn
                assert "moe_oracle" not in txt, fn


def test_time_next_gemm_pairs(lib):
    assert lib.moe_time_next_gemm(A, None) == 1 and "both" in _err(lib)
    assert lib.moe_time_next_gemm(None, A) == 1
    assert lib.moe_time_next_gemm(None, None) == 0 and _err(lib) == ""


def test_refused_gemm_call_disarms_timing(lib):
    # armed with dummy handles: a refused GEMM call must disarm, so the next
    # valid call never touches them (here the next call is refused too)
    assert lib.moe_time_next_gemm(A, A2) == 0
    assert lib.moe_grouped_gemm_down(A, 8, 16, DN, 8, 20, A, A, None, A, None) == 3
    assert lib.moe_router_logits(None, 0, 16, None, 8, None, None, None) == 0


@pytest.mark.parametrize("E,K,score,n_group,topk_group,gscore,renorm,status,word", [
    (8, 2, 2, 1, 1, 0, 1, 1, "score"),
    (8, 2, 0, 1, 1, 2, 1, 1, "group_score"),
    (8, 2, 0, 1, 1, 0, 2, 1, "renormalize"),
    (8, 2, 0, 3, 1, 0, 1, 3, "n_group"),          # 3 does not divide 8
    (128, 2, 0, 128, 1, 0, 1, 3, "n_group"),      # more than 64 groups
    (8, 2, 0, 4, 5, 0, 1, 3, "topk_group"),
    (8, 5, 1, 4, 2, 1, 1, 3, "fewer than K"),     # 2 groups of 2 hold 4 experts
])
def test_route_scored_refusals(lib, E, K, score, n_group, topk_group, gscore, renorm, status,
                               word):
    st = lib.moe_route_scored(A, 4, E, K, score, None, n_group, topk_group, gscore, renorm,
                              A, A, A, A, None, 0, None)
    assert st == status and word in _err(lib) and "moe_route_scored" in _err(lib)


def test_packed_weight_bytes(lib):
    # 1 KiB blocks of 16 rows x 32 k; gate-up pairs gate and up blocks
    assert lib.moe_packed_weight_bytes(128, 2048, 768, 0) == 128 * 128 * 24 * 1024
    assert lib.moe_packed_weight_bytes(128, 1536, 2048, 1) == 128 * 48 * 64 * 2 * 1024
    assert lib.moe_packed_weight_bytes(2, 40, 72, 0) == 2 * 3 * 3 * 1024
    assert lib.moe_packed_weight_bytes(1, 80, 136, 1) == 1 * 3 * 5 * 2 * 1024
    assert lib.moe_packed_weight_bytes(1, 81, 136, 1) == 0       # odd R for gate-up
    assert lib.moe_packed_weight_bytes(1, 80, 12, 0) == 0        # K not a multiple of 8
    assert lib.moe_packed_weight_bytes(0, 80, 16, 0) == 0


def test_pack_refusals(lib):
    d = moe.MoeWeights()
    D = ctypes.byref(d)
    assert lib.moe_pack_weights(A, 2, 40, 12, 0, A2, D, None) == 3 and "K=12" in _err(lib)
    assert lib.moe_pack_weights(A, 2, 41, 16, 1, A2, D, None) == 3 and "even" in _err(lib)
    assert lib.moe_pack_weights(A, 2, 40, 16, 2, A2, D, None) == 1 and "kind" in _err(lib)
    assert lib.moe_pack_weights(MIS, 2, 40, 16, 0, A2, D, None) == 1 and "aligned" in _err(lib)
    assert lib.moe_pack_weights(A, 2, 40, 16, 0, None, D, None) == 1 and "packed" in _err(lib)
    assert lib.moe_pack_weights(A, 2, 40, 16, 0, A2, None, None) == 1 and "desc" in _err(lib)
    assert d.layout == 0                       # refusals leave the descriptor untouched


def test_keepquant_refusals(lib):
    assert lib.moe_q8k_bytes(4, 300) == 0 and lib.moe_q8k_bytes(0, 256) == 0
    assert lib.moe_q8k_bytes(4, 512) == 2048 + 256 + 512       # quants, scales, sums (aligned)
    assert lib.moe_quantize_q8k(A, 4, 300, A2, None) == 3 and "256" in _err(lib)
    q = lib.moe_grouped_qgemm_gateup_silu
    assert q(A, 4, 512, A2, 2, 8, 256, A, A, 2, A, None) == 2 and "MOE_Q4_K" in _err(lib)
    assert q(A, 4, 500, A2, 12, 8, 256, A, A, 2, A, None) == 3
    assert q(A, 4, 512, A2, 12, 8, 256, None, A, 2, A, None) == 1 and "both" in _err(lib)
    d = lib.moe_grouped_qgemm_down
    assert d(A, 8, 300, A2, 12, 8, 512, A, A, None, A, None) == 3
    assert d(A, 8, 256, A2, 12, 2, 512, None, None, None, A, None) == 1 and "E=1" in _err(lib)
    assert q(None, 0, 512, None, 12, 8, 256, A, A, 2, None, None) == 0
    for wt in (8, 13, 14):                                    # the other formats pass validation
        assert q(None, 0, 512, None, wt, 8, 256, A, A, 2, None, None) == 0
        assert q(A, 4, 300, A2, wt, 8, 256, A, A, 2, A, None) == 3 and "256" in _err(lib)
    assert q(A, 4, 512, A2, 15, 8, 256, A, A, 2, A, None) == 2 and "MOE_Q6_K" in _err(lib)


def test_q8_0_buffer_and_refusals(lib):
    assert lib.moe_q8_0_bytes(4, 40) == 0 and lib.moe_q8_0_bytes(0, 64) == 0
    assert lib.moe_q8_0_bytes(4, 512) == 2048 + 256             # quants, f16 scales (aligned)
    assert lib.moe_q8_0_bytes(3, 96) == 512 + 256               # 288 quant bytes, 18 scale bytes
    assert lib.moe_quantize_q8_0(A, 4, 40, A2, None) == 3 and "32" in _err(lib)
    assert lib.moe_quantize_q8_0(None, 0, 64, None, None) == 0
    assert lib.moe_quantize_q8_0(MIS, 4, 64, A2, None) == 1 and "aligned" in _err(lib)


def test_fused_ffn_workspace_and_refusals(lib):
    wb = lib.moe_fused_expert_ffn_workspace_bytes
    assert wb(32, 128, 8, 1) == (2 * (16 + 128) + 1) * 4        # 16-row slots + one per expert
    assert wb(40, 1, 1, 0) == (2 * 3 + 1) * 4                    # identity rows: 3 slots
    assert wb(0, 8, 2, 1) == 0 and wb(4, 0, 1, 1) == 0
    f = lib.moe_fused_expert_ffn
    need = wb(4, 8, 2, 1)
    G, D = _desc(1, 8, 128, 256), _desc(0, 8, 256, 64)
    #     x  T  H   w_gu w_d E  I   sorted offs K  pair_w act eo  ws  ws_bytes
    assert f(A, 4, 256, G, D, 8, 64, A, A, 2, A, A, A, A, need - 4, None) == 4
    assert "workspace" in _err(lib)
    assert f(A, 4, 256, G, D, 8, 64, A, A, 2, A, A, A, None, need, None) == 4
    assert f(A, 4, 256, G, D, 8, 64, A, A, 9, A, A, A, A, need, None) == 3 and "K=9" in _err(lib)
    assert f(A, 4, 256, G, D, 8, 64, None, A, 2, A, A, A, A, need, None) == 1
    assert f(A, 4, 250, G, D, 8, 64, A, A, 2, A, A, A, A, need, None) == 3
    assert f(A, 4, 256, G, D, 2, 64, None, None, 2, A, A, A, A, need, None) == 1
    assert f(MIS, 4, 256, G, D, 8, 64, A, A, 2, A, A, A, A, need, None) == 1
    assert "aligned" in _err(lib)
    assert f(None, 0, 256, None, None, 8, 64, A, A, 2, None, None, None, None, 0, None) == 0


def test_probe_sizes_and_refusals(lib):
    # 1,024 workgroups of 256 threads; 4 chains of 32x32x16 MFMAs per wave
    assert lib.moe_probe_out_values() == 262144
    assert lib.moe_probe_mfma_flops(10) == 4096 * 10 * 4 * 32 * 32 * 16 * 2
    assert lib.moe_probe_mfma_flops(0) == 0.0
    assert lib.moe_probe_hbm_read(None, 1024, A, None) == 1 and "buf" in _err(lib)
    assert lib.moe_probe_hbm_read(MIS, 1024, A, None) == 1 and "aligned" in _err(lib)
    assert lib.moe_probe_hbm_read(A, 1000, A2, None) == 1 and "multiple of 16" in _err(lib)
    assert lib.moe_probe_hbm_read(A, 0, A2, None) == 1
    assert lib.moe_probe_mfma_bf16(A, 0, 10, A2, None) == 1 and "n_ops" in _err(lib)
    assert lib.moe_probe_mfma_bf16(A, 64, 0, A2, None) == 1 and "iters" in _err(lib)
    assert lib.moe_probe_mfma_bf16(A, 64, 1 << 21, A2, None) == 1
    assert lib.moe_probe_mfma_bf16(A, 64, 10, None, None) == 1 and "out" in _err(lib)


def test_refused_probe_call_disarms_timing(lib):
    assert lib.moe_time_next_gemm(A, A2) == 0
    assert lib.moe_probe_hbm_read(A, 8, A2, None) == 1
    assert lib.moe_router_logits(None, 0, 16, None, 8, None, None, None) == 0


def test_packed_weights_expert_block_views(lib):
    """PackedWeights.experts views the block of experts one expert-parallel
    owner holds: the same bytes, one packed expert after another."""
    import torch
    E, R, K = 8, 2 * 96, 136
    n = moe.moe_packed_weight_bytes(E, R, K, "gateup")
    per = n // E
    assert per * E == n and per % 1024 == 0
    data = torch.arange(n, dtype=torch.int64).remainder(251).to(torch.uint8)
    desc = _desc(1, E, R, K, data=data.data_ptr())._obj
    pw = moe.PackedWeights(data, desc)
    blk = pw.experts(2, 5)
    assert (blk.E, blk.R, blk.K, blk.kind) == (3, R, K, "gateup")
    assert blk.data.numel() == moe.moe_packed_weight_bytes(3, R, K, "gateup")
    assert blk.data.data_ptr() == data.data_ptr() + 2 * per == blk.desc.data
    assert torch.equal(blk.data, data[2 * per:5 * per])
    assert pw.experts(0, E).data.numel() == n
    for e0, e1 in [(-1, 2), (3, 3), (5, 2), (0, E + 1)]:
        with pytest.raises(moe.MoeError):
            pw.experts(e0, e1)
