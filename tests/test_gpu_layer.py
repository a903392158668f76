"""End-to-end GPU parity of one MoE layer (logits -> route -> gate-up ->
down -> shared expert -> combine) on every workload, in the launch
configuration the benchmark times, plus hipGraph replay and determinism.

Each stage is held to its own bar given the inputs it actually received: the
oracle routes on the GPU's f32 logits (bit-exact; a different summation order
can flip a near-tie, so routing parity is judged on identical logits), act is
compared with the oracle's act from x (GEMM bar), expert_out with the
oracle's down-projection of the GPU's act (GEMM bar), the combine with the
oracle's combine of the GPU's expert_out / shared / gate logit (bit-exact).
The whole chain against the oracle's own chain must keep NMSE <= 1e-5 (its
element errors are sums of the stage errors, so the element bar is applied
stage by stage). The routing the oracle computes from its own logits may
differ only on tokens whose K-th / (K+1)-th logit gap is below the logit
error.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from conftest import cached_inputs
from gpu_helpers import (DEV, assert_bits_equal, assert_gemm_close, bits, packed_d, packed_gu,
                         sample_rows, sub_down, sub_gateup, to_dev_bf16)

import mixture_experts_ffn_expert_amd as moe

pytestmark = pytest.mark.gpu


def _dev_inputs(d):
    t = {k: to_dev_bf16(d[k]) for k in ("x", "w_r")}
    t["w_gu"], t["w_d"] = packed_gu(d["w_gu"]), packed_d(d["w_d"])
    t["router_bias"] = None
    if "router_bias" in d:
        t["router_bias"] = torch.from_numpy(d["router_bias"]).to(DEV)
    t["selection_bias"] = None
    if "selection_bias" in d:
        t["selection_bias"] = torch.from_numpy(d["selection_bias"]).to(DEV)
    t["router"] = W.router_args(d["cfg"])
    t["w_gu_s"] = packed_gu(d["w_gu_s"]) if "w_gu_s" in d else None
    t["w_d_s"] = packed_d(d["w_d_s"]) if "w_d_s" in d else None
    t["w_g"] = to_dev_bf16(d["w_g"]) if "w_g" in d else None
    return t


def _run(t, K, bufs=None):
    router = None if t["router"] is None else dict(t["router"])
    scale = 1.0 if router is None else router.pop("routed_scale")
    return moe.moe_layer(t["x"], t["w_r"], t["w_gu"], t["w_d"], K, t["router_bias"], t["w_gu_s"],
                         t["w_d_s"], t["w_g"], bufs=bufs, router=router,
                         selection_bias=t["selection_bias"], routed_scale=scale)


def _routing_flips_are_near_ties(gpu_logits, ref_logits, K):
    ids_gpu = O.topk_ids(gpu_logits, K)
    ids_ref = O.topk_ids(ref_logits, K)
    diff = np.any(ids_gpu != ids_ref, axis=1)
    if not diff.any():
        return 0
    err = np.max(np.abs(gpu_logits.astype(np.float64) - ref_logits), axis=1)
    srt = -np.sort(-ref_logits.astype(np.float64), axis=1)
    gaps = np.min(np.abs(np.diff(srt[:, :K + 1], axis=1)), axis=1)
    assert np.all(gaps[diff] <= 2 * err[diff]), "routing differs away from a near-tie"
    return int(diff.sum())


@pytest.mark.parametrize("n", [1, 2, 3, 4, 6])
def test_layer_end_to_end(gpu_lib, n):
    d = cached_inputs(n)
    cfg = d["cfg"]
    print(f"layer cfg={n} T={cfg.T}", flush=True)
    t = _dev_inputs(d)
    bufs = {}
    out = _run(t, cfg.K, bufs)
    torch.cuda.synchronize()
    g_logits = bits(bufs["logits"])
    ref = O.moe_layer(d, logits=g_logits, keep=True)
    assert_bits_equal(bits(bufs["ids"]), ref["ids"], "ids")
    assert_bits_equal(bits(bufs["w"]), ref["w"], "weights")
    assert_bits_equal(bits(bufs["offsets"]), ref["offsets"], "offsets")
    assert_bits_equal(bits(bufs["sorted"]), ref["sorted_pairs"], "sorted_pairs")
    act = bits(bufs["act"])
    assert_gemm_close(act, ref["act"], "act")
    w_flat = ref["w"].reshape(-1)
    eo_ref = O.down_proj(act, d["w_d"], ref["sorted_pairs"], ref["offsets"], w_flat)
    eo = bits(bufs["expert_out"])
    assert_gemm_close(eo, eo_ref, "expert_out")
    sd = gl = None
    if ref["sd"] is not None:
        sa = bits(bufs["sd_act"])
        assert_gemm_close(sa, O.gateup_silu(d["x"], d["w_gu_s"][None], None, None, 1), "shared act")
        sd = bits(bufs["sd"])
        assert_gemm_close(sd, O.down_proj(sa, d["w_d_s"][None], None, None, None), "shared out")
        gl = bits(bufs["gl"]).reshape(-1)
        assert np.max(np.abs(gl.astype(np.float64) - ref["gl"])) <= 1e-4 * np.max(np.abs(ref["gl"])) + 1e-6
    scale = 1.0 if t["router"] is None else t["router"]["routed_scale"]
    assert_bits_equal(bits(out), O.combine_gate(eo, cfg.T, cfg.K, cfg.H, None, scale, sd, gl),
                      "combine")
    g = O.f32_from_bf16(bits(out)).astype(np.float64)
    r = O.f32_from_bf16(ref["out"]).astype(np.float64)
    nmse = float(np.sum((g - r) ** 2) / np.sum(r * r))
    assert nmse <= 1e-5, f"layer chain NMSE {nmse:.3e}"
    # the oracle's own logits route the same way except at near-ties
    if t["router"] is None:
        o_logits = O.router_logits(d["x"], d["w_r"], d.get("router_bias"))
        flips = _routing_flips_are_near_ties(g_logits, o_logits, cfg.K)
        print(f"cfg{n}: tokens routed differently on own logits: {flips}")


def test_layer_skewed_full_size_sampled(gpu_lib):
    d = cached_inputs(5)
    cfg = d["cfg"]
    print(f"layer cfg=5 T={cfg.T}", flush=True)
    t = _dev_inputs(d)
    bufs = {}
    out = _run(t, cfg.K, bufs)
    torch.cuda.synchronize()
    g_logits = bits(bufs["logits"])
    ids, w, off, sp = O.route(g_logits, cfg.K)
    assert_bits_equal(bits(bufs["ids"]), ids, "ids")
    assert_bits_equal(bits(bufs["w"]), w, "weights")
    assert_bits_equal(bits(bufs["offsets"]), off, "offsets")
    assert_bits_equal(bits(bufs["sorted"]), sp, "sorted_pairs")
    counts = np.diff(off)
    assert counts.max() > 10 * counts.mean()
    # sampled tokens: their K pairs through the oracle, then the combine
    rng = np.random.Generator(np.random.PCG64(55))
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.integers(0, cfg.T, 62)]))
    inv = np.empty_like(sp)
    inv[sp] = np.arange(sp.size)
    pairs = (toks[:, None] * cfg.K + np.arange(cfg.K)[None, :]).reshape(-1)
    qs = inv[pairs]
    order = np.argsort(qs)
    qs_sorted = qs[order]
    act_ref = sub_gateup(d["x"], d["w_gu"], sp, off, cfg.K, qs_sorted)
    act_gpu = bits(bufs["act"])[qs_sorted]
    assert_gemm_close(act_gpu, act_ref, "act (sampled)")
    eo_ref = sub_down(act_gpu, d["w_d"], off, qs_sorted, w.reshape(-1)[sp[qs_sorted]])
    eo_ref_rows = np.empty((pairs.size, cfg.H), np.uint16)
    eo_ref_rows[order] = eo_ref
    eo_gpu_rows = bits(bufs["expert_out"])[pairs]
    assert_gemm_close(eo_gpu_rows, eo_ref_rows, "expert_out (sampled)")
    assert_bits_equal(bits(out)[toks], O.combine_gate(eo_gpu_rows, toks.size, cfg.K, cfg.H),
                      "combine (sampled)")
    chain = O.combine_gate(sub_down(act_ref, d["w_d"], off, qs_sorted,
                                    w.reshape(-1)[sp[qs_sorted]])[np.argsort(order)],
                           toks.size, cfg.K, cfg.H)
    g = O.f32_from_bf16(bits(out)[toks]).astype(np.float64)
    r = O.f32_from_bf16(chain).astype(np.float64)
    assert float(np.sum((g - r) ** 2) / np.sum(r * r)) <= 1e-5


def test_layer_deterministic_and_graph_replay(gpu_lib):
    d = cached_inputs(4)
    cfg = d["cfg"]
    t = _dev_inputs(d)
    bufs = {}
    out = _run(t, cfg.K, bufs).clone()
    torch.cuda.synchronize()
    again = _run(t, cfg.K, bufs).clone()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))
    moe.moe_init()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        _run(t, cfg.K, bufs)          # warm-up on the capture stream
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        _run(t, cfg.K, bufs)
    for i in range(4):
        bufs["out"].zero_()
        bufs["act"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs["out"].view(torch.int16), out.view(torch.int16)), f"replay {i}"


@pytest.mark.parametrize("n", [1, 4, 6])
def test_shared_expert_on_a_second_stream(gpu_lib, n):
    """The benchmark's layer schedule: the shared expert (gate-up, down, gate
    logit) on a second stream forked from the layer's stream, the routed path
    on the layer's stream, joined before the combine; three steps in a row and
    a graph replay of the same schedule, each bit-identical to the sequential
    layer."""
    d = cached_inputs(n)
    cfg = d["cfg"]
    print(f"two-stream layer cfg={n} T={cfg.T}", flush=True)
    t = _dev_inputs(d)
    ref = bits(_run(t, cfg.K)).copy()
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)
    b = {}
    router = None if t["router"] is None else dict(t["router"])
    scale = 1.0 if router is None else router.pop("routed_scale")

    def step():
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            sa = moe.moe_grouped_gemm_gateup_silu(t["x"], t["w_gu_s"], None, None, 1, b.get("sa"))
            sd = moe.moe_grouped_gemm_down(sa, t["w_d_s"], None, None, None, b.get("sd"))
            gl = moe.moe_router_logits(t["x"], t["w_g"].view(1, -1), None, b.get("gl"))
        b.update(sa=sa, sd=sd, gl=gl)
        logits = moe.moe_router_logits(t["x"], t["w_r"], t["router_bias"], b.get("logits"))
        if router is None:
            ids, w, off, sp = moe.moe_route(logits, cfg.K, b.get("ids"), b.get("w"),
                                            b.get("off"), b.get("sp"), b.get("ws"))
        else:
            ids, w, off, sp = moe.moe_route_scored(
                logits, cfg.K, selection_bias=t["selection_bias"], **router, topk_ids=b.get("ids"),
                topk_w=b.get("w"), expert_offsets=b.get("off"), sorted_pairs=b.get("sp"),
                workspace=b.get("ws"))
        act = moe.moe_grouped_gemm_gateup_silu(t["x"], t["w_gu"], sp, off, cfg.K, b.get("act"))
        eo = moe.moe_grouped_gemm_down(act, t["w_d"], sp, off, w, b.get("eo"))
        b.update(logits=logits, ids=ids, w=w, off=off, sp=sp, act=act, eo=eo)
        main.wait_stream(side)
        out = moe.moe_combine_gate(eo, cfg.T, cfg.K, None, scale, sd, gl, b.get("out"))
        b["out"] = out
        return out

    nws = moe.moe_route_workspace_bytes(cfg.T, cfg.E, cfg.K)
    b["ws"] = torch.empty((nws,), dtype=torch.uint8, device=DEV) if nws else None
    for _ in range(3):
        out = step()
        torch.cuda.synchronize()
        assert_bits_equal(bits(out), ref, "two-stream layer output")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        b["out"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(bits(b["out"]), ref, "two-stream layer output, graph replay")
