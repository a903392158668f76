"""The benchmark's command-line contract.

* CPU: `--gpus N` with N > 1 exits with a message (one GPU only); the
  algorithmic byte and flop counts of the roofline follow their formulas for
  the bf16 and the keep-quant workloads.
* CPU: the staged CPU baseline reports every stage, the host's CPU count and
  one-thread times of the tiny and decode layers.
* GPU: a short default run prints one JSON line carrying every field of the
  contract (metric, value, unit, steps, warmup, ms_per_step, dtype, config
  with the workload, roofline with bound / achieved / peak / frac / traffic,
  cpu_baseline null when skipped) for the skewed 8192-token layer, with the
  MFMA roofline, the cold-cache combine, the routing check and the compact
  runs of the decode, prefill and 256-expert layers; a decode run carries the
  HBM roofline and the expert-parallel owner shares.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_multi_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_kernel_fingerprint_covers_every_local_header():
    """roofline.traffic is reported only while the GEMM kernel code matches the
    fingerprint recorded with the counters; the fingerprint must cover
    gemm.hip and every header of the library that it includes, so a change in
    any of them drops the stale traffic figure."""
    import re
    sys.path.insert(0, ROOT)
    import bench
    csrc = os.path.join(ROOT, "mixture_experts_ffn_expert_amd", "csrc")
    seen, todo = set(), ["gemm.hip"]
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        seen.add(name)
        for inc in re.findall(r'#include\s+"([^"]+)"', open(os.path.join(csrc, name)).read()):
            if os.path.exists(os.path.join(csrc, inc)):
                todo.append(inc)
    assert seen == set(bench.KERNEL_CODE_FILES), (sorted(seen), bench.KERNEL_CODE_FILES)
    a = bench.kernel_code_fingerprint()
    assert len(a) == 64 and a == bench.kernel_code_fingerprint()


def test_algorithmic_work_formulas():
    sys.path.insert(0, ROOT)
    import bench
    import workloads as W
    cfg = W.config(2)
    T, H, E, K, I = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I
    P = T * K
    counts = np.zeros(E, np.int64)
    counts[:100] = 2
    counts[100] = P - 200                       # 101 touched experts
    offsets = np.concatenate([[0], np.cumsum(counts)])
    gu, dn, touched = bench.algorithmic_work(cfg, offsets)
    assert touched == 101
    assert gu["flops"] == 2.0 * P * 2 * I * H and dn["flops"] == 2.0 * P * H * I
    assert gu["bytes"] == 101 * 2 * I * H * 2 + T * H * 2 + P * I * 2 + P * 4 + (E + 1) * 4
    assert dn["bytes"] == 101 * H * I * 2 + P * I * 2 + P * H * 2 + P * 8 + (E + 1) * 4
    for n, blk, vals in [(7, 144, 256), (9, 210, 256), (10, 34, 32)]:
        c = W.config(n)
        gq, dq, t2 = bench.algorithmic_work(c, offsets)
        assert t2 == 101
        wbytes = 101 * 2 * I * (H // vals) * blk
        assert wbytes < gq["bytes"] < wbytes + 1_000_000


def test_cpu_baseline_reports_stages_and_cores():
    sys.path.insert(0, ROOT)
    import bench
    import workloads as W
    r = bench.cpu_baseline(W.make_inputs(1), 16, single_thread_workloads=(1,))
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0
    assert set(r["stages_s"]) == {"router_logits", "route", "gateup", "down", "shared", "combine"}
    assert r["nproc"] == os.cpu_count() and 1 <= r["cores"] <= r["affinity_cpus"]
    one = r["single_thread"]["tiny_T16_H64_E8_K2_I32_shared32"]
    assert one["tokens_per_s"] > 0 and abs(sum(one["stages_s"].values()) - one["seconds"]) < 1e-9


def _run(args):
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py")] + args,
                       capture_output=True, text=True, cwd=ROOT, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "tokens/s" and d["value"] > 0 and d["higher_is_better"] is True
    assert d["cpu_baseline"] is None
    return d


def _check_combine(c, cfg):
    T, K, H, I_s = cfg["T"], cfg["K"], cfg["H"], cfg["I_shared"]
    assert c["bytes"] == T * K * H * 2 + T * H * 2 + (T * H * 2 + T * 4 if I_s else 0)
    assert c["us"] > 0 and abs(c["gbs"] - c["bytes"] / (c["us"] * 1e-6) / 1e9) < 1e-6 * c["gbs"]
    assert 0 < c["frac_of_hbm_peak"] < 1.2


@pytest.mark.gpu
def test_default_run_is_the_skewed_layer_with_compact_configs():
    d = _run(["--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--no-graph", "--no-fused",
              "--sub-steps", "2"])
    assert d["config"]["workload"] == "skewed_T8192_H4096_E128_K8_I1536"
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9 and 0 < roof["frac"] < 1
    gu_us = d["grouped_gemm"]["gateup_us"]
    assert abs(roof["achieved"] - roof["algorithmic"]["flops_per_launch"] / gu_us / 1e6) < 1e-6 * roof["achieved"]
    c = d["measured_ceilings"]
    assert abs(roof["frac_of_measured"] - roof["achieved"] / c["mfma_bf16_tflops"]) < 1e-9
    _check_combine(d["combine"], d["config"])
    rc = d["routing_check"]
    assert rc["tokens"] == 8192 and 0 <= rc["logit_max_abs_err"] < 1e-3
    assert rc["tokens_whose_topk_set_differs_from_f64"] <= rc["tokens_with_gap_within_2x_err"]
    subs = d["configs"]
    assert set(subs) == {"decode_T32_H2048_E128_K8_I768", "prefill_T4096_H2048_E128_K8_I768",
                         "shared_T512_H2048_E256_K8_I512_shared512"}
    # the prefill gate-up's intensity (about 237 flop/B) sits below the ridge
    # of 2.5 PFLOP/s over 8 TB/s (312.5 flop/B): HBM-bound by the roofline
    bounds = {"decode_T32_H2048_E128_K8_I768": "hbm", "prefill_T4096_H2048_E128_K8_I768": "hbm",
              "shared_T512_H2048_E256_K8_I512_shared512": "hbm"}
    for name, r in subs.items():
        assert r["tokens_per_s"] > 0 and r["gateup_us"] > 0 and r["down_us"] > 0
        assert r["roofline"]["bound"] == bounds[name]
        assert abs(r["roofline"]["frac"] - r["roofline"]["achieved"] / r["roofline"]["peak"]) < 1e-9
        assert (r["roofline"]["flop_per_byte"] < 312.5) == (r["roofline"]["bound"] == "hbm")
        assert abs(r["roofline"]["frac_of_mfma_peak"] * 2500.0 - r["roofline"]["tflops"]) < 1e-6
        T = int(name.split("_T")[1].split("_")[0])
        H = int(name.split("_H")[1].split("_")[0])
        K = int(name.split("_K")[1].split("_")[0])
        _check_combine(r["combine"], {"T": T, "K": K, "H": H, "I_shared": 512 if "shared512" in name else 0})


@pytest.mark.gpu
def test_decode_run_prints_the_contract_line():
    d = _run(["--workload", "2", "--steps", "3", "--warmup", "1", "--no-cpu-baseline",
              "--no-graph", "--no-fused", "--ep-share"])
    assert d["config"]["workload"].startswith("decode_T32")
    assert d["configs"] is None
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    assert 0 < roof["frac"] < 1
    # the chip's own ceilings from the library's micro-kernels, and the same
    # achieved figure against the measured read ceiling
    c = d["measured_ceilings"]
    assert 1000 < c["hbm_read_gbs"] < 8000 and 100 < c["mfma_bf16_tflops"] < 2600
    assert abs(roof["frac_of_measured"] - roof["achieved"] / c["hbm_read_gbs"]) < 1e-9
    # the GEMMs at each expert-parallel owner's share: every pair belongs to
    # exactly one owner, and the slowest owner bounds the layer
    ep = d["expert_parallel_share"]
    assert ep["shards"] == 8 and ep["experts_per_shard"] == 16
    rows = ep["per_shard"]
    assert sum(r["pairs"] for r in rows) == 32 * 8
    assert [r["experts"] for r in rows] == [[16 * b, 16 * b + 16] for b in range(8)]
    tot = [r["gateup_us"] + r["down_us"] for r in rows]
    assert all(t > 0 for t, r in zip(tot, rows) if r["pairs"] > 0)
    assert ep["max_gemm_us"] == max(tot)
    # GPU clock / power while the steps ran (sysfs of the device, best effort)
    # and the cache-resident read that the 2 GiB read is compared against
    gs = d["gpu_state"]
    assert gs["samples"] >= 1 and gs["sysfs"].startswith("/sys/bus/pci/devices/")
    assert c["control_64MiB_read_gbs"] > 0
