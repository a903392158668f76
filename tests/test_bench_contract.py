"""The benchmark's command-line contract.

* CPU: `--gpus N` with N > 1 exits with a message (one GPU only); the
  algorithmic byte and flop counts of the roofline follow their formulas for
  the bf16 and the keep-quant workloads.
* GPU: a short default run prints one JSON line carrying every field of the
  contract (metric, value, unit, steps, warmup, ms_per_step, dtype, config
  with the workload, roofline with bound / achieved / peak / frac / traffic,
  cpu_baseline null when skipped), and the roofline fraction is achieved over
  peak.
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


@pytest.mark.gpu
def test_default_run_prints_the_contract_line():
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--no-cpu-baseline", "--no-graph", "--no-fused",
                        "--ep-share"],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
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
    assert d["config"]["workload"].startswith("decode_T32")
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    assert 0 < roof["frac"] < 1
    assert d["cpu_baseline"] is None
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
