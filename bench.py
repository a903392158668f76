"""Benchmark of one MoE layer of the BF16 expert path on one MI355X.

A step is one whole layer over one batch of synthetic tokens: router logits,
softmax top-k routing with expert grouping, grouped gate-up GEMM + SiLU-mul,
grouped down-projection with the routing weight in its epilogue, the shared
expert when the workload has one, and the combine. Inputs (seeded, random
weights of the workload's shape) are resident in HBM before timing starts.

Prints ONE JSON line. The headline workload (default 5) is the largest
configuration: 8192 tokens, H=4096, 128 experts, top-8, I=1536, with the
Zipf-skewed router. `value` is its layer tokens/s (T * steps / elapsed).
The `roofline` object describes the dominant kernel (the grouped gate-up
GEMM), timed on every fifth step of the timed region by HIP events that its
kernel records itself (start and end of the kernel, on the stream it runs
on); `traffic` is its HBM bytes per launch from committed rocprofv3 counter
runs, while the kernel code is the one they were taken on. `combine` times
the combine alone under a cold-cache protocol (a 1 GiB read between
launches evicts the 256 MB last-level cache). `routing_check` compares the
GPU's router logits with float64 dot products and counts the tokens whose
K-th / (K+1)-th logit gap is within that error. `configs` holds compact
results of the decode (2), prefill (3) and 256-expert shared-expert (4)
layers, each against its own roofline. `cpu_baseline` times the CPU oracle
stage by stage on a bounded sample of the headline workload, with one-thread
times of the tiny and decode layers.

The steps cycle through `--layers` weight sets (same values, distinct
addresses), so no step finds its weights in the last-level cache left by the
step before, as in a model whose consecutive MoE layers hold distinct
weights. `hipgraph` times the same steps captured once into a HIP graph and
replayed. `measured_ceilings` holds the chip's read and MFMA ceilings from
the library's micro-kernels (with a cache-resident read as a control) and
`gpu_state` the clock, power and temperature sampled while the steps ran.
With `--ep-share`, `expert_parallel_share` times the grouped GEMMs of each
owner of E/8 experts on its own pairs (one GPU's share of an 8-way
expert-parallel layer).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N]
       (--workload picks one of the ten workloads: 1 tiny, 2 decode, 3
       prefill, 4 256 experts with a gated shared expert, 5 skewed 8192
       tokens (default), 6 the 256-expert layer with the grouped sigmoid
       router, 7-10 the decode layer with Q4_K, Q5_K, Q6_K and Q8_0 expert
       weights on the keep-quant path). Progress goes to stderr.
"""
import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
# The GEMM kernels record their own start and end on every TIMING_EVERY-th
# timed step: a launch armed that way (hipExtLaunchKernel with events) adds
# about 10 us to a 173 us decode step, so arming every step would understate
# the layer's throughput.
TIMING_EVERY = 5
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
MFMA_I8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s


def algorithmic_work(cfg, offsets):
    """Algorithmic bytes and flops of the GEMM launches (touched experts only)."""
    T, H, E, K, I = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I
    P = T * K
    counts = np.diff(offsets)
    touched = int(np.count_nonzero(counts))
    wtype = getattr(cfg, "weights", "bf16")
    if wtype != "bf16":
        # GGUF weight blocks (bytes per block of `vals` weights); activations
        # quantized to 1 byte per value plus, per 256 values, a 4-byte scale
        # and sixteen 4-byte sums (Q8_K), or per 32 a 2-byte scale (Q8_0)
        blk, vals = {"q4_k": (144, 256), "q5_k": (176, 256), "q6_k": (210, 256),
                     "q8_0": (34, 32)}[wtype]
        if wtype == "q8_0":
            q8 = lambda rows, k: rows * k + rows * (k // 32) * 2
        else:
            q8 = lambda rows, k: rows * k + rows * (k // 256) * 4 + rows * (k // 16) * 4
        gu = {
            "flops": 2.0 * P * (2 * I) * H,
            "bytes": touched * 2 * I * (H // vals) * blk + q8(T, H) + P * I * 2 + P * 4
                     + (E + 1) * 4,
        }
        dn = {
            "flops": 2.0 * P * H * I,
            "bytes": touched * H * (I // vals) * blk + q8(P, I) + P * H * 2 + P * 4 + P * 4
                     + (E + 1) * 4,
        }
        return gu, dn, touched
    gu = {
        "flops": 2.0 * P * (2 * I) * H,
        # weights of touched experts once + x once + act written + routing arrays
        "bytes": touched * 2 * I * H * 2 + T * H * 2 + P * I * 2 + P * 4 + (E + 1) * 4,
    }
    dn = {
        "flops": 2.0 * P * H * I,
        # weights of touched experts once + act read + expert_out written + weights, arrays
        "bytes": touched * H * I * 2 + P * I * 2 + P * H * 2 + P * 4 + P * 4 + (E + 1) * 4,
    }
    return gu, dn, touched


KERNEL_CODE_FILES = ("gemm.hip", "device_math.h", "launch.h", "lds_dma.h", "silu_table.h")


def kernel_code_fingerprint():
    """sha256 of the GEMM kernel code (gemm.hip and its headers) with
    comments and whitespace removed: it changes when the code changes, not
    when a comment does."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in KERNEL_CODE_FILES:
        txt = open(os.path.join(ROOT, "mixture_experts_ffn_expert_amd", "csrc", name)).read()
        txt = re.sub(r"/\*.*?\*/", " ", txt, flags=re.S)
        txt = re.sub(r"//[^\n]*", " ", txt)
        h.update(re.sub(r"\s+", "", txt).encode())
    return h.hexdigest()


# committed rocprofv3 FETCH_SIZE / WRITE_SIZE summaries of the gate-up GEMM
TRAFFIC_SUMMARIES = {2: "decode_gateup_hbm_traffic.md", 3: "prefill_gateup_hbm_traffic.md",
                     4: "e256_gateup_hbm_traffic.md", 5: "skewed_gateup_hbm_traffic.md"}


def measured_traffic(workload):
    """HBM bytes per gate-up launch from the committed rocprofv3 counter runs.

    Only valid while the GEMM kernel code is the one the counters were taken
    on (its fingerprint is recorded in the summary); otherwise None.
    """
    import re
    name = TRAFFIC_SUMMARIES.get(workload)
    if name is None:
        return None
    try:
        txt = open(os.path.join(ROOT, "profiles", name)).read()
        sha = kernel_code_fingerprint()
    except OSError:
        return None
    m_sha = re.search(r"kernel_code_sha256:\s*([0-9a-f]{64})", txt)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", txt)
    if not m_sha or not m_val or m_sha.group(1) != sha:
        return None
    return int(m_val.group(1))


def measure_ceilings(moe, torch, dev, reps=5):
    """The chip's own ceilings, from the library's two micro-kernels: a
    streaming read of a 2 GiB buffer (8x the last-level cache) and a
    register-only bf16 MFMA loop on random operands. Each is timed by the
    events its kernel records, mean of `reps` launches after two warm-ups."""
    stream = torch.cuda.current_stream()

    def timed(launch):
        for _ in range(2):
            launch()
        evs = []
        for _ in range(reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            for x in e:
                x.record(stream)
            evs.append(e)
        torch.cuda.synchronize()
        for a, b in evs:
            moe.moe_time_next_gemm(a, b)
            launch()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e-3  # s

    nbytes = 1 << 31
    buf = torch.full((nbytes,), 1, dtype=torch.uint8, device=dev)
    out_i = torch.empty((moe.moe_probe_out_values(),), dtype=torch.int32, device=dev)
    t_read = timed(lambda: moe.moe_probe_hbm_read(buf, out_i))
    del buf
    # negative control: the same read of a 64 MiB buffer, which the 256 MB
    # last-level cache can hold between launches
    small = 1 << 26
    buf = torch.full((small,), 1, dtype=torch.uint8, device=dev)
    t_small = timed(lambda: moe.moe_probe_hbm_read(buf, out_i))
    del buf
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    ops = torch.randn((1 << 21,), generator=gen, device=dev).to(torch.bfloat16)
    out_f = torch.empty((moe.moe_probe_out_values(),), dtype=torch.float32, device=dev)
    iters = 2000
    t_mfma = timed(lambda: moe.moe_probe_mfma_bf16(ops, iters, out_f))
    return {"hbm_read_gbs": nbytes / t_read / 1e9,
            "control_64MiB_read_gbs": small / t_small / 1e9,
            "mfma_bf16_tflops": moe.moe_probe_mfma_flops(iters) / t_mfma / 1e12,
            "method": "library micro-kernels (moe_probe_hbm_read on a 2 GiB buffer; "
                      "moe_probe_mfma_bf16, register-only v_mfma_f32_32x32x16_bf16 on random bf16 "
                      f"operands, {iters} iterations), kernel-recorded events, mean of {reps}"}


class GpuStateSampler:
    """Clock, power and temperature of the GPU in use, read from its sysfs
    node (found by PCI address) by a thread that samples them 5 ms into a
    region, then every 50 ms, and once at its end. Best effort: None where
    the node is not readable."""

    def __init__(self, torch, dev):
        import threading
        p = torch.cuda.get_device_properties(dev)
        self.base = (f"/sys/bus/pci/devices/{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:"
                     f"{p.pci_device_id:02x}.0")
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _cur_mhz(self, name):
        import re
        try:
            for line in open(os.path.join(self.base, name)):
                if line.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                    return int(m.group(1)) if m else None
        except OSError:
            pass
        return None

    def _hwmon(self, name, scale):
        import glob
        for f in sorted(glob.glob(os.path.join(self.base, "hwmon", "hwmon*", name))):
            try:
                return int(open(f).read().strip()) / scale
            except (OSError, ValueError):
                continue
        return None

    def read(self):
        return {"sclk_mhz": self._cur_mhz("pp_dpm_sclk"), "mclk_mhz": self._cur_mhz("pp_dpm_mclk"),
                "power_w": self._hwmon("power1_average", 1e6) or self._hwmon("power1_input", 1e6),
                "temp_c": self._hwmon("temp2_input", 1e3) or self._hwmon("temp1_input", 1e3)}

    def _run(self):
        # the first sample 5 ms in, when the clock has had time to follow the
        # load, then every 50 ms
        while not self._stop.wait(0.005 if not self.samples else 0.05):
            self.samples.append(self.read())

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()
        self.samples.append(self.read())  # at the end of the region

    def summary(self, idle):
        out = {"sysfs": self.base, "samples": len(self.samples), "idle_before": idle}
        for k in ("sclk_mhz", "mclk_mhz", "power_w", "temp_c"):
            v = [s[k] for s in self.samples if s[k] is not None]
            out[k] = ({"min": min(v), "median": float(np.median(v)), "max": max(v)} if v else None)
        return out


EP_SHARDS = 8


def expert_parallel_share(moe, torch, x, layers, off_dev, sp_dev, w_dev, cfg, reps=10):
    """The grouped GEMMs that each GPU of an EP_SHARDS-way expert-parallel
    layer would run, timed one owner at a time on this GPU. The owner of a
    contiguous block of E / EP_SHARDS experts receives only its own pairs,
    their x rows grouped by expert (what the all-to-all would deliver; the
    gather is done here outside the timed region), and runs the same gate-up
    and down calls on them with K = 1, identity pair order and offsets
    rebased to its first pair, on its experts' packed weights only. The
    exchange itself is not part of it. Weight sets rotate over the layers so
    that every timed call reads its weights from HBM."""
    E, K, H, I = cfg.E, cfg.K, cfg.H, cfg.I
    dev = x.device
    nb = E // EP_SHARDS
    off = off_dev.cpu().numpy().astype(np.int64)
    sp = sp_dev.cpu().numpy().astype(np.int64)
    w_flat = w_dev.reshape(-1)
    L = len(layers)
    shards = []
    for b in range(EP_SHARDS):
        e0, e1 = b * nb, (b + 1) * nb
        q0, q1 = int(off[e0]), int(off[e1])
        n = q1 - q0
        row = {"experts": [e0, e1], "pairs": n,
               "touched_experts": int(np.count_nonzero(np.diff(off[e0:e1 + 1])))}
        if n == 0:
            row.update(gateup_us=0.0, down_us=0.0)
            shards.append(row)
            continue
        pairs = torch.from_numpy(sp[q0:q1]).to(dev)
        xs = x.index_select(0, pairs // K).contiguous()
        offs = torch.from_numpy((off[e0:e1 + 1] - q0).astype(np.int32)).to(dev)
        idn = torch.arange(n, dtype=torch.int32, device=dev)
        ws = w_flat.index_select(0, pairs).contiguous()
        act = torch.empty((n, I), dtype=torch.bfloat16, device=dev)
        eo = torch.empty((n, H), dtype=torch.bfloat16, device=dev)
        wsets = [(lw["w_gu"].experts(e0, e1), lw["w_d"].experts(e0, e1)) for lw in layers]

        def call(i, evs=None):
            wgu, wd = wsets[i % L]
            if evs:
                moe.moe_time_next_gemm(evs[0], evs[1])
            moe.moe_grouped_gemm_gateup_silu(xs, wgu, idn, offs, 1, act)
            if evs:
                moe.moe_time_next_gemm(evs[2], evs[3])
            moe.moe_grouped_gemm_down(act, wd, idn, offs, ws, eo)

        for i in range(2 * L):
            call(i)
        pool = []
        for _ in range(reps):
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            for e in evs:
                e.record()
            pool.append(evs)
        torch.cuda.synchronize()
        for i in range(reps):
            call(i, pool[i])
        torch.cuda.synchronize()
        gu = float(np.mean([a.elapsed_time(b_) for a, b_, _, _ in pool])) * 1e3
        dn = float(np.mean([c.elapsed_time(d_) for _, _, c, d_ in pool])) * 1e3
        row.update(gateup_us=gu, down_us=dn)
        shards.append(row)
    tot = [r["gateup_us"] + r["down_us"] for r in shards]
    hot = int(np.argmax(tot))
    flops_hot = 2.0 * shards[hot]["pairs"] * 3 * H * I
    return {
        "shards": EP_SHARDS, "experts_per_shard": nb, "per_shard": shards,
        "max_gemm_us": max(tot), "mean_gemm_us": float(np.mean(tot)),
        "imbalance": max(tot) / float(np.mean(tot)) if np.mean(tot) > 0 else None,
        "slowest_shard": hot,
        "slowest_shard_tflops": flops_hot / (tot[hot] * 1e-6) / 1e12 if tot[hot] > 0 else None,
        "note": "GEMMs only, at each owner's real pair count; the two all-to-all "
                "exchanges are not built (one GPU)",
    }


def log(msg):
    """Progress on stderr (stdout carries the one JSON line)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def combine_bytes(cfg):
    """Algorithmic bytes of one combine launch: expert_out read, the shared
    term and gate logit read (when present), out written."""
    T, H, K = cfg.T, cfg.H, cfg.K
    b = T * K * H * 2 + T * H * 2
    if cfg.I_s:
        b += T * H * 2 + T * 4
    return b


class Layer:
    """Device state of one workload: `n_layers` weight sets (the same values
    at distinct addresses), the routing workspace and the output buffers of
    the last step, and the step itself."""

    def __init__(self, moe, torch, dev, workload, n_layers, fused=True):
        import workloads
        self.moe, self.torch, self.dev = moe, torch, dev
        self.workload = workload
        d = workloads.make_inputs(workload)
        self.d = d
        cfg = self.cfg = d["cfg"]

        def bf(a):
            return torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(dev)

        self.x = bf(d["x"])
        self.bias = torch.from_numpy(d["router_bias"]).to(dev) if "router_bias" in d else None
        router = workloads.router_args(cfg)
        self.routed_scale = 1.0
        self.sel_bias = None
        if router is not None:
            router = dict(router)
            self.routed_scale = router.pop("routed_scale")
            self.sel_bias = torch.from_numpy(d["selection_bias"]).to(dev)
        self.router = router
        # expert weights are packed once into the library's layout (a
        # load-time format change, outside the timed region)
        pack_kind = {"w_gu": "gateup", "w_d": "plain", "w_gu_s": "gateup", "w_d_s": "plain"}
        names = [n for n in ("w_r", "w_gu", "w_d", "w_gu_s", "w_d_s", "w_g") if n in d]
        self.wtype = cfg.weights
        self.keepquant = self.wtype != "bf16"
        self.layers = []
        for _ in range(max(1, n_layers)):
            lw = {}
            for n in names:
                if self.keepquant and n in ("w_gu", "w_d"):
                    continue
                t = bf(d[n])
                lw[n] = moe.moe_pack_weights(t, pack_kind[n]) if n in pack_kind else t
                del t
            if self.keepquant:
                # GGUF blocks are used as they are (keep-quant)
                lw["w_gu"] = torch.from_numpy(d["w_gu_kq"]).to(dev)
                lw["w_d"] = torch.from_numpy(d["w_d_kq"]).to(dev)
            torch.cuda.synchronize()
            self.layers.append(lw)
        T, E, K = cfg.T, cfg.E, cfg.K
        self.bufs = {}
        ws_bytes = moe.moe_route_workspace_bytes(T, E, K)
        self.ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev) if ws_bytes else None
        # the decode shapes also time the layer with the fused expert FFN
        # (moe_fused_expert_ffn) in place of the two GEMM calls
        self.fused_ok = (not self.keepquant) and T * K <= 8 * E and fused
        self.ws_f = None
        if self.fused_ok:
            nws = moe.moe_fused_expert_ffn_workspace_bytes(T, E, K, True) // 4
            self.ws_f = torch.zeros((nws,), dtype=torch.int32, device=dev)
        # the shared expert does not depend on the routing: it runs on a
        # second stream (default priority), forked from and joined back into
        # the layer's stream, so its small launches overlap the routing and
        # the routed GEMMs
        self.side = torch.cuda.Stream(device=dev)
        self.ev = []

    def release(self):
        self.layers.clear()
        self.bufs.clear()
        self.x = self.ws = self.ws_f = None

    def step(self, record, li, fused=False):
        moe, torch, bufs = self.moe, self.torch, self.bufs
        cfg = self.cfg
        T, H, K = cfg.T, cfg.H, cfg.K
        lw = self.layers[li % len(self.layers)]
        x = self.x
        w_r, w_gu, w_d = lw["w_r"], lw["w_gu"], lw["w_d"]
        w_gu_s, w_d_s, w_g = lw.get("w_gu_s"), lw.get("w_d_s"), lw.get("w_g")
        main = torch.cuda.current_stream()  # the capture stream under graph capture
        sd = gl = None
        if w_gu_s is not None:
            self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                sa = moe.moe_grouped_gemm_gateup_silu(x, w_gu_s, None, None, 1, bufs.get("sd_act"))
                sd = moe.moe_grouped_gemm_down(sa, w_d_s, None, None, None, bufs.get("sd"))
                gl = moe.moe_router_logits(x, w_g.view(1, H), None, bufs.get("gl"))
            bufs.update(sd_act=sa, sd=sd, gl=gl)
        logits = moe.moe_router_logits(x, w_r, self.bias, bufs.get("logits"))
        bufs["logits"] = logits
        if self.router is None:
            ids, w, off, sp = moe.moe_route(logits, K, bufs.get("ids"), bufs.get("w"),
                                            bufs.get("offsets"), bufs.get("sorted"), self.ws)
        else:
            ids, w, off, sp = moe.moe_route_scored(
                logits, K, selection_bias=self.sel_bias, **self.router,
                topk_ids=bufs.get("ids"), topk_w=bufs.get("w"),
                expert_offsets=bufs.get("offsets"), sorted_pairs=bufs.get("sorted"),
                workspace=self.ws)
        bufs.update(ids=ids, w=w, offsets=off, sorted=sp)
        if self.keepquant:
            xq = moe.moe_quantize_act(self.wtype, x, bufs.get("xq_buf"))
            bufs["xq_buf"] = xq.data
        evs = record
        if record:
            # the GEMM kernels record their own start and end (no packets
            # added to the queue), on the stream they run on
            moe.moe_time_next_gemm(evs[0], evs[1])
        if fused:
            act, eo = moe.moe_fused_expert_ffn(x, w_gu, w_d, sp, off, K, w, self.ws_f,
                                               bufs.get("act"), bufs.get("expert_out"))
        elif self.keepquant:
            act = moe.moe_grouped_qgemm_gateup_silu(xq, w_gu, sp, off, K, bufs.get("act"),
                                                    wtype=self.wtype)
            aq = moe.moe_quantize_act(self.wtype, act, bufs.get("aq_buf"))
            bufs["aq_buf"] = aq.data
        else:
            act = moe.moe_grouped_gemm_gateup_silu(x, w_gu, sp, off, K, bufs.get("act"))
        if not fused:
            if record:
                moe.moe_time_next_gemm(evs[2], evs[3])
            if self.keepquant:
                eo = moe.moe_grouped_qgemm_down(aq, w_d, sp, off, w, bufs.get("expert_out"),
                                                wtype=self.wtype)
            else:
                eo = moe.moe_grouped_gemm_down(act, w_d, sp, off, w, bufs.get("expert_out"))
        if record:
            self.ev.append(evs)
        bufs.update(act=act, expert_out=eo)
        if w_gu_s is not None:
            main.wait_stream(self.side)
        out = moe.moe_combine_gate(eo, T, K, None, self.routed_scale, sd, gl, bufs.get("out"))
        bufs["out"] = out

    def new_event(self):
        # recorded once here so that the HIP event exists before a kernel
        # records into it
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.torch.cuda.current_stream())
        return e

    def timed_steps(self, steps, warmup, fused=False, sampler=None):
        """Eager steps: `warmup` untimed, then `steps` timed (wall clock), the
        GEMMs timed by their own events on every TIMING_EVERY-th step."""
        torch = self.torch
        L = len(self.layers)
        self.ev.clear()
        for i in range(max(warmup, L)):
            self.step(False, i, fused)
        pool = [[self.new_event() for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        import contextlib
        with (sampler if sampler is not None else contextlib.nullcontext()):
            t0 = time.perf_counter()
            for i in range(steps):
                self.step(pool[i] if i % TIMING_EVERY == 0 else False, i, fused)
            torch.cuda.synchronize()
            elapsed = time.perf_counter() - t0
        gu = [a.elapsed_time(b) for a, b, _, _ in self.ev]
        dn = [c.elapsed_time(d_) for _, _, c, d_ in self.ev] if not fused else []
        return elapsed, gu, dn

    def graph_steps(self, steps, fused=False):
        """The same steps captured once (one per weight set) and replayed: no
        host launch work between kernels; every buffer already exists, so the
        capture allocates nothing."""
        torch = self.torch
        L = len(self.layers)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(L):
                self.step(False, i, fused)
        reps = max(1, steps // L)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        el = time.perf_counter() - t1
        del g
        return {"steps": reps * L, "ms_per_step": el / (reps * L) * 1e3,
                "tokens_per_s": self.cfg.T * reps * L / el}

    def combine_cold(self, reps=10):
        """The combine alone on the last step's expert_out (and shared term),
        cold: before each launch a 1 GiB read (a reduction over a buffer four
        times the 256 MB last-level cache) evicts what the layer left there;
        the combine records its own start and end."""
        torch, moe, cfg, bufs = self.torch, self.moe, self.cfg, self.bufs
        flush = torch.ones((1 << 28,), dtype=torch.int32, device=self.dev)  # 1 GiB
        sink = torch.empty((reps + 2,), dtype=torch.int64, device=self.dev)
        pool = [[self.new_event() for _ in range(2)] for _ in range(reps)]
        torch.cuda.synchronize()

        def one(i, evs=None):
            torch.sum(flush, dim=0, out=sink[i])
            if evs:
                moe.moe_time_next_gemm(evs[0], evs[1])
            moe.moe_combine_gate(bufs["expert_out"], cfg.T, cfg.K, None, self.routed_scale,
                                 bufs.get("sd"), bufs.get("gl"), bufs["out"])

        for i in range(2):
            one(reps + i)
        for i in range(reps):
            one(i, pool[i])
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 for a, b in pool]
        del flush
        nbytes = combine_bytes(cfg)
        mean = float(np.mean(us))
        return {"us": mean, "us_median": float(np.median(us)), "us_min": float(np.min(us)),
                "bytes": nbytes, "gbs": nbytes / (mean * 1e-6) / 1e9,
                "frac_of_hbm_peak": nbytes / (mean * 1e-6) / 1e9 / HBM_PEAK_GBS,
                "roofline_us": nbytes / (HBM_PEAK_GBS * 1e9) * 1e6,
                "protocol": f"1 GiB read between launches; kernel-recorded events, mean of {reps}"}

    def routing_check(self):
        """The GPU's router logits against float64 dot products (plus the
        f32 bias where the workload has one): the largest error, and the
        tokens whose K-th / (K+1)-th largest logit gap is within twice that
        error (their selection could differ from exact logits). Routing
        parity itself is judged on identical logits; this reports how far
        the GPU's own logits are from exact."""
        torch, cfg = self.torch, self.cfg
        K, E = cfg.K, cfg.E
        if K >= E:
            return None
        xs = self.x.float().cpu().double()
        wr = self.layers[0]["w_r"].float().cpu().double()
        ref = xs @ wr.T
        if self.bias is not None:
            ref = ref + self.bias.cpu().double()[None, :]
        got = self.bufs["logits"].cpu().double()
        err = float((got - ref).abs().max())
        top = torch.topk(got, K + 1, dim=1).values
        gap = top[:, K - 1] - top[:, K]
        ids_gpu = torch.topk(got, K, dim=1).indices.sort(dim=1).values
        ids_ref = torch.topk(ref, K, dim=1).indices.sort(dim=1).values
        return {"logit_max_abs_err": err, "min_kth_gap": float(gap.min()),
                "tokens_with_gap_within_2x_err": int((gap <= 2 * err).sum()),
                "tokens_whose_topk_set_differs_from_f64": int((ids_gpu != ids_ref).any(1).sum()),
                "tokens": cfg.T}


def roofline_of(gu, gu_ms, keepquant):
    """Roofline object of the gate-up GEMM: the bound from its algorithmic
    intensity against the ridge, achieved = algorithmic bytes or flops per
    launch / the kernel's mean duration."""
    mfma_peak = MFMA_I8_PEAK_TOPS if keepquant else MFMA_BF16_PEAK_TFLOPS
    hbm_bound = (gu["flops"] / gu["bytes"]) < (mfma_peak * 1e12) / (HBM_PEAK_GBS * 1e9)
    if hbm_bound:
        achieved = gu["bytes"] / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None}
    else:
        achieved = gu["flops"] / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": mfma_peak,
                "unit": "TOP/s" if keepquant else "TFLOP/s", "frac": achieved / mfma_peak,
                "traffic": None}
        # the attainable figure at this intensity: min(MFMA, HBM x flop/byte)
        attain = min(mfma_peak, HBM_PEAK_GBS * 1e9 * gu["flops"] / gu["bytes"] / 1e12)
        roof["frac_of_attainable"] = achieved / attain
    # the same launch in flop terms, against the dense MFMA peak (the target
    # for the grouped GEMMs at T >= 4096 is stated that way)
    roof["tflops"] = gu["flops"] / (gu_ms * 1e-3) / 1e12
    roof["frac_of_mfma_peak"] = roof["tflops"] / mfma_peak
    roof["flop_per_byte"] = gu["flops"] / gu["bytes"]
    return roof, hbm_bound


def sub_config(moe, torch, dev, workload, steps, warmup, n_layers):
    """A compact result of another workload: layer tokens/s, the gate-up and
    down GEMMs' kernel-recorded times against their rooflines, and the
    combine under the cold-cache protocol."""
    lay = Layer(moe, torch, dev, workload, n_layers, fused=False)
    cfg = lay.cfg
    elapsed, gu_l, dn_l = lay.timed_steps(steps, warmup)
    gu_ms, dn_ms = float(np.mean(gu_l)), float(np.mean(dn_l))
    gu, dn, touched = algorithmic_work(cfg, lay.bufs["offsets"].cpu().numpy())
    roof, _ = roofline_of(gu, gu_ms, lay.keepquant)
    roof["traffic"] = measured_traffic(workload)
    droof, _ = roofline_of(dn, dn_ms, lay.keepquant)
    droof.pop("traffic", None)
    res = {"workload": cfg.name, "steps": steps,
           "tokens_per_s": cfg.T * steps / elapsed, "ms_per_step": elapsed / steps * 1e3,
           "gateup_us": gu_ms * 1e3, "down_us": dn_ms * 1e3,
           "roofline": roof | {"kernel": "grouped gate-up GEMM + SiLU-mul"},
           "down_roofline": droof,
           "combine": lay.combine_cold(),
           "routing_check": lay.routing_check()}
    lay.release()
    del lay
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def _oracle_stages(d, sample_tokens):
    """One pass of the oracle over the first `sample_tokens` tokens, stage by
    stage; returns {stage: seconds}."""
    import oracle
    cfg = d["cfg"]
    T, K, H = sample_tokens, cfg.K, cfg.H
    x = d["x"][:T]
    st = {}
    t = time.perf_counter()
    logits = oracle.router_logits(x, d["w_r"], d.get("router_bias"))
    st["router_logits"] = time.perf_counter() - t
    t = time.perf_counter()
    routed_scale = 1.0
    if cfg.router == "grouped_sigmoid":
        ids, w, off, sp = oracle.route_scored(logits, K, "sigmoid", d["selection_bias"], 8, 4,
                                              "top2", True)
        routed_scale = 2.5
    else:
        ids, w, off, sp = oracle.route(logits, K)
    st["route"] = time.perf_counter() - t
    wtype = cfg.weights
    t = time.perf_counter()
    if wtype != "bf16":
        # keep-quant experts: GGUF weight blocks, quantized activations
        from oracle.keepquant import kq_down, kq_gateup_silu
        act, _ = kq_gateup_silu(x, d["w_gu_kq"], sp, off, K, wtype)
    else:
        act = oracle.gateup_silu(x, d["w_gu"], sp, off, K)
    st["gateup"] = time.perf_counter() - t
    t = time.perf_counter()
    if wtype != "bf16":
        eo, _ = kq_down(act, d["w_d_kq"], sp, off, w.reshape(-1), wtype)
    else:
        eo = oracle.down_proj(act, d["w_d"], sp, off, w)
    st["down"] = time.perf_counter() - t
    sd = gl = None
    if "w_gu_s" in d:
        t = time.perf_counter()
        sd = oracle.shared_expert(x, d["w_gu_s"], d["w_d_s"])
        gl = oracle.gate_logit(x, d["w_g"])
        st["shared"] = time.perf_counter() - t
    t = time.perf_counter()
    oracle.combine_gate(eo, T, K, H, None, routed_scale, sd, gl)
    st["combine"] = time.perf_counter() - t
    return st


def cpu_baseline(d, sample_tokens, single_thread_workloads=(1, 2)):
    """The oracle (as it stands: numpy, float64 GEMMs through the BLAS) on the
    first `sample_tokens` tokens of the workload, stage by stage, with the
    BLAS thread pool set to every CPU this process may run on; then the tiny
    and decode layers whole with one thread."""
    import workloads
    from threadpoolctl import threadpool_info, threadpool_limits
    cpus = len(os.sched_getaffinity(0))
    cfg = d["cfg"]
    with threadpool_limits(limits=cpus):
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        st = _oracle_stages(d, sample_tokens)
    total = sum(st.values())
    single = {}
    with threadpool_limits(limits=1):
        for wl in single_thread_workloads:
            dd = workloads.make_inputs(wl)
            s1 = _oracle_stages(dd, dd["cfg"].T)
            tt = sum(s1.values())
            single[dd["cfg"].name] = {"tokens_per_s": dd["cfg"].T / tt, "seconds": tt,
                                      "stages_s": s1}
            del dd
    return {"value": sample_tokens / total, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"whole layer (router logits, routing, both grouped GEMMs, "
                      f"{'shared expert, ' if cfg.I_s else ''}combine) on the first "
                      f"{sample_tokens} of {cfg.T} tokens of {cfg.name}, numpy with float64 BLAS "
                      f"GEMMs on {threads} threads; {total:.2f} s",
            "stages_s": st, "nproc": os.cpu_count(), "affinity_cpus": cpus,
            "single_thread": single}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the extra timing of the layer with the fused expert FFN")
    ap.add_argument("--layers", type=int, default=2,
                    help="distinct weight sets (layers) the steps cycle through, so that no "
                         "step finds its weights in the 256 MB last-level cache (default 2)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the hipGraph-replay timing of the same steps")
    ap.add_argument("--ep-share", action="store_true",
                    help="also time the GEMMs at each expert-parallel owner's share (the "
                         "same kernels at other shapes: kept out of the default run so that "
                         "a kernel trace of it averages the layer's launches only)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the HBM-read and MFMA ceiling micro-kernels")
    ap.add_argument("--no-sub-configs", action="store_true",
                    help="skip the compact runs of the decode, prefill and 256-expert layers")
    ap.add_argument("--sub-steps", type=int, default=20,
                    help="timed steps of each compact run (default 20)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM byte-counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; the expert-parallel multi-GPU "
                                   "path is designed but not built, so --gpus must be 1"}))
        sys.exit(2)

    import torch

    import mixture_experts_ffn_expert_amd as moe

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        n = 1 << 29                               # 2^29 bf16 = 1 GiB read + 1 GiB written
        a = torch.ones(n, dtype=torch.bfloat16, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": 2 * n, "bytes_written": 2 * n,
                          "launches": 3}))
        return
    moe.load()
    moe.moe_init()
    log(f"workload {args.workload}: inputs and weights")
    lay = Layer(moe, torch, dev, args.workload, args.layers, fused=not args.no_fused)
    cfg, d = lay.cfg, lay.d
    T, H, E, K, I = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I
    keepquant = lay.keepquant

    log(f"{cfg.name}: {args.warmup} warm-up and {args.steps} timed steps")
    sampler = GpuStateSampler(torch, dev)
    idle = sampler.read()
    elapsed, gu_list, dn_list = lay.timed_steps(args.steps, args.warmup, sampler=sampler)
    gpu_state = sampler.summary(idle)
    graph = None if args.no_graph else lay.graph_steps(args.steps)
    gu_ms = float(np.mean(gu_list))
    dn_ms = float(np.mean(dn_list))

    fused_res = None
    if lay.fused_ok:
        # the same steps with the fused expert FFN: eager (the fused kernel
        # timed by its own events), then captured and replayed
        log("fused expert FFN steps")
        f_el, f_list, _ = lay.timed_steps(args.steps, args.warmup, fused=True)
        fused_res = {"ms_per_step": f_el / args.steps * 1e3,
                     "tokens_per_s": T * args.steps / f_el,
                     "ffn_kernel_us": float(np.mean(f_list)) * 1e3,
                     "status": moe.fused_ffn_status(lay.ws_f)}
        if not args.no_graph:
            gf = lay.graph_steps(args.steps, fused=True)
            fused_res["hipgraph_ms_per_step"] = gf["ms_per_step"]
            fused_res["hipgraph_tokens_per_s"] = gf["tokens_per_s"]
            fused_res["status"] = moe.fused_ffn_status(lay.ws_f)
    offsets = lay.bufs["offsets"].cpu().numpy()
    gu, dn, touched = algorithmic_work(cfg, offsets)
    ep = None
    if args.ep_share and not keepquant and E % EP_SHARDS == 0:
        log("expert-parallel owner shares")
        ep = expert_parallel_share(moe, torch, lay.x, lay.layers, lay.bufs["offsets"],
                                   lay.bufs["sorted"], lay.bufs["w"], cfg)
    log("combine (cold cache) and routing check")
    comb = lay.combine_cold()
    rcheck = lay.routing_check()
    lay.release()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    ceilings = None
    if not args.no_ceilings:
        log("ceiling micro-kernels")
        ceilings = measure_ceilings(moe, torch, dev)
    roof, hbm_bound = roofline_of(gu, gu_ms, keepquant)
    roof["traffic"] = measured_traffic(args.workload)
    if ceilings is not None:
        # the same achieved figure against the chip's measured ceiling (the
        # keep-quant kernels' int8 MFMAs have no measured ceiling here)
        if hbm_bound:
            roof["frac_of_measured"] = roof["achieved"] / ceilings["hbm_read_gbs"]
        elif not keepquant:
            roof["frac_of_measured"] = roof["achieved"] / ceilings["mfma_bf16_tflops"]
    # the shader clock the chip ran the timed steps at (its power management
    # lowers it under sustained MFMA load; the datasheet peak assumes 2.4 GHz)
    sclk = (gpu_state or {}).get("sclk_mhz") or {}
    roof["sclk_mhz_median"] = sclk.get("median")
    roof["kernel"] = (f"grouped keep-quant gate-up GEMM + SiLU-mul ({lay.wtype.upper()})"
                      if keepquant else "grouped gate-up GEMM + SiLU-mul")
    roof["algorithmic"] = {"bytes_per_launch": gu["bytes"], "flops_per_launch": gu["flops"],
                           "touched_experts": touched}
    droof, _ = roofline_of(dn, dn_ms, keepquant)
    droof.pop("traffic", None)
    gemm_ms = gu_ms + dn_ms
    gemm_flops = gu["flops"] + dn["flops"]
    gemm_bytes = gu["bytes"] + dn["bytes"]
    ms_per_step = elapsed / args.steps * 1e3
    res = {
        "metric": "MoE-layer tokens/s + grouped-GEMM bf16 TFLOP/s (% MFMA/HBM roofline), 1 GPU",
        "value": T * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (f"{lay.wtype} weights, {'q8_0' if lay.wtype == 'q8_0' else 'q8_k'} activations, "
                  "i8 MFMA") if keepquant else "bf16",
        "data": (f"synthetic (seeded random valid {lay.wtype.upper()} expert blocks, N(0,1/fan_in) "
                 "router weights, of the workload's shapes)" if keepquant else
                 "synthetic (seeded N(0,1/fan_in) bf16 weights of the workload's shapes)"),
        "config": {"workload": cfg.name, "T": T, "H": H, "E": E, "K": K, "I": I,
                   "I_shared": cfg.I_s, "skewed_router": cfg.skew_bias, "router": cfg.router,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "grouped_gemm": {
            "gateup_us": gu_ms * 1e3, "down_us": dn_ms * 1e3,
            "gateup_us_median": float(np.median(gu_list)) * 1e3,
            "gateup_us_min": float(np.min(gu_list)) * 1e3,
            "down_us_median": float(np.median(dn_list)) * 1e3,
            "down_us_min": float(np.min(dn_list)) * 1e3,
            "down_roofline": droof,
            "tflops": gemm_flops / (gemm_ms * 1e-3) / 1e12,
            "tflops_frac_of_mfma_peak": gemm_flops / (gemm_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "algorithmic_gbs": gemm_bytes / (gemm_ms * 1e-3) / 1e9,
            "gbs_frac_of_hbm_peak": gemm_bytes / (gemm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        },
        "combine": comb,
        "routing_check": rcheck,
        "hipgraph": graph,
        "fused_ffn": fused_res,
        "expert_parallel_share": ep,
        "weight_sets": args.layers,
        "measured_ceilings": ceilings,
        "gpu_state": gpu_state,
        "configs": None,
        "cpu_baseline": None,
    }
    if args.workload == 5 and not args.no_sub_configs:
        subs = {}
        for wl in (2, 3, 4):
            log(f"compact run of workload {wl}")
            r = sub_config(moe, torch, dev, wl, args.sub_steps, min(args.warmup, 5), args.layers)
            subs[r["workload"]] = r
        res["configs"] = subs
    if not args.no_cpu_baseline:
        # about 10-30 s of CPU work: all tokens of the small workloads, a
        # prefix of the large ones
        sample = {1: 16, 2: 32, 3: 4096, 4: 512, 5: 8192, 6: 512}.get(args.workload, 32)
        log(f"CPU oracle on {min(sample, T)} tokens, then the tiny and decode layers on one thread")
        res["cpu_baseline"] = cpu_baseline(d, min(sample, T))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
