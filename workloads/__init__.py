"""Seeded synthetic inputs for the BF16 MoE expert-path workloads.

This module is shared by the tests, the benchmark and the oracle's callers. It
only draws random numbers and stores them; it holds none of the MoE method's
arithmetic (no routing, no GEMM, no activation, no combine). Conversion of the
drawn f32 values to bf16 storage is done by torch's CPU cast, a library
routine, so that neither the oracle nor the HIP path lends it code.

Recipe (one numpy ``SeedSequence(seed)``, children spawned in a fixed order):

  child 0  x      [T,H]        ~ N(0,1)
  child 1  W_r    [E,H]        ~ N(0,1/H)
  child 2  W_gu   [E,2I,H]     ~ N(0,1/H)   one grandchild per expert
           (Q4_K workloads: random valid Q4_K blocks of that spread instead)
  child 3  W_d    [E,H,I]      ~ N(0,1/I)   one grandchild per expert (or Q4_K)
  child 4  W_gu_s [2I_s,H]     ~ N(0,1/H)   (shared expert, if I_s > 0)
  child 5  W_d_s  [H,I_s]      ~ N(0,1/I_s)
  child 6  w_g    [H]          ~ N(0,1/H)   (shared-expert gate vector)
  child 7  ranking             permutation of E experts (skewed router only)
  child 8  selection bias [E] ~ N(0, 0.1^2) float32 (grouped sigmoid router only)

N(0, v) names the variance, so the standard deviation is 1/sqrt(fan_in). Each
value is drawn as float32 by PCG64, multiplied by float32(1/sqrt(fan_in)) and
cast to bf16 round-to-nearest-even. Gate rows of W_gu are [0, I) and up rows
[I, 2I). The skewed router adds b_e = 2*ln(1/rank_e), rank_e = 1 + perm[e],
computed in float64 and stored as float32.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int
    H: int
    E: int
    K: int
    I: int
    I_s: int = 0          # shared-expert intermediate size (0: no shared expert)
    skew_bias: bool = False  # router bias 2*ln(1/rank_e)
    # "softmax": ungrouped softmax top-k, renormalised. "grouped_sigmoid":
    # sigmoid scores, a per-expert selection bias, 8 groups of which the 4
    # with the largest top-2 sums stay allowed, renormalised weights and a
    # routed scale of 2.5 in the combine (the DeepSeek-V3 router shape).
    router: str = "softmax"
    # expert weight format: "bf16", or a GGUF block format of the keep-quant
    # path ("q4_k", "q5_k", "q6_k", "q8_0")
    weights: str = "bf16"

    @property
    def P(self) -> int:
        return self.T * self.K


# The five workloads: a tiny layer with a shared expert, a 128-expert top-8
# decode layer and the same layer in prefill, a 256-expert layer with a gated
# shared expert, and a large layer whose router bias makes routing Zipf-skewed.
# A sixth has the 256-expert layer's shapes with the grouped sigmoid router;
# the seventh to tenth are the decode layer with Q4_K, Q5_K, Q6_K and Q8_0
# expert weights (keep-quant path).
CONFIGS = {
    1: MoeConfig("tiny_T16_H64_E8_K2_I32_shared32", 16, 64, 8, 2, 32, I_s=32),
    2: MoeConfig("decode_T32_H2048_E128_K8_I768", 32, 2048, 128, 8, 768),
    3: MoeConfig("prefill_T4096_H2048_E128_K8_I768", 4096, 2048, 128, 8, 768),
    4: MoeConfig("shared_T512_H2048_E256_K8_I512_shared512", 512, 2048, 256, 8, 512, I_s=512),
    5: MoeConfig("skewed_T8192_H4096_E128_K8_I1536", 8192, 4096, 128, 8, 1536, skew_bias=True),
    6: MoeConfig("grouped_T512_H2048_E256_K8_I512_shared512", 512, 2048, 256, 8, 512, I_s=512,
                 router="grouped_sigmoid"),
    7: MoeConfig("keepquant_decode_T32_H2048_E128_K8_I768_q4k", 32, 2048, 128, 8, 768,
                 weights="q4_k"),
    8: MoeConfig("keepquant_decode_T32_H2048_E128_K8_I768_q5k", 32, 2048, 128, 8, 768,
                 weights="q5_k"),
    9: MoeConfig("keepquant_decode_T32_H2048_E128_K8_I768_q6k", 32, 2048, 128, 8, 768,
                 weights="q6_k"),
    10: MoeConfig("keepquant_decode_T32_H2048_E128_K8_I768_q8_0", 32, 2048, 128, 8, 768,
                  weights="q8_0"),
}


def router_args(cfg) -> dict:
    """Router form of a workload, as keyword arguments of the general router
    (score, n_group, topk_group, group_score, renormalize) plus the combine's
    routed_scale; None for the ungrouped softmax router."""
    if config(cfg).router == "softmax":
        return None
    return {"score": "sigmoid", "n_group": 8, "topk_group": 4, "group_score": "top2",
            "renormalize": True, "routed_scale": 2.5}


def config(n_or_cfg) -> MoeConfig:
    return n_or_cfg if isinstance(n_or_cfg, MoeConfig) else CONFIGS[int(n_or_cfg)]


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns via torch's RNE cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.uint16).numpy().copy()


def _normal_bf16(seq: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seq))
    v = g.standard_normal(shape, dtype=np.float32)
    v *= np.float32(std)
    return _to_bf16_bits(v)


def _per_expert_bf16(seq: np.random.SeedSequence, E: int, shape, std: float,
                     threads: int) -> np.ndarray:
    out = np.empty((E,) + tuple(shape), dtype=np.uint16)
    kids = seq.spawn(E)

    def one(e):
        out[e] = _normal_bf16(kids[e], shape, std)

    if threads <= 1 or E == 1:
        for e in range(E):
            one(e)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(E)))
    return out


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_inputs(cfg, seed: int | None = None, *, T: int | None = None,
                threads: int | None = None, experts: bool = True) -> dict:
    """Generate the inputs of one workload.

    ``seed`` defaults to the workload number for numbered configs. ``T``
    overrides the token count (the weights do not depend on T, the tokens are
    the first T rows drawn for that T). ``experts=False`` skips the expert
    weights (every tensor has its own seed child, so the others do not
    change). Returns a dict of numpy arrays; bf16 tensors are uint16 bits.
    """
    cfg = config(cfg)
    if seed is None:
        seed = next((k for k, v in CONFIGS.items() if v == cfg), 0)
    if T is not None:
        cfg = dataclasses.replace(cfg, name=cfg.name + f"_T{T}", T=T)
    threads = _threads() if threads is None else threads
    H, E, I, I_s = cfg.H, cfg.E, cfg.I, cfg.I_s
    kids = np.random.SeedSequence(seed).spawn(9)
    d = {"cfg": cfg, "seed": seed}
    d["x"] = _normal_bf16(kids[0], (cfg.T, H), 1.0)
    d["w_r"] = _normal_bf16(kids[1], (E, H), 1.0 / math.sqrt(H))
    if experts and cfg.weights != "bf16":
        d["w_gu_kq"] = random_kq_blocks(cfg.weights, kids[2], (E, 2 * I), H, 1.0 / math.sqrt(H))
        d["w_d_kq"] = random_kq_blocks(cfg.weights, kids[3], (E, H), I, 1.0 / math.sqrt(I))
    elif experts:
        d["w_gu"] = _per_expert_bf16(kids[2], E, (2 * I, H), 1.0 / math.sqrt(H), threads)
        d["w_d"] = _per_expert_bf16(kids[3], E, (H, I), 1.0 / math.sqrt(I), threads)
    if I_s > 0:
        d["w_gu_s"] = _normal_bf16(kids[4], (2 * I_s, H), 1.0 / math.sqrt(H))
        d["w_d_s"] = _normal_bf16(kids[5], (H, I_s), 1.0 / math.sqrt(I_s))
        d["w_g"] = _normal_bf16(kids[6], (1, H), 1.0 / math.sqrt(H))
    if cfg.skew_bias:
        perm = np.random.Generator(np.random.PCG64(kids[7])).permutation(E)
        rank = 1.0 + perm.astype(np.float64)
        d["router_bias"] = (2.0 * np.log(1.0 / rank)).astype(np.float32)
    if cfg.router == "grouped_sigmoid":
        g = np.random.Generator(np.random.PCG64(kids[8]))
        d["selection_bias"] = g.standard_normal(E, dtype=np.float32) * np.float32(0.1)
    return d


# bytes and values per block of the GGUF weight formats
KQ_FORMATS = {"q4_k": (144, 256), "q5_k": (176, 256), "q6_k": (210, 256), "q8_0": (34, 32)}


def random_kq_blocks(wtype: str, seed, shape, K: int, std: float) -> np.ndarray:
    """Valid random GGUF blocks of format wtype (uint8 [*shape, nb, bytes])
    for weights of roughly the given standard deviation: f16 scale fields
    drawn near std divided by the format's typical code magnitude, random
    scale bytes and random quant bytes. Random bytes and scale values only;
    the format's arithmetic lives elsewhere."""
    nbytes, nval = KQ_FORMATS[wtype]
    g = np.random.Generator(np.random.PCG64(seed))
    full = tuple(shape) + (K // nval,)
    out = np.zeros(full + (nbytes,), np.uint8)

    def f16(v):
        return v.astype(np.float16)[..., None].view(np.uint8)

    def jitter():
        return 0.75 + 0.5 * g.random(full)

    def rnd(n):
        return g.integers(0, 256, size=full + (n,), dtype=np.uint8)

    if wtype in ("q4_k", "q5_k"):
        s = (std / (150.0 if wtype == "q4_k" else 300.0)) * jitter()
        out[..., 0:2] = f16(s)
        out[..., 2:4] = f16(s * jitter())
        out[..., 4:] = rnd(nbytes - 4)          # scales/mins, (qh,) quants
    elif wtype == "q6_k":
        out[..., 0:208] = rnd(208)              # ql, qh, int8 scales
        out[..., 208:210] = f16((std / 1400.0) * jitter())
    else:
        out[..., 0:2] = f16((std / 73.0) * jitter())
        out[..., 2:34] = rnd(32)
    return out


def random_q4k_blocks(seed, shape, K: int, std: float) -> np.ndarray:
    """Valid random GGUF Q4_K blocks (uint8 [*shape, K/256, 144])."""
    return random_kq_blocks("q4_k", seed, shape, K, std)


def random_f32(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """Seeded N(0, scale^2) float32 values (for stage-level test inputs)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    v = g.standard_normal(shape, dtype=np.float32)
    v *= np.float32(scale)
    return v


def random_bf16(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """Seeded N(0, scale^2) values stored as bf16 bit patterns."""
    return _to_bf16_bits(random_f32(seed, shape, scale))
