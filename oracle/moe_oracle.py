"""Plain CPU oracle of the BF16 Mixture-of-Experts expert path.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the CPU
baseline of the benchmark. Shares no code with the HIP library.

Sources (web pages; cited by title and section):

* [Issue 3094] vllm.cpp issue #3094, row "BACKEND-ROCM-BF16-MOE", the row
  statement: the BF16 grouped expert GEMMs (plain, and gate-up with SiLU) and
  the numeric contract they must keep -- (N1) the GEMM result is narrowed to
  bf16 before the activation, (N2) the routing weight is applied before the
  down-projection result is stored, (N3) the final reduction must not apply
  the routing weights a second time.
* [PR 509] vllm.cpp PR #509 "feat(rocm): MoE combine/gate ops --
  SharedExpertGate, MoeCombine, MoeCombineGate": "What changed" (the three
  combine-side formulas), "Honest gaps" (the covered router is the ungrouped
  softmax top-k), the review comment (f32/bf16 arms only, f16 refused by
  name; bit-exact is achievable because each output element is its own
  thread with a single store rounding), the rework commit (bit-exact recipe:
  thread per element, same sequential k order, one store rounding, no FP
  contraction) and the routed_scale commit (one multiply on the finished
  routed sum, before the shared term is added; default 1.0).
* [PR 523] keep-quant grouped expert GEMM, "What changed": the grouped op
  runs over the expert ids of each routed row.
* [Issue 1590] "Qwen3.5/3.6 MoE GGUFs cannot run on discrete ROCm", body:
  kMoeGateUpSwiGLUGrouped, kMoeCombine and kSharedExpertGate are on the same
  MoE forward.

Readings of points the pages leave open are marked READING in the docstrings
and listed in the design doc.

Conventions: bf16 tensors are numpy uint16 bit patterns; f32 arithmetic is
numpy float32 (IEEE round-to-nearest-even, every operation rounded on its own,
no fused multiply-add); dot products accumulate in float64. Shapes: x [T,H];
W_gu [E,2I,H] (gate rows [0,I), up rows [I,2I)); W_d [E,H,I]; the pair index
is p = t*K + k; "sorted order" groups pairs by expert, stable in p.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_from_f32", "f32_from_bf16", "pexp", "sigmoid", "silu",
    "router_logits", "topk_ids", "topk_weights", "route", "group_pairs",
    "tree_sum64", "router_scores", "select_scored", "route_scored",
    "gateup_silu", "down_proj", "shared_expert", "gate_logit",
    "combine_gate", "moe_layer",
]

F32 = np.float32


# ---------------------------------------------------------------------------
# bf16 storage
# ---------------------------------------------------------------------------
def bf16_from_f32(a) -> np.ndarray:
    """IEEE float32 -> bfloat16 bits, round to nearest, ties to even.

    bf16 keeps the top 16 bits of the f32 pattern. Rounding adds 0x7FFF plus
    the lowest kept bit, then truncates, which is round-half-even on the
    dropped 16 bits; the carry walks into the exponent, so the largest finite
    values round to infinity as IEEE requires. A NaN keeps its sign and top
    payload bits and has the quiet bit (0x0040) forced. Subnormals are kept.
    """
    u = np.ascontiguousarray(a, dtype=F32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = np.where(nan, (u >> 16) | 0x0040, r)
    return r.astype(np.uint16)


def f32_from_bf16(b) -> np.ndarray:
    """bfloat16 bits -> float32 (exact: the bits are the f32's top half)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(F32)


# ---------------------------------------------------------------------------
# exp, sigmoid, SiLU
# ---------------------------------------------------------------------------
# READING: the pages ask the gated combine to be bit-exact between devices but
# never name an exp. Library expf differs between host and device, so both
# sides implement one published algorithm: Cody & Waite (1980) argument
# reduction n = rint(x/ln2), r = x - n*ln2 with ln2 split into a 9-bit head
# (so n*head is exact) and an f32 tail, then the degree-7 Taylor polynomial of
# e^r in Horner form, then scaling by 2^n. Every step is one f32 operation
# rounded on its own. Coefficients are the f32 roundings of 1/k!.
_L2E = F32(1.4426950408889634)       # f32(1/ln 2)
_LN2_HI = F32(0.693359375)           # ln 2 to 9 significant bits
_LN2_LO = F32(0.6931471805599453 - 0.693359375)  # f32(ln 2 - head)
_INV_FACT = [F32(1.0 / f) for f in (1, 1, 2, 6, 24, 120, 720, 5040)]
_EXP_HI = F32(88.0)    # above: +inf
_EXP_LO = F32(-87.0)   # below: +0 (keeps every finite result normal)


def pexp(x) -> np.ndarray:
    """e^x in float32 by Cody-Waite reduction and a degree-7 Taylor polynomial.

    Special cases: NaN -> NaN, x > 88 -> +inf, x < -87 -> +0. On [-87, 88]
    every result is a normal float, so the final scaling by 2^n is exact.
    """
    x = np.asarray(x, dtype=F32)
    xs = np.where(np.isnan(x) | (x > _EXP_HI) | (x < _EXP_LO), F32(0), x).astype(F32)
    n = np.rint(xs * _L2E).astype(F32)
    r = (xs - n * _LN2_HI).astype(F32)
    r = (r - n * _LN2_LO).astype(F32)
    p = np.full_like(r, _INV_FACT[7])
    for k in range(6, -1, -1):
        p = (p * r).astype(F32)
        p = (p + _INV_FACT[k]).astype(F32)
    y = np.ldexp(p, n.astype(np.int32)).astype(F32)
    y = np.where(x > _EXP_HI, F32(np.inf), y)
    y = np.where(x < _EXP_LO, F32(0), y)
    y = np.where(np.isnan(x), F32(np.nan), y)
    return y.astype(F32)


def sigmoid(z) -> np.ndarray:
    """sigma(z) = 1 / (1 + e^-z) in f32 (correctly rounded divide)."""
    z = np.asarray(z, dtype=F32)
    d = (F32(1) + pexp(-z)).astype(F32)
    return (F32(1) / d).astype(F32)


def silu(g) -> np.ndarray:
    """SiLU(g) = g / (1 + e^-g) in f32 (READING: this form, one divide)."""
    g = np.asarray(g, dtype=F32)
    d = (F32(1) + pexp(-g)).astype(F32)
    return (g / d).astype(F32)


# ---------------------------------------------------------------------------
# Small dense products
# ---------------------------------------------------------------------------
def _dot_f32(a_bf16, b_bf16) -> np.ndarray:
    """fl32(A @ B^T) for bf16 A [m,k], B [n,k]: f64 accumulation, one f32 rounding.

    bf16*bf16 products are exact in f64, so this is the f32 rounding of the
    exact dot product up to f64 summation error (about k*2^-53 relative).
    """
    a = f32_from_bf16(a_bf16).astype(np.float64)
    b = f32_from_bf16(b_bf16).astype(np.float64)
    return (a @ b.T).astype(F32)


def router_logits(x, w_r, bias=None) -> np.ndarray:
    """Router logits l[t,e] = x[t] . W_r[e], f32; optional f32 bias added after.

    READING: the router itself comes from an earlier PR the pages only name
    ([PR 509] "Row"); logits are f32 and a per-expert bias, when present, is
    one f32 add on the finished logit.
    """
    l = _dot_f32(x, w_r)
    if bias is not None:
        l = (l + np.asarray(bias, dtype=F32)[None, :]).astype(F32)
    return l


def gate_logit(x, w_g) -> np.ndarray:
    """Shared-expert gate logit gl[t] = x[t] . w_g in f32 ([PR 509] What changed)."""
    return _dot_f32(x, np.asarray(w_g).reshape(1, -1))[:, 0]


# ---------------------------------------------------------------------------
# Routing: ungrouped softmax top-k, renormalised ([PR 509] Honest gaps)
# ---------------------------------------------------------------------------
def topk_ids(logits, K: int) -> np.ndarray:
    """The K experts with the largest logits per token, in selection order.

    READING: order by logit descending, ties to the lower expert id; a NaN
    logit ranks as -inf. Softmax is strictly increasing, so this is a top-k of
    the probabilities as well. Selection is K rounds of "pick the largest
    remaining entry", the plainest statement of top-k.
    """
    l = np.asarray(logits, dtype=F32)
    T, E = l.shape
    if not 1 <= K <= E:
        raise ValueError(f"topk_ids: need 1 <= K <= E, got K={K}, E={E}")
    key = np.where(np.isnan(l), F32(-np.inf), l)
    taken = np.zeros((T, E), dtype=bool)
    ids = np.empty((T, K), dtype=np.int32)
    rows = np.arange(T)
    for k in range(K):
        best = np.max(np.where(taken, F32(-np.inf), key), axis=1)
        cand = (~taken) & (key == best[:, None])
        pick = np.argmax(cand, axis=1)  # first (lowest id) candidate
        ids[:, k] = pick
        taken[rows, pick] = True
    return ids


def topk_weights(logits, ids) -> np.ndarray:
    """Renormalised softmax weights of the selected experts, f32.

    READING: softmax over all E followed by renormalisation over the chosen K
    equals e^(l_k - m) / sum_j e^(l_j - m) over the chosen set, m the top
    logit; that cancelled form is computed: the f32 difference first, then
    pexp, then a sequential f32 sum in selection order, then one divide.
    NaN logits are used as -inf, as in the selection.
    """
    l = np.asarray(logits, dtype=F32)
    key = np.where(np.isnan(l), F32(-np.inf), l)
    sel = np.take_along_axis(key, np.asarray(ids, dtype=np.int64), axis=1).astype(F32)
    m = sel[:, :1]
    with np.errstate(invalid="ignore"):
        d = (sel - m).astype(F32)
    e = pexp(d)
    S = e[:, 0].copy()
    for k in range(1, e.shape[1]):
        S = (S + e[:, k]).astype(F32)
    with np.errstate(invalid="ignore", divide="ignore"):
        return (e / S[:, None]).astype(F32)


def group_pairs(ids, E: int):
    """Group the routed pairs by expert: counts, offsets and a stable order.

    [Issue 3094]/[PR 523]: the grouped expert GEMMs run over rows grouped per
    expert. Pair p = t*K + k goes to expert ids_flat[p]; offsets[e] is the
    number of pairs of experts below e; sorted_pairs lists, for each expert in
    turn, its pairs in increasing p (READING: stable order). A counting sort.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("group_pairs: expert id out of range")
    cnt = np.zeros(E, dtype=np.int64)
    for e in flat:
        cnt[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + cnt[e]
    cursor = offsets[:-1].copy()
    sorted_pairs = np.empty(flat.size, dtype=np.int64)
    for p, e in enumerate(flat):
        sorted_pairs[cursor[e]] = p
        cursor[e] += 1
    return offsets.astype(np.int32), sorted_pairs.astype(np.int32)


def route(logits, K: int):
    """Top-k ids, renormalised weights, expert offsets and sorted pairs."""
    ids = topk_ids(logits, K)
    w = topk_weights(logits, ids)
    offsets, sorted_pairs = group_pairs(ids, np.asarray(logits).shape[1])
    return ids, w, offsets, sorted_pairs


# ---------------------------------------------------------------------------
# Routing: sigmoid, biased and group-limited router forms. [Issue 3094] row
# statement and [PR 509] Honest gaps name them only as the router gaps that
# remain (the DeepSeek-V2 / Dots3 grouped and sigmoid forms, the grouped /
# bias / noaux_tc forms). READING: their arithmetic is taken from the
# published DeepSeek-V2 and DeepSeek-V3 technical reports -- affinity scores
# by softmax or sigmoid; an optional per-expert bias that steers selection
# only; selection limited to the top groups of consecutive experts, a group
# scored by its best expert (V2) or by its two best experts summed (V3);
# gate weights from the unbiased scores, optionally renormalised over the
# chosen experts.
# ---------------------------------------------------------------------------
def tree_sum64(z) -> np.ndarray:
    """f32 sum over the last axis in the order of a 64-lane butterfly.

    READING (the order a full softmax sums in): element e goes to lane
    e mod 64, each lane adds its elements in increasing e (a lane with none
    holds +0), then for m = 32, 16, 8, 4, 2, 1 every lane l adds lane l xor m;
    lane 0's value is the sum. Each addition is one rounded f32 add.
    """
    z = np.asarray(z, dtype=F32)
    T, E = z.shape
    p = np.zeros((T, 64), dtype=F32)
    for lane in range(min(64, E)):
        acc = z[:, lane].copy()
        for e in range(lane + 64, E, 64):
            acc = (acc + z[:, e]).astype(F32)
        p[:, lane] = acc
    partner = np.arange(64)
    for m in (32, 16, 8, 4, 2, 1):
        p = (p + p[:, partner ^ m]).astype(F32)
    return p[:, 0].copy()


def router_scores(logits, score: str) -> np.ndarray:
    """Affinity scores s[t,e] of every expert, f32.

    sigmoid: s = 1 / (1 + e^-l). softmax (over all E): m = max_e l,
    z = pexp(l - m), S = tree_sum64(z), s = z / S (one correctly rounded
    divide). A NaN logit is used as -inf, as in the selection.
    """
    l = np.asarray(logits, dtype=F32)
    l = np.where(np.isnan(l), F32(-np.inf), l).astype(F32)
    if score == "sigmoid":
        return sigmoid(l)
    if score != "softmax":
        raise ValueError(f"router_scores: unknown score function {score!r}")
    m = np.max(l, axis=1, keepdims=True)
    with np.errstate(invalid="ignore"):
        z = pexp((l - m).astype(F32))
    S = tree_sum64(z)
    with np.errstate(invalid="ignore", divide="ignore"):
        return (z / S[:, None]).astype(F32)


def _rounds_of_max(val, allowed, n: int) -> np.ndarray:
    """n rounds of "take the largest remaining allowed entry, ties to the
    lower index" over the last axis; returns the picked indices in order."""
    T = val.shape[0]
    taken = np.zeros(val.shape, dtype=bool)
    out = np.empty((T, n), dtype=np.int64)
    rows = np.arange(T)
    for k in range(n):
        live = allowed & ~taken
        best = np.max(np.where(live, val, F32(-np.inf)), axis=1)
        pick = np.argmax(live & (val == best[:, None]), axis=1)
        out[:, k] = pick
        taken[rows, pick] = True
    return out


def select_scored(scores, K: int, bias=None, n_group: int = 1, topk_group: int = 1,
                  group_score: str = "max") -> np.ndarray:
    """Expert ids [T, K] chosen from the scores, in selection order.

    Selection value c = s (+ bias[e], one f32 add when a bias is given); NaN
    ranks as -inf. With n_group > 1 the experts form n_group groups of
    E / n_group consecutive ids; a group's score is its largest c ("max") or
    the f32 sum of its two largest c ("top2"; a NaN sum ranks as -inf); the
    topk_group best groups (ties to the lower group) stay allowed. Then K
    rounds pick the largest allowed c, ties to the lower id.
    """
    s = np.asarray(scores, dtype=F32)
    T, E = s.shape
    c = s if bias is None else (s + np.asarray(bias, dtype=F32)[None, :]).astype(F32)
    c = np.where(np.isnan(c), F32(-np.inf), c).astype(F32)
    allowed = np.ones((T, E), dtype=bool)
    if n_group > 1:
        if E % n_group or not 1 <= topk_group <= n_group:
            raise ValueError("select_scored: bad group shape")
        gs = E // n_group
        cg = c.reshape(T, n_group, gs)
        if group_score == "max":
            g = np.max(cg, axis=2)
        elif group_score == "top2":
            srt = -np.sort(-cg, axis=2)
            g = srt[:, :, 0] if gs == 1 else (srt[:, :, 0] + srt[:, :, 1]).astype(F32)
        else:
            raise ValueError(f"select_scored: unknown group score {group_score!r}")
        g = np.where(np.isnan(g), F32(-np.inf), g).astype(F32)
        groups = _rounds_of_max(g, np.ones(g.shape, dtype=bool), topk_group)
        gmask = np.zeros((T, n_group), dtype=bool)
        np.put_along_axis(gmask, groups, True, axis=1)
        allowed = np.repeat(gmask, gs, axis=1)
        if topk_group * gs < K:
            raise ValueError("select_scored: fewer allowed experts than K")
    return _rounds_of_max(c, allowed, K).astype(np.int32)


def route_scored(logits, K: int, score: str = "softmax", bias=None, n_group: int = 1,
                 topk_group: int = 1, group_score: str = "max", renormalize: bool = True):
    """Ids, gate weights, expert offsets and sorted pairs of the general router.

    Weights are the unbiased scores of the chosen experts, w_k = s[e_k]; with
    renormalize, w_k = s[e_k] / (((s[e_0] + s[e_1]) + ...) + s[e_{K-1}]).
    """
    s = router_scores(logits, score)
    ids = select_scored(s, K, bias, n_group, topk_group, group_score)
    w = np.take_along_axis(s, ids.astype(np.int64), axis=1).astype(F32)
    if renormalize:
        S = w[:, 0].copy()
        for k in range(1, K):
            S = (S + w[:, k]).astype(F32)
        with np.errstate(invalid="ignore", divide="ignore"):
            w = (w / S[:, None]).astype(F32)
    offsets, sorted_pairs = group_pairs(ids, s.shape[1])
    return ids, w, offsets, sorted_pairs


# ---------------------------------------------------------------------------
# Grouped expert GEMMs ([Issue 3094] row statement)
# ---------------------------------------------------------------------------
def gateup_silu(x, w_gu, sorted_pairs, offsets, K: int) -> np.ndarray:
    """Grouped gate-up GEMM with SiLU-mul; output act [P, I] in sorted order.

    For sorted row q of expert e (pair p = sorted_pairs[q], token t = p // K):
    gu = fl32(x[t] . W_gu[e]^T) over all 2I rows, narrowed to bf16 (N1), then
    act[q,i] = bf16( silu(g_i) * u_i ) with g = gu[:I], u = gu[I:] read back
    as f32 (READING: one rounding after the product). With sorted_pairs None
    the rows are the tokens themselves (E = 1, K = 1: the shared expert).
    """
    E, twoI, H = w_gu.shape
    I = twoI // 2
    if sorted_pairs is None:
        rows_tok = np.arange(x.shape[0])
        offsets = np.array([0, x.shape[0]])
    else:
        rows_tok = np.asarray(sorted_pairs, dtype=np.int64) // K
    P = rows_tok.size
    act = np.zeros((P, I), dtype=np.uint16)
    for e in range(E):
        q0, q1 = int(offsets[e]), int(offsets[e + 1])
        if q0 == q1:
            continue
        acc = _dot_f32(x[rows_tok[q0:q1]], w_gu[e])           # [m, 2I] f32
        gu = f32_from_bf16(bf16_from_f32(acc))                 # N1
        g, u = gu[:, :I], gu[:, I:]
        act[q0:q1] = bf16_from_f32((silu(g) * u).astype(F32))
    return act


def down_proj(act, w_d, sorted_pairs, offsets, pair_w=None) -> np.ndarray:
    """Grouped down-projection; output [P, H] in pair order.

    y = fl32(act[q] . W_d[e]^T); with routing weights the f32 accumulator is
    multiplied by pair_w[p] before the single bf16 rounding of the store (N2,
    READING: on the accumulator). Row q is stored at pair row p =
    sorted_pairs[q], so [P, H] is also [T, K, H]. Without sorted_pairs the
    rows stay in place (E = 1, the shared expert).
    """
    E, H, I = w_d.shape
    P = act.shape[0]
    if sorted_pairs is None:
        dest = np.arange(P)
        offsets = np.array([0, P])
    else:
        dest = np.asarray(sorted_pairs, dtype=np.int64)
    out = np.zeros((P, H), dtype=np.uint16)
    for e in range(E):
        q0, q1 = int(offsets[e]), int(offsets[e + 1])
        if q0 == q1:
            continue
        acc = _dot_f32(act[q0:q1], w_d[e])                     # [m, H] f32
        if pair_w is not None:
            w = np.asarray(pair_w, dtype=F32).reshape(-1)[dest[q0:q1]]
            acc = (acc * w[:, None]).astype(F32)               # N2
        out[dest[q0:q1]] = bf16_from_f32(acc)
    return out


def shared_expert(x, w_gu_s, w_d_s) -> np.ndarray:
    """Shared expert: gate-up + SiLU-mul and down with E = 1, no weight."""
    act = gateup_silu(x, w_gu_s[None], None, None, 1)
    return down_proj(act, w_d_s[None], None, None, None)


# ---------------------------------------------------------------------------
# Combine ([PR 509] What changed, rework and routed_scale commits)
# ---------------------------------------------------------------------------
def combine_gate(expert_out, T: int, K: int, H: int, topk_w=None,
                 routed_scale: float = 1.0, shared=None, gate_logit_=None,
                 eo_bf16: bool = True, sh_bf16: bool = True,
                 out_bf16: bool = True) -> np.ndarray:
    """Weighted top-k sum, routed scale, optional (gated) shared term.

    For each (t, h), in f32 with every operation rounded on its own:
      acc = +0; for k in 0..K-1: v = expert_out[t,k,h]; (v = w[t,k]*v if
      weighted); acc = acc + v.  acc = acc * routed_scale (always).
      With a shared term s = shared[t,h]: gated -> s = f32(bf16(sigma(gl[t])*s))
      (the shared term is rounded through bf16), then acc = acc + s.
      Output: bf16(acc) or acc.
    topk_w None means the weights were already applied (the layer path, N3).
    READING: the accumulator starts at +0.
    """
    eo = np.asarray(expert_out)
    eo = f32_from_bf16(eo) if eo_bf16 else eo.astype(F32)
    eo = eo.reshape(T, K, H)
    acc = np.zeros((T, H), dtype=F32)
    for k in range(K):
        v = eo[:, k, :]
        if topk_w is not None:
            v = (np.asarray(topk_w, dtype=F32).reshape(T, K)[:, k:k + 1] * v).astype(F32)
        acc = (acc + v).astype(F32)
    acc = (acc * F32(routed_scale)).astype(F32)
    if shared is not None:
        s = np.asarray(shared)
        s = (f32_from_bf16(s) if sh_bf16 else s.astype(F32)).reshape(T, H)
        if gate_logit_ is not None:
            sg = sigmoid(np.asarray(gate_logit_, dtype=F32).reshape(T, 1))
            s = f32_from_bf16(bf16_from_f32((sg * s).astype(F32)))
        acc = (acc + s).astype(F32)
    return bf16_from_f32(acc) if out_bf16 else acc


# ---------------------------------------------------------------------------
# The whole layer
# ---------------------------------------------------------------------------
def moe_layer(inp: dict, logits=None, keep: bool = False) -> dict:
    """One MoE layer on a workload dict (see ``workloads.make_inputs``).

    logits defaults to ``router_logits(x, W_r, bias)``; pass the f32 logits to
    route on a given array. The routed outputs carry their weight from the
    down-projection, so the combine runs unweighted (N3) with routed_scale 1
    (2.5 with the grouped sigmoid router), plus the sigmoid-gated shared
    expert when the workload has one.
    """
    cfg = inp["cfg"]
    T, K, H, E = cfg.T, cfg.K, cfg.H, cfg.E
    x = inp["x"]
    if logits is None:
        logits = router_logits(x, inp["w_r"], inp.get("router_bias"))
    routed_scale = 1.0
    if getattr(cfg, "router", "softmax") == "grouped_sigmoid":
        # sigmoid scores, selection bias, 8 groups keep 4 by top-2 sums,
        # renormalised, routed scale 2.5 (see route_scored)
        ids, w, offsets, sorted_pairs = route_scored(logits, K, "sigmoid",
                                                     inp["selection_bias"], 8, 4, "top2", True)
        routed_scale = 2.5
    else:
        ids, w, offsets, sorted_pairs = route(logits, K)
    wtype = getattr(cfg, "weights", "bf16")
    if wtype != "bf16":
        # keep-quant experts (GGUF weight blocks, quantized activations; see
        # keepquant.py)
        from .keepquant import kq_down, kq_gateup_silu
        act, _ = kq_gateup_silu(x, inp["w_gu_kq"], sorted_pairs, offsets, K, wtype)
        eo, _ = kq_down(act, inp["w_d_kq"], sorted_pairs, offsets, w.reshape(-1), wtype)
    else:
        act = gateup_silu(x, inp["w_gu"], sorted_pairs, offsets, K)
        eo = down_proj(act, inp["w_d"], sorted_pairs, offsets, w)
    sd = gl = None
    if "w_gu_s" in inp:
        sd = shared_expert(x, inp["w_gu_s"], inp["w_d_s"])
        gl = gate_logit(x, inp["w_g"])
    out = combine_gate(eo, T, K, H, None, routed_scale, sd, gl)
    res = {"logits": logits, "ids": ids, "w": w, "offsets": offsets,
           "sorted_pairs": sorted_pairs, "out": out}
    if keep:
        res.update(act=act, expert_out=eo, sd=sd, gl=gl)
    return res
