"""Plain CPU oracle of the keep-quant grouped expert GEMM -- TEST
INFRASTRUCTURE ONLY (imported by tests, the smoke check and the benchmark's
CPU baseline; shares no code with the HIP library).

Source: [PR 523] (keep-quant grouped expert GEMM, "What changed"): expert
weights stay in their GGUF quantized block formats (Q8_0 / Q4_K / Q5_K /
Q6_K); activations are quantized on the fly (Q8_0 / Q8_K quantizers); the dot
products run over (super-)blocks with an integer core (DotQ8_0, DotQ4K,
DotQ5K, DotQ6K); "Evidence": the grouped case is checked against a CPU
keep-quant reference, NMSE <= 5e-4.

READING: the block formats are the published GGUF (ggml) ones; K-quant
weights pair with Q8_K activations, Q8_0 weights with Q8_0 activations.
* Q4_K, 144 bytes per super-block of 256 weights: f16 d, f16 dmin, 12 bytes
  of packed 6-bit sub-block scales and mins (8 sub-blocks of 32), 128 bytes of
  4-bit quants (byte b of 32-byte group i holds value b of sub-block 2i in its
  low nibble and value b of sub-block 2i+1 in its high nibble). Weight value
  w = d * sc_j * q - dmin * m_j.
* Q5_K, 176 bytes: f16 d, f16 dmin, the same 12 scale/min bytes, 32 bytes of
  high bits qh, 128 bytes of low nibbles as in Q4_K. Value b of sub-block 2i
  (2i+1) adds 16 * bit 2i (2i+1) of qh[b]; q in 0..31.
* Q6_K, 210 bytes: 128 bytes of low nibbles ql, 64 bytes of 2-bit high parts
  qh, 16 int8 scales (sub-blocks of 16), f16 d. For half h and l < 32, the
  values 128h + 32c + l (c = 0..3) take the low (c = 0, 1) or high (c = 2, 3)
  nibble of ql[64h + 32(c % 2) + l] and bits 2c, 2c+1 of qh[32h + l] as bits
  4-5; q6 = that 6-bit value - 32; w = d * sc_{v/16} * q6.
* Q8_0, 34 bytes per block of 32: f16 d, 32 int8 quants; w = d * q.
* Q8_K activations, per 256: f32 d, 256 int8 quants, sums of 16-element
  groups. The quantizer takes the entry of largest magnitude (the first one)
  as `max`, iscale = -127 / max, q = min(127, round-half-even(iscale * x)),
  d = 1 / iscale (all f32); an all-zero block gives d = 0, q = 0.
* Q8_0 activations, per 32: amax = max |x|, d = amax / 127, id = 1/d (0 when
  d = 0), q = round-half-away-from-zero(x * id) (all f32), d stored as f16.
Dot products, per (super-)block:
  Q4_K, Q5_K: d_w d_x sum_j sc_j (sum_{l in j} q_l q8_l) - dmin_w d_x sum_j m_j bsum_j
  Q6_K:       d_w d_x sum_{j<16} sc_j (sum_{l in j} q6_l q8_l)
  Q8_0:       d_w d_x sum_l q_l q8_l          (d_x the stored f16 value)
each equal to the dot product of the dequantized vectors. The oracle sums
the terms exactly (every product is split so that it is exact in f64, then
math.fsum) and rounds the sum to f32.
"""
from __future__ import annotations

import math

import numpy as np

from .moe_oracle import F32, bf16_from_f32, f32_from_bf16, silu

__all__ = ["Q4K_BLOCK", "KQ_BLOCK", "KQ_VALUES", "q4k_scale_min", "q4k_unpack",
           "q4k_dequant", "q5k_unpack", "q5k_dequant", "q6k_unpack", "q6k_dequant",
           "q8_0_unpack", "q8_0_dequant", "kq_dequant", "quantize_q8k", "q8k_dequant",
           "quantize_q8_0", "q8_0_act_dequant", "quantize_act", "act_dequant",
           "qdot_q4k_q8k", "qdot", "kq_gateup_silu", "kq_down"]

Q4K_BLOCK = 144   # bytes per super-block of 256 weights
QK = 256
# bytes and values per block of each weight format
KQ_BLOCK = {"q4_k": 144, "q5_k": 176, "q6_k": 210, "q8_0": 34}
KQ_VALUES = {"q4_k": 256, "q5_k": 256, "q6_k": 256, "q8_0": 32}


def q4k_scale_min(scales12: np.ndarray):
    """The 8 six-bit scales and 8 six-bit mins packed in 12 bytes [..., 12].

    Sub-blocks 0-3: scale = low 6 bits of byte j, min = low 6 bits of byte
    j+4. Sub-blocks 4-7: low 4 bits from byte j+4 (scale: low nibble, min: high
    nibble), top 2 bits from the top 2 bits of byte j-4 (scale) / byte j (min).
    """
    s = scales12.astype(np.int32)
    sc = np.empty(s.shape[:-1] + (8,), np.int32)
    mn = np.empty(s.shape[:-1] + (8,), np.int32)
    for j in range(4):
        sc[..., j] = s[..., j] & 63
        mn[..., j] = s[..., j + 4] & 63
    for j in range(4, 8):
        sc[..., j] = (s[..., j + 4] & 0xF) | ((s[..., j - 4] >> 6) << 4)
        mn[..., j] = (s[..., j + 4] >> 4) | ((s[..., j] >> 6) << 4)
    return sc, mn


def q4k_unpack(blocks: np.ndarray):
    """blocks uint8 [..., 144] -> d, dmin (f32), sc, mn [..., 8], q [..., 256]."""
    b = np.ascontiguousarray(blocks)
    d = b[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float32)
    dmin = b[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float32)
    sc, mn = q4k_scale_min(b[..., 4:16])
    qs = b[..., 16:144].astype(np.int32).reshape(b.shape[:-1] + (4, 32))
    q = np.empty(b.shape[:-1] + (8, 32), np.int32)
    q[..., 0::2, :] = qs & 0xF
    q[..., 1::2, :] = qs >> 4
    return d, dmin, sc, mn, q.reshape(b.shape[:-1] + (256,))


def q4k_dequant(blocks: np.ndarray) -> np.ndarray:
    """Q4_K rows [..., nsb, 144] -> float64 weights [..., nsb*256] (exact)."""
    d, dmin, sc, mn, q = q4k_unpack(blocks)
    d = d.astype(np.float64)[..., None]
    dmin = dmin.astype(np.float64)[..., None]
    scv = np.repeat(sc, 32, axis=-1).astype(np.float64)
    mnv = np.repeat(mn, 32, axis=-1).astype(np.float64)
    w = d * scv * q - dmin * mnv
    return w.reshape(w.shape[:-2] + (-1,))


def _f16_at(b: np.ndarray, off: int) -> np.ndarray:
    return b[..., off:off + 2].copy().view(np.float16)[..., 0].astype(np.float32)


def q5k_unpack(blocks: np.ndarray):
    """blocks uint8 [..., 176] -> d, dmin (f32), sc, mn [..., 8], q [..., 256]
    with q in 0..31 (low nibble as in Q4_K plus 16 * the qh bit)."""
    b = np.ascontiguousarray(blocks)
    d, dmin = _f16_at(b, 0), _f16_at(b, 2)
    sc, mn = q4k_scale_min(b[..., 4:16])
    qh = b[..., 16:48].astype(np.int32)                   # [..., 32]
    qs = b[..., 48:176].astype(np.int32).reshape(b.shape[:-1] + (4, 32))
    q = np.empty(b.shape[:-1] + (8, 32), np.int32)
    for i in range(4):
        q[..., 2 * i, :] = (qs[..., i, :] & 0xF) + 16 * ((qh >> (2 * i)) & 1)
        q[..., 2 * i + 1, :] = (qs[..., i, :] >> 4) + 16 * ((qh >> (2 * i + 1)) & 1)
    return d, dmin, sc, mn, q.reshape(b.shape[:-1] + (256,))


def q5k_dequant(blocks: np.ndarray) -> np.ndarray:
    """Q5_K rows [..., nsb, 176] -> float64 weights [..., nsb*256]."""
    d, dmin, sc, mn, q = q5k_unpack(blocks)
    w = (d.astype(np.float64)[..., None] * np.repeat(sc, 32, axis=-1) * q
         - dmin.astype(np.float64)[..., None] * np.repeat(mn, 32, axis=-1))
    return w.reshape(w.shape[:-2] + (-1,))


def q6k_unpack(blocks: np.ndarray):
    """blocks uint8 [..., 210] -> d (f32), sc int [..., 16] (signed), q6
    [..., 256] in -32..31."""
    b = np.ascontiguousarray(blocks)
    ql = b[..., 0:128].astype(np.int32)
    qh = b[..., 128:192].astype(np.int32)
    sc = b[..., 192:208].view(np.int8).astype(np.int32)
    d = _f16_at(b, 208)
    q = np.empty(b.shape[:-1] + (256,), np.int32)
    for h in range(2):
        for c in range(4):
            low = ql[..., 64 * h + 32 * (c % 2):64 * h + 32 * (c % 2) + 32]
            nib = (low & 0xF) if c < 2 else (low >> 4)
            hi2 = (qh[..., 32 * h:32 * h + 32] >> (2 * c)) & 3
            q[..., 128 * h + 32 * c:128 * h + 32 * c + 32] = (nib | (hi2 << 4)) - 32
    return d, sc, q


def q6k_dequant(blocks: np.ndarray) -> np.ndarray:
    """Q6_K rows [..., nsb, 210] -> float64 weights [..., nsb*256]."""
    d, sc, q = q6k_unpack(blocks)
    w = d.astype(np.float64)[..., None] * np.repeat(sc, 16, axis=-1) * q
    return w.reshape(w.shape[:-2] + (-1,))


def q8_0_unpack(blocks: np.ndarray):
    """blocks uint8 [..., 34] -> d (f32) [...], q int [..., 32]."""
    b = np.ascontiguousarray(blocks)
    return _f16_at(b, 0), b[..., 2:34].view(np.int8).astype(np.int32)


def q8_0_dequant(blocks: np.ndarray) -> np.ndarray:
    """Q8_0 rows [..., nb, 34] -> float64 weights [..., nb*32] (exact)."""
    d, q = q8_0_unpack(blocks)
    w = d.astype(np.float64)[..., None] * q
    return w.reshape(w.shape[:-2] + (-1,))


def kq_dequant(wtype: str, blocks: np.ndarray) -> np.ndarray:
    return {"q4_k": q4k_dequant, "q5_k": q5k_dequant, "q6_k": q6k_dequant,
            "q8_0": q8_0_dequant}[wtype](blocks)


def _round_half_even_f32(v: np.ndarray) -> np.ndarray:
    return np.rint(v.astype(F32)).astype(np.int32)   # numpy rint: round half to even


def quantize_q8k(x) -> tuple:
    """Q8_K quantization of f32 rows [R, K] (K % 256 == 0): returns qs int8
    [R, K], d f32 [R, K/256], bsums int32 [R, K/16]."""
    x = np.asarray(x, dtype=F32)
    R, K = x.shape
    nsb = K // QK
    xb = x.reshape(R, nsb, QK)
    ax = np.abs(xb)
    first = np.argmax(ax == ax.max(axis=2, keepdims=True), axis=2)       # first largest
    mx = np.take_along_axis(xb, first[..., None], axis=2)[..., 0].astype(F32)
    amax = np.take_along_axis(ax, first[..., None], axis=2)[..., 0]
    with np.errstate(divide="ignore", invalid="ignore"):
        iscale = (F32(-127.0) / mx).astype(F32)
        q = _round_half_even_f32((iscale[..., None] * xb).astype(F32))
        d = (F32(1.0) / iscale).astype(F32)
    q = np.minimum(q, 127)
    zero = amax == 0
    q = np.where(zero[..., None], 0, q)
    d = np.where(zero, F32(0.0), d).astype(F32)
    qs = q.reshape(R, K).astype(np.int8)
    bsums = q.reshape(R, K // 16, 16).sum(axis=2).astype(np.int32)
    return qs, d, bsums


def q8k_dequant(qs, d) -> np.ndarray:
    R, K = qs.shape
    return (qs.reshape(R, K // QK, QK).astype(np.float64) *
            d.astype(np.float64)[..., None]).reshape(R, K)


def quantize_q8_0(x) -> tuple:
    """Q8_0 quantization of f32 rows [R, K] (K % 32 == 0): returns qs int8
    [R, K] and the stored scales as float16 [R, K/32]."""
    x = np.asarray(x, dtype=F32)
    R, K = x.shape
    xb = x.reshape(R, K // 32, 32)
    amax = np.abs(xb).max(axis=2)
    d = (amax / F32(127.0)).astype(F32)
    with np.errstate(divide="ignore"):
        idv = np.where(d != 0, F32(1.0) / d, F32(0.0)).astype(F32)
    v = (xb * idv[..., None]).astype(F32).astype(np.float64)
    q = np.sign(v) * np.floor(np.abs(v) + 0.5)           # half away from zero, exact in f64
    return q.reshape(R, K).astype(np.int8), d.astype(np.float16)


def q8_0_act_dequant(qs, d16) -> np.ndarray:
    R, K = qs.shape
    return (qs.reshape(R, K // 32, 32).astype(np.float64) *
            d16.astype(np.float64)[..., None]).reshape(R, K)


def quantize_act(wtype: str, x):
    """The activation quantizer that pairs with a weight format."""
    return quantize_q8_0(x) if wtype == "q8_0" else quantize_q8k(x)


def act_dequant(wtype: str, xq) -> np.ndarray:
    return q8_0_act_dequant(xq[0], xq[1]) if wtype == "q8_0" else q8k_dequant(xq[0], xq[1])


def _split14(v: np.ndarray):
    """Integer array -> (hi, lo) with v = hi * 2^14 + lo, 0 <= lo < 2^14."""
    v = v.astype(np.int64)
    lo = v & ((1 << 14) - 1)
    return (v - lo) >> 14, lo


def _exact_terms(coef: np.ndarray, ints: np.ndarray) -> list:
    """Terms whose exact sum is coef * ints, each exact in f64: coef holds
    products of an f16 and an f32 value (at most 35 significant bits) and
    |ints| < 2^38, so both partial products fit in 53 bits."""
    hi, lo = _split14(ints)
    return [coef * hi.astype(np.float64) * 16384.0, coef * lo.astype(np.float64)]


def _fsum_rows(terms: list) -> tuple:
    """terms: arrays [R, N, S] -> (f32 [R, N] of the exact sums, magnitude)."""
    allt = np.concatenate(terms, axis=2)
    R, N = allt.shape[:2]
    out = np.empty((R, N), np.float64)
    for r in range(R):
        for n in range(N):
            out[r, n] = math.fsum(allt[r, n])
    return out.astype(F32), np.abs(allt).sum(axis=2)


def qdot(wtype: str, xq, wblocks) -> tuple:
    """out[r, n] = fl32 of the exact keep-quant dot product of activation row
    r (the quantizer output paired with wtype) with weight row n (blocks
    [N, nb, KQ_BLOCK[wtype]]), and the sum of the magnitudes of its terms."""
    N = wblocks.shape[0]
    if wtype == "q8_0":
        qs, d16 = xq
        R, K = qs.shape
        nb = K // 32
        dw, qw = q8_0_unpack(wblocks)                    # [N, nb], [N, nb, 32]
        dots = np.einsum("rbl,nbl->rnb", qs.reshape(R, nb, 32).astype(np.int64),
                         qw.astype(np.int64))
        coef = d16.astype(np.float64)[:, None, :] * dw.astype(np.float64)[None, :, :]
        return _fsum_rows(_exact_terms(coef, dots))
    qs, dx, bs = xq
    R, K = qs.shape
    nsb = K // QK
    q8 = qs.reshape(R, nsb, QK).astype(np.int64)
    if wtype == "q6_k":
        d, sc, q6 = q6k_unpack(wblocks)
        dots = np.einsum("rsjl,nsjl->rnsj", q8.reshape(R, nsb, 16, 16),
                         q6.reshape(N, nsb, 16, 16).astype(np.int64))
        sumi = np.einsum("rnsj,nsj->rns", dots, sc.astype(np.int64))
        coef = d.astype(np.float64)[None, :, :] * dx.astype(np.float64)[:, None, :]
        return _fsum_rows(_exact_terms(coef, sumi))
    d, dmin, sc, mn, q = (q4k_unpack if wtype == "q4_k" else q5k_unpack)(wblocks)
    dots = np.einsum("rsjl,nsjl->rnsj", q8.reshape(R, nsb, 8, 32),
                     q.reshape(N, nsb, 8, 32).astype(np.int64))
    sumi = np.einsum("rnsj,nsj->rns", dots, sc.astype(np.int64))
    bsj = bs.reshape(R, nsb, 8, 2).sum(axis=3).astype(np.int64)   # sums of 32
    summ = np.einsum("rsj,nsj->rns", bsj, mn.astype(np.int64))
    dall = d.astype(np.float64)[None, :, :] * dx.astype(np.float64)[:, None, :]
    dmn = dmin.astype(np.float64)[None, :, :] * dx.astype(np.float64)[:, None, :]
    return _fsum_rows(_exact_terms(dall, sumi) + _exact_terms(-dmn, summ))


def qdot_q4k_q8k(xq, wblocks) -> tuple:
    """qdot for Q4_K weights [N, nsb, 144] and Q8_K activations."""
    return qdot("q4_k", xq, wblocks)


def kq_gateup_silu(x_bf16, w_gu, sorted_pairs, offsets, K: int, wtype: str = "q4_k"):
    """Keep-quant grouped gate-up with SiLU-mul ([PR 523] + [Issue 3094] N1).

    x bf16 [T, H] is quantized row by row (Q8_0 for Q8_0 weights, else Q8_K);
    w_gu blocks of format wtype [E, 2I, nb, bytes] (gate rows [0, I), up rows
    [I, 2I)); sorted row q of
    expert e takes token t = sorted[q] // K. g, u = the keep-quant dots;
    act[q] = bf16(silu(bf16(g)) * bf16(u)). Returns act bf16 [P, I] and the
    magnitudes of g and u (for error bounds)."""
    xf = f32_from_bf16(np.asarray(x_bf16))
    xq = quantize_act(wtype, xf)
    E, twoI = w_gu.shape[0], w_gu.shape[1]
    I = twoI // 2
    P = len(sorted_pairs)
    act = np.zeros((P, I), np.uint16)
    gmag = np.zeros((P, twoI))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        toks = np.asarray(sorted_pairs[lo:hi]) // K
        sub = tuple(a[toks] for a in xq)
        gu, mag = qdot(wtype, sub, w_gu[e])
        g = f32_from_bf16(bf16_from_f32(gu[:, :I]))
        u = f32_from_bf16(bf16_from_f32(gu[:, I:]))
        act[lo:hi] = bf16_from_f32((silu(g) * u).astype(F32))
        gmag[lo:hi] = mag
    return act, gmag


def kq_down(act_bf16, w_d, sorted_pairs, offsets, pair_w=None, wtype: str = "q4_k"):
    """Keep-quant grouped down projection ([PR 523] + [Issue 3094] N2).

    act bf16 [P, I] (sorted order) is quantized row by row (Q8_0 or Q8_K as
    for gate-up); w_d blocks of format wtype [E, H, nb, bytes]; expert_out[p] = bf16(y * pair_w[p]) at pair row
    p = sorted[q] (y the keep-quant dot, one f32 multiply, one rounding).
    Returns expert_out bf16 [P, H] and the magnitudes of y."""
    af = f32_from_bf16(np.asarray(act_bf16))
    aq = quantize_act(wtype, af)
    E, H = w_d.shape[0], w_d.shape[1]
    P = af.shape[0]
    out = np.zeros((P, H), np.uint16)
    ymag = np.zeros((P, H))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        sub = tuple(a[lo:hi] for a in aq)
        y, mag = qdot(wtype, sub, w_d[e])
        rows = np.asarray(sorted_pairs[lo:hi])
        if pair_w is not None:
            y = (y * np.asarray(pair_w, F32)[rows][:, None]).astype(F32)
        out[rows] = bf16_from_f32(y)
        ymag[rows] = mag
    return out, ymag
