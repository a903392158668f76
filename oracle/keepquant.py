"""Plain CPU oracle of the keep-quant grouped expert GEMM -- TEST
INFRASTRUCTURE ONLY (imported by tests, the smoke check and the benchmark's
CPU baseline; shares no code with the HIP library).

Source: [PR 523] (keep-quant grouped expert GEMM, "What changed"): expert
weights stay in their GGUF quantized block formats (Q8_0 / Q4_K / Q5_K /
Q6_K); activations are quantized on the fly (Q8_0 / Q8_K quantizers); the dot
products run over super-blocks with an integer core (DotQ4K ...); "Evidence":
the grouped case is checked against a CPU keep-quant reference, NMSE <= 5e-4.
This oracle covers Q4_K weights with Q8_K activations.

READING: the block formats are the published GGUF (ggml) ones:
* Q4_K, 144 bytes per super-block of 256 weights: f16 d, f16 dmin, 12 bytes
  of packed 6-bit sub-block scales and mins (8 sub-blocks of 32), 128 bytes of
  4-bit quants (byte b of 32-byte group i holds value b of sub-block 2i in its
  low nibble and value b of sub-block 2i+1 in its high nibble). Weight value
  w = d * sc_j * q - dmin * m_j.
* Q8_K, per 256 activations: f32 d, 256 int8 quants, 16 int16 sums of
  16-element groups. The quantizer takes the entry of largest magnitude (the
  first one) as `max`, iscale = -127 / max, q = min(127, round-half-even(
  iscale * x)), d = 1 / iscale (all f32); an all-zero block gives d = 0, q = 0.
The dot product of a Q4_K row with a Q8_K row is, per super-block,
  d_w d_x sum_j sc_j (sum_{l in j} q4_l q8_l) - dmin_w d_x sum_j m_j bsum_j,
which equals the dot product of the dequantized vectors. The oracle sums it
exactly (math.fsum over exact f64 terms) and rounds once to f32.
"""
from __future__ import annotations

import math

import numpy as np

from .moe_oracle import F32, bf16_from_f32, f32_from_bf16, silu

__all__ = ["Q4K_BLOCK", "q4k_scale_min", "q4k_unpack", "q4k_dequant",
           "quantize_q8k", "q8k_dequant", "qdot_q4k_q8k", "kq_gateup_silu", "kq_down"]

Q4K_BLOCK = 144   # bytes per super-block of 256 weights
QK = 256


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


def qdot_q4k_q8k(xq, wblocks) -> np.ndarray:
    """out[r, n] = fl32(sum over super-blocks of the keep-quant dot product of
    activation row r (Q8_K: qs, d, bsums) with weight row n (Q4_K blocks
    [N, nsb, 144])), summed exactly. Also returns the sum of the magnitudes of
    the per-super-block terms (for error bounds)."""
    qs, dx, bs = xq
    R, K = qs.shape
    N, nsb, _ = wblocks.shape
    d, dmin, sc, mn, q4 = q4k_unpack(wblocks)            # [N, nsb, ...]
    q8 = qs.reshape(R, nsb, 8, 32).astype(np.int64)
    q4 = q4.reshape(N, nsb, 8, 32).astype(np.int64)
    dots = np.einsum("rsjl,nsjl->rnsj", q8, q4)           # integer sub-block dots
    sumi = np.einsum("rnsj,nsj->rns", dots, sc.astype(np.int64))
    bsj = bs.reshape(R, nsb, 8, 2).sum(axis=3).astype(np.int64)   # sums of 32
    summ = np.einsum("rsj,nsj->rns", bsj, mn.astype(np.int64))
    dall = d.astype(np.float64)[None, :, :] * dx.astype(np.float64)[:, None, :]
    dmn = dmin.astype(np.float64)[None, :, :] * dx.astype(np.float64)[:, None, :]
    t1 = dall * sumi                                       # exact in f64
    t2 = dmn * summ
    out = np.empty((R, N), np.float64)
    for r in range(R):
        for n in range(N):
            out[r, n] = math.fsum(list(t1[r, n]) + list(-t2[r, n]))
    mag = (np.abs(t1) + np.abs(t2)).sum(axis=2)
    return out.astype(F32), mag


def kq_gateup_silu(x_bf16, w_gu, sorted_pairs, offsets, K: int):
    """Keep-quant grouped gate-up with SiLU-mul ([PR 523] + [Issue 3094] N1).

    x bf16 [T, H] is quantized row by row to Q8_K; w_gu Q4_K blocks
    [E, 2I, H/256, 144] (gate rows [0, I), up rows [I, 2I)); sorted row q of
    expert e takes token t = sorted[q] // K. g, u = the keep-quant dots;
    act[q] = bf16(silu(bf16(g)) * bf16(u)). Returns act bf16 [P, I] and the
    magnitudes of g and u (for error bounds)."""
    xf = f32_from_bf16(np.asarray(x_bf16))
    xq = quantize_q8k(xf)
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
        gu, mag = qdot_q4k_q8k(sub, w_gu[e])
        g = f32_from_bf16(bf16_from_f32(gu[:, :I]))
        u = f32_from_bf16(bf16_from_f32(gu[:, I:]))
        act[lo:hi] = bf16_from_f32((silu(g) * u).astype(F32))
        gmag[lo:hi] = mag
    return act, gmag


def kq_down(act_bf16, w_d, sorted_pairs, offsets, pair_w=None):
    """Keep-quant grouped down projection ([PR 523] + [Issue 3094] N2).

    act bf16 [P, I] (sorted order) is quantized row by row to Q8_K; w_d Q4_K
    blocks [E, H, I/256, 144]; expert_out[p] = bf16(y * pair_w[p]) at pair row
    p = sorted[q] (y the keep-quant dot, one f32 multiply, one rounding).
    Returns expert_out bf16 [P, H] and the magnitudes of y."""
    af = f32_from_bf16(np.asarray(act_bf16))
    aq = quantize_q8k(af)
    E, H = w_d.shape[0], w_d.shape[1]
    P = af.shape[0]
    out = np.zeros((P, H), np.uint16)
    ymag = np.zeros((P, H))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        sub = tuple(a[lo:hi] for a in aq)
        y, mag = qdot_q4k_q8k(sub, w_d[e])
        rows = np.asarray(sorted_pairs[lo:hi])
        if pair_w is not None:
            y = (y * np.asarray(pair_w, F32)[rows][:, None]).astype(F32)
        out[rows] = bf16_from_f32(y)
        ymag[rows] = mag
    return out, ymag
