"""Pins of the keep-quant oracle (Q4_K / Q5_K / Q6_K weights with Q8_K
activations, Q8_0 weights with Q8_0 activations).

* The 6-bit scale / min packing and the nibble order against an independent
  packer written from the format statement (round trips); the same for the
  Q5_K high bits, the Q6_K nibble / 2-bit / signed-scale layout and Q8_0.
* The Q8_K quantizer element by element against its definition in plain
  Python (first entry of largest magnitude, iscale = -127/max, round half to
  even, clamp at 127, d = 1/iscale), including an all-zero block and ties.
* The keep-quant dot against the float64 product of the dequantized operands.
* The gate-up and down steps against a dense brute force on dequantized
  values with the same N1 / N2 roundings.
* The Q8_0 quantizer against its definition (round half away from zero,
  f16 scale), with exact halves where half-to-even would differ.
* Planted mistakes (swapped nibbles, unsigned max, Q6_K without its offset
  of 32, Q5_K high bits in the wrong order, half-to-even Q8_0 rounding) fail
  a pin.
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W

F32 = np.float32


def _pack_scales(sc, mn):
    """Independent packer: 8 six-bit scales and mins -> 12 bytes."""
    b = [0] * 12
    for j in range(8):
        s, m = int(sc[j]), int(mn[j])
        if j < 4:
            b[j] |= s & 63
            b[j + 4] |= m & 63
        else:
            b[j + 4] |= (s & 0xF) | ((m & 0xF) << 4)
            b[j - 4] |= (s >> 4) << 6
            b[j] |= (m >> 4) << 6
    return np.array(b, np.uint8)


def _pack_quants(q):
    """256 four-bit values -> 128 bytes (group i: sub-block 2i low, 2i+1 high)."""
    out = np.zeros(128, np.uint8)
    for i in range(4):
        for l in range(32):
            out[32 * i + l] = int(q[64 * i + l]) | (int(q[64 * i + 32 + l]) << 4)
    return out


def test_scale_min_and_nibble_round_trip():
    g = np.random.Generator(np.random.PCG64(1))
    for _ in range(200):
        sc = g.integers(0, 64, 8)
        mn = g.integers(0, 64, 8)
        q = g.integers(0, 16, 256)
        blk = np.zeros(144, np.uint8)
        blk[0:2] = np.array([0.5], np.float16).view(np.uint8)
        blk[2:4] = np.array([0.25], np.float16).view(np.uint8)
        blk[4:16] = _pack_scales(sc, mn)
        blk[16:] = _pack_quants(q)
        d, dmin, s2, m2, q2 = O.q4k_unpack(blk)
        assert d == 0.5 and dmin == 0.25
        assert np.array_equal(s2, sc) and np.array_equal(m2, mn) and np.array_equal(q2, q)
        w = O.q4k_dequant(blk[None, :])           # one row of one super-block
        want = [0.5 * sc[l // 32] * q[l] - 0.25 * mn[l // 32] for l in range(256)]
        assert np.array_equal(w, np.array(want))


def test_planted_nibble_swap_fails_round_trip():
    q = np.random.Generator(np.random.PCG64(3)).integers(0, 16, 256)
    blk = np.zeros(144, np.uint8)
    packed = _pack_quants(q)
    blk[16:] = ((packed & 0xF) << 4) | (packed >> 4)        # swapped nibbles
    assert not np.array_equal(O.q4k_unpack(blk)[4], q)


def _q8k_python(block):
    """Definition of Q8_K on one block of 256 f32 values, plain Python."""
    xs = [F32(v) for v in block]
    amax, mx = F32(0), F32(0)
    for v in xs:
        if abs(v) > amax:
            amax, mx = abs(v), v
    if amax == 0:
        return [0] * 256, F32(0)
    iscale = F32(F32(-127.0) / mx)
    q = [min(127, int(round(float(F32(iscale * v))))) for v in xs]   # round: half to even
    return q, F32(F32(1.0) / iscale)


def test_q8k_quantizer_against_definition():
    g = np.random.Generator(np.random.PCG64(2))
    x = g.standard_normal((6, 512)).astype(F32)
    x[1, :256] = 0.0                                   # all-zero block
    x[2, 10], x[2, 20] = F32(5.0), F32(-5.0)           # tie in magnitude: first wins
    x[3, :256] = g.integers(-4, 5, 256).astype(F32) * F32(0.5)   # many exact halves
    qs, d, bs = O.quantize_q8k(x)
    for r in range(6):
        for b in range(2):
            q, dd = _q8k_python(x[r, 256 * b:256 * (b + 1)])
            assert qs[r, 256 * b:256 * (b + 1)].tolist() == q
            assert d[r, b] == dd
            for k in range(16):
                assert bs[r, 16 * b + k] == sum(q[16 * k:16 * k + 16])
    assert d[1, 0] == 0 and not qs[1, :256].any()
    assert qs[2, 10] == -127                            # the first max maps to -127
    err = np.abs(O.q8k_dequant(qs, d) - x.astype(np.float64))
    assert np.all(err <= np.abs(np.repeat(d, 256, axis=1)) * (0.5 + 1e-6) + 1e-30)


def test_planted_unsigned_max_changes_codes():
    x = np.linspace(1, -0.5, 256, dtype=F32)[None, :] * F32(3)   # largest entry positive
    qs, d, _ = O.quantize_q8k(x)
    bad = np.rint(x * (F32(127) / np.abs(x).max())).astype(np.int8)   # +127/amax
    assert not np.array_equal(qs, bad)


@pytest.mark.parametrize("K", [256, 768, 2048])
def test_qdot_equals_dequantized_product(K):
    g = np.random.Generator(np.random.PCG64(K))
    w = W.random_q4k_blocks(g.integers(1 << 30), (24,), K, 1 / math.sqrt(K))
    x = g.standard_normal((5, K)).astype(F32)
    xq = O.quantize_q8k(x)
    out, mag = O.qdot_q4k_q8k(xq, w)
    ref = O.q8k_dequant(xq[0], xq[1]) @ O.q4k_dequant(w).T
    assert np.all(np.abs(out - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-12 * mag)
    assert np.all(mag >= np.abs(ref) * (1 - 1e-12))


def test_layer_steps_against_dense_brute_force():
    g = np.random.Generator(np.random.PCG64(7))
    T, H, E, K, I = 12, 512, 4, 2, 256
    x = O.bf16_from_f32(g.standard_normal((T, H)).astype(F32))
    wgu = W.random_q4k_blocks(g.integers(1 << 30), (E, 2 * I), H, 1 / math.sqrt(H))
    wd = W.random_q4k_blocks(g.integers(1 << 30), (E, H), I, 1 / math.sqrt(I))
    logits = g.standard_normal((T, E)).astype(F32)
    ids, w, off, sp = O.route(logits, K)
    act, _ = O.kq_gateup_silu(x, wgu, sp, off, K)
    xd = O.q8k_dequant(*O.quantize_q8k(O.f32_from_bf16(x))[:2])
    wf = O.q4k_dequant(wgu)
    for q in range(T * K):
        p = sp[q]
        e = int(np.searchsorted(off, q, side="right") - 1)
        gu = (xd[p // K] @ wf[e].T).astype(F32)
        gb = O.f32_from_bf16(O.bf16_from_f32(gu[:I]))
        ub = O.f32_from_bf16(O.bf16_from_f32(gu[I:]))
        want = O.bf16_from_f32((O.silu(gb) * ub).astype(F32))
        assert np.max(np.abs(want.astype(np.int32) - act[q].astype(np.int32))) <= 1
    eo, _ = O.kq_down(act, wd, sp, off, w.reshape(-1))
    ad = O.q8k_dequant(*O.quantize_q8k(O.f32_from_bf16(act))[:2])
    wdf = O.q4k_dequant(wd)
    for q in range(T * K):
        p = sp[q]
        e = int(np.searchsorted(off, q, side="right") - 1)
        y = (ad[q] @ wdf[e].T).astype(F32)
        want = O.bf16_from_f32((y * w.reshape(-1)[p]).astype(F32))
        assert np.max(np.abs(want.astype(np.int32) - eo[p].astype(np.int32))) <= 1


# ---------------------------------------------------------------------------
# Q5_K, Q6_K, Q8_0 packers written from the format statements
# ---------------------------------------------------------------------------
def _f16_bytes(v):
    return np.array([v], np.float16).view(np.uint8)


def _pack_q5k(d, dmin, sc, mn, q):
    """q: 256 values in 0..31 -> one 176-byte Q5_K block."""
    blk = np.zeros(176, np.uint8)
    blk[0:2], blk[2:4] = _f16_bytes(d), _f16_bytes(dmin)
    blk[4:16] = _pack_scales(sc, mn)
    qh = [0] * 32
    for v in range(256):
        j, l = v // 32, v % 32
        if q[v] >= 16:
            qh[l] |= 1 << j
    blk[16:48] = qh
    blk[48:176] = _pack_quants([int(t) & 15 for t in q])
    return blk


def _pack_q6k(d, sc, q6):
    """q6: 256 values in -32..31, sc: 16 int8 -> one 210-byte Q6_K block."""
    blk = np.zeros(210, np.uint8)
    ql, qh = [0] * 128, [0] * 64
    for v in range(256):
        h, c, l = v // 128, (v % 128) // 32, v % 32
        u = int(q6[v]) + 32
        i = 64 * h + 32 * (c % 2) + l
        ql[i] |= (u & 15) << (0 if c < 2 else 4)
        qh[32 * h + l] |= (u >> 4) << (2 * c)
    blk[0:128], blk[128:192] = ql, qh
    blk[192:208] = np.array(sc, np.int8).view(np.uint8)
    blk[208:210] = _f16_bytes(d)
    return blk


def _pack_q8_0(d, q):
    blk = np.zeros(34, np.uint8)
    blk[0:2] = _f16_bytes(d)
    blk[2:34] = np.array(q, np.int8).view(np.uint8)
    return blk


def test_q5k_round_trip():
    g = np.random.Generator(np.random.PCG64(11))
    for _ in range(100):
        sc, mn, q = g.integers(0, 64, 8), g.integers(0, 64, 8), g.integers(0, 32, 256)
        blk = _pack_q5k(0.5, 0.125, sc, mn, q)
        d, dmin, s2, m2, q2 = O.q5k_unpack(blk)
        assert d == 0.5 and dmin == 0.125
        assert np.array_equal(s2, sc) and np.array_equal(m2, mn) and np.array_equal(q2, q)
        want = [0.5 * sc[v // 32] * q[v] - 0.125 * mn[v // 32] for v in range(256)]
        assert np.array_equal(O.q5k_dequant(blk[None, :]), np.array(want))


def test_planted_q5k_high_bit_order_fails():
    q = np.random.Generator(np.random.PCG64(12)).integers(0, 32, 256)
    blk = _pack_q5k(1.0, 0.0, np.ones(8, int), np.zeros(8, int), q)
    rev = blk.copy()
    for l in range(32):                       # qh bits in reverse sub-block order
        b = int(blk[16 + l])
        rev[16 + l] = int(f"{b:08b}"[::-1], 2)
    assert not np.array_equal(O.q5k_unpack(rev)[4], q)


def test_q6k_round_trip():
    g = np.random.Generator(np.random.PCG64(13))
    for _ in range(100):
        sc, q6 = g.integers(-128, 128, 16), g.integers(-32, 32, 256)
        blk = _pack_q6k(0.25, sc, q6)
        d, s2, q2 = O.q6k_unpack(blk)
        assert d == 0.25
        assert np.array_equal(s2, sc) and np.array_equal(q2, q6)
        want = [0.25 * sc[v // 16] * q6[v] for v in range(256)]
        assert np.array_equal(O.q6k_dequant(blk[None, :]), np.array(want))


def test_planted_q6k_offset_missing_fails():
    g = np.random.Generator(np.random.PCG64(14))
    q6 = g.integers(-32, 32, 256)
    blk = _pack_q6k(1.0, np.ones(16, int), q6)
    _, _, q2 = O.q6k_unpack(blk)
    assert np.array_equal(q2, q6) and q2.min() < 0         # the round-trip pin
    assert not np.array_equal(q2 + 32, q6)                 # an unpacker without the offset fails it


def test_q8_0_round_trip():
    g = np.random.Generator(np.random.PCG64(15))
    for _ in range(50):
        q = g.integers(-128, 128, 32)
        d, q2 = O.q8_0_unpack(_pack_q8_0(0.75, q))
        assert d == 0.75 and np.array_equal(q2, q)


def _q8_0_python(block):
    """Definition of Q8_0 on one block of 32 f32 values, plain Python."""
    xs = [F32(v) for v in block]
    amax = max(abs(v) for v in xs)
    d = F32(amax / F32(127.0))
    idv = F32(F32(1.0) / d) if d != 0 else F32(0.0)
    q = []
    for v in xs:
        t = float(F32(v * idv))
        q.append(int(math.copysign(math.floor(abs(t) + 0.5), t)))   # half away from zero
    return q, np.float16(d)


def test_q8_0_quantizer_against_definition():
    g = np.random.Generator(np.random.PCG64(16))
    x = g.standard_normal((4, 96)).astype(F32)
    x[1, :32] = 0.0                                          # all-zero block
    x[2, :32] = np.arange(-16, 16, dtype=F32) + F32(0.5)     # amax 15.5, d exact? no
    x[3, :32] = 0.0
    x[3, 0] = F32(127.0)                                     # d = 1, id = 1: exact halves
    x[3, 1:6] = [2.5, -2.5, 0.5, -0.5, 3.5]
    qs, d16 = O.quantize_q8_0(x)
    for r in range(4):
        for b in range(3):
            q, dd = _q8_0_python(x[r, 32 * b:32 * b + 32])
            assert qs[r, 32 * b:32 * b + 32].tolist() == q
            assert d16[r, b] == dd
    assert qs[3, 1:6].tolist() == [3, -3, 1, -1, 4]          # away from zero, not to even
    assert d16[1, 0] == 0 and not qs[1, :32].any()


def test_planted_half_even_q8_0_fails():
    x = np.zeros((1, 32), F32)
    x[0, 0], x[0, 1] = 127.0, 2.5
    qs, _ = O.quantize_q8_0(x)
    assert qs[0, 1] != int(np.rint(2.5))                     # half-even would give 2


@pytest.mark.parametrize("wtype", ["q4_k", "q5_k", "q6_k", "q8_0"])
@pytest.mark.parametrize("K", [256, 768])
def test_qdot_all_formats_equal_dequantized_product(wtype, K):
    g = np.random.Generator(np.random.PCG64(K + len(wtype)))
    w = W.random_kq_blocks(wtype, g.integers(1 << 30), (20,), K, 1 / math.sqrt(K))
    x = g.standard_normal((5, K)).astype(F32)
    xq = O.quantize_act(wtype, x)
    out, mag = O.qdot(wtype, xq, w)
    ref = O.act_dequant(wtype, xq) @ O.kq_dequant(wtype, w).T
    assert np.all(np.abs(out - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-12 * mag)
    assert np.all(mag >= np.abs(ref) * (1 - 1e-12))
    # and the dequantized weights are what the packers say: spot-check one
    # row against an independent decode of its first block
    wd = O.kq_dequant(wtype, w[:1])[0]
    assert np.all(np.isfinite(wd)) and np.abs(wd).max() > 0


def test_qdot_exact_under_cancellation():
    """Scale and mins terms of size ~2e5 that cancel exactly: w = d*sc*q -
    dmin*m = 63*15 - 15*63 = 0 for every weight, so the product is 0."""
    blk = _pack_q4k_block(1.0, 15.0, np.full(8, 63), np.full(8, 63), np.full(256, 15))
    x = np.ones((1, 256), F32)
    out, mag = O.qdot("q4_k", O.quantize_q8k(x), blk[None, None, :])
    assert out[0, 0] == 0.0 and mag[0, 0] > 1e5


def test_exact_terms_against_rational_arithmetic():
    """The split products sum to coef * ints exactly, where one f64 product
    would round (35-bit coefficient times a 26-bit integer)."""
    from fractions import Fraction
    coef = np.array([[[float(np.float16(1 + 2 ** -10)) * float(F32(1 + 2 ** -23))]]])
    ints = np.array([[[(1 << 25) + 12345]]])
    exact = Fraction(coef[0, 0, 0]) * int(ints[0, 0, 0])
    terms = O.keepquant._exact_terms(coef, ints)
    assert sum(Fraction(float(t[0, 0, 0])) for t in terms) == exact
    assert Fraction(coef[0, 0, 0] * float(ints[0, 0, 0])) != exact   # one product rounds


def _pack_q4k_block(d, dmin, sc, mn, q):
    blk = np.zeros(144, np.uint8)
    blk[0:2], blk[2:4] = _f16_bytes(d), _f16_bytes(dmin)
    blk[4:16] = _pack_scales(sc, mn)
    blk[16:] = _pack_quants(q)
    return blk


@pytest.mark.parametrize("wtype", ["q6_k", "q8_0"])
def test_layer_steps_other_formats_against_dense_brute_force(wtype):
    g = np.random.Generator(np.random.PCG64(8))
    T, H, E, K, I = 8, 512, 4, 2, 256
    x = O.bf16_from_f32(g.standard_normal((T, H)).astype(F32))
    wgu = W.random_kq_blocks(wtype, g.integers(1 << 30), (E, 2 * I), H, 1 / math.sqrt(H))
    wd = W.random_kq_blocks(wtype, g.integers(1 << 30), (E, H), I, 1 / math.sqrt(I))
    ids, w, off, sp = O.route(g.standard_normal((T, E)).astype(F32), K)
    act, _ = O.kq_gateup_silu(x, wgu, sp, off, K, wtype)
    xd = O.act_dequant(wtype, O.quantize_act(wtype, O.f32_from_bf16(x)))
    wf = O.kq_dequant(wtype, wgu)
    for q in range(T * K):
        p = sp[q]
        e = int(np.searchsorted(off, q, side="right") - 1)
        gu = (xd[p // K] @ wf[e].T).astype(F32)
        gb = O.f32_from_bf16(O.bf16_from_f32(gu[:I]))
        ub = O.f32_from_bf16(O.bf16_from_f32(gu[I:]))
        want = O.bf16_from_f32((O.silu(gb) * ub).astype(F32))
        assert np.max(np.abs(want.astype(np.int32) - act[q].astype(np.int32))) <= 1
    eo, _ = O.kq_down(act, wd, sp, off, w.reshape(-1), wtype)
    ad = O.act_dequant(wtype, O.quantize_act(wtype, O.f32_from_bf16(act)))
    wdf = O.kq_dequant(wtype, wd)
    for q in range(T * K):
        p = sp[q]
        e = int(np.searchsorted(off, q, side="right") - 1)
        y = (ad[q] @ wdf[e].T).astype(F32)
        want = O.bf16_from_f32((y * w.reshape(-1)[p]).astype(F32))
        assert np.max(np.abs(want.astype(np.int32) - eo[p].astype(np.int32))) <= 1
