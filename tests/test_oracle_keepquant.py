"""Pins of the keep-quant oracle (Q4_K weights, Q8_K activations).

* The 6-bit scale / min packing and the nibble order against an independent
  packer written from the format statement (round trips).
* The Q8_K quantizer element by element against its definition in plain
  Python (first entry of largest magnitude, iscale = -127/max, round half to
  even, clamp at 127, d = 1/iscale), including an all-zero block and ties.
* The keep-quant dot against the float64 product of the dequantized operands.
* The gate-up and down steps against a dense brute force on dequantized
  values with the same N1 / N2 roundings.
* Planted mistakes (swapped nibbles, unsigned max) fail a pin.
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
