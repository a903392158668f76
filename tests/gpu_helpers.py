"""Helpers of the GPU parity tests: host<->device moves and the tolerances.

Tolerances (the stated parity bar):
  * integer / index / routing-weight / combine results: bit-exact (NaN equals
    NaN in position, whatever its payload);
  * GEMM outputs (bf16): an element passes when its distance to the oracle is
    at most 2 bf16 ulps, or at most 1e-2 * rms(oracle tensor) (elements near
    zero after cancellation); the tensor passes when every element passes and
    NMSE = sum (gpu - ref)^2 / sum ref^2 <= 1e-5.
"""
import numpy as np
import torch

import oracle as O

DEV = torch.device("cuda:0")


def to_dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16)).view(torch.bfloat16).to(DEV)


def packed_gu(w):
    """Gate-up weights (bf16 bits [E, 2I, H] or [2I, H]) packed on the GPU."""
    import mixture_experts_ffn_expert_amd as moe
    return moe.moe_pack_weights(to_dev_bf16(w), "gateup")


def packed_d(w):
    """Down weights (bf16 bits [E, H, I] or [H, I]) packed on the GPU."""
    import mixture_experts_ffn_expert_amd as moe
    return moe.moe_pack_weights(to_dev_bf16(w), "plain")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bits(t):
    """Device tensor -> numpy (bf16 as uint16 bit patterns)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.uint16).cpu().numpy()
    return t.cpu().numpy()


def _ordered(b):
    b = b.astype(np.int32)
    return np.where(b & 0x8000, 0x8000 - b, b)


def bf16_ulp_distance(a, b):
    return np.abs(_ordered(a) - _ordered(b))


def assert_gemm_close(gpu_bits, ref_bits, what=""):
    gpu_bits = np.asarray(gpu_bits, np.uint16)
    ref_bits = np.asarray(ref_bits, np.uint16)
    assert gpu_bits.shape == ref_bits.shape, (what, gpu_bits.shape, ref_bits.shape)
    g = O.f32_from_bf16(gpu_bits).astype(np.float64)
    r = O.f32_from_bf16(ref_bits).astype(np.float64)
    assert np.all(np.isfinite(g)) and np.all(np.isfinite(r)), what
    rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
    ulp = bf16_ulp_distance(gpu_bits, ref_bits)
    ok = (ulp <= 2) | (np.abs(g - r) <= 1e-2 * rms)
    nbad = int(np.count_nonzero(~ok))
    den = np.sum(r * r)
    nmse = float(np.sum((g - r) ** 2) / den) if den > 0 else 0.0
    assert nbad == 0, f"{what}: {nbad}/{ok.size} elements outside 2 ulp / 1e-2 rms (max ulp {ulp.max()})"
    assert nmse <= 1e-5, f"{what}: NMSE {nmse:.3e} > 1e-5"
    return {"max_ulp": int(ulp.max()) if ulp.size else 0, "nmse": nmse, "n": int(ok.size)}


def assert_bits_equal(gpu, ref, what=""):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if gpu.dtype == np.float32:
        gn, rn = np.isnan(gpu), np.isnan(ref)
        assert np.array_equal(gn, rn), f"{what}: NaN positions differ"
        gpu = np.where(gn, 0, gpu.view(np.uint32))
        ref = np.where(rn, 0, ref.view(np.uint32))
    diff = int(np.count_nonzero(gpu != ref))
    assert diff == 0, f"{what}: {diff}/{gpu.size} elements differ"
    return gpu.size


def sub_gateup(x, w_gu, sorted_pairs, offsets, K, q_list):
    """Oracle act rows for sorted positions q_list (rows are independent)."""
    q_list = np.asarray(q_list, np.int64)
    e_of_q = np.searchsorted(offsets, q_list, side="right") - 1
    I = w_gu.shape[1] // 2
    out = np.zeros((q_list.size, I), np.uint16)
    for e in np.unique(e_of_q):
        sel = np.nonzero(e_of_q == e)[0]
        sp = np.asarray(sorted_pairs)[q_list[sel]]
        out[sel] = O.gateup_silu(x, w_gu[e:e + 1], sp, np.array([0, sel.size]), K)
    return out


def sub_down(act_rows, w_d, offsets, q_list, pair_w_of_rows):
    """Oracle expert_out rows for sorted positions q_list given their act rows."""
    q_list = np.asarray(q_list, np.int64)
    e_of_q = np.searchsorted(offsets, q_list, side="right") - 1
    H = w_d.shape[1]
    out = np.zeros((q_list.size, H), np.uint16)
    for e in np.unique(e_of_q):
        sel = np.nonzero(e_of_q == e)[0]
        n = sel.size
        w = None if pair_w_of_rows is None else np.asarray(pair_w_of_rows, np.float32)[sel]
        out[sel] = O.down_proj(act_rows[sel], w_d[e:e + 1], np.arange(n), np.array([0, n]), w)
    return out


def sample_rows(offsets, n_per_expert=3, seed=0):
    """Sorted positions to check: first, last and a random row of each touched
    expert (covering tile edges and ragged tails)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    qs = []
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        qs += [a, b - 1]
        qs += list(rng.integers(a, b, size=max(0, n_per_expert - 2)))
    return np.unique(np.array(qs, np.int64))
