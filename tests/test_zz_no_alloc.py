"""The allocation-free routing entry point (moe_route_noalloc), called through
the C ABI, against moe_route with a caller workspace: every output
(topk_ids, topk_w bits, expert_offsets, sorted_pairs) identical, on two calls
in a row whose second is smaller (so the library's scratch still holds the
first call's counts when the second starts), and on a size that needs no
scratch. Runs alone or after the other GPU tests."""
import ctypes

import numpy as np
import pytest
import torch

import mixture_experts_ffn_expert_amd as moe

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _logits(T, E, seed, skew):
    g = np.random.Generator(np.random.PCG64(seed))
    l = g.standard_normal((T, E)).astype(np.float32)
    if skew:   # a Zipf-like per-expert bias: a few experts take most pairs
        rank = 1 + g.permutation(E)
        l = (l + (2.0 * np.log(1.0 / rank)).astype(np.float32)[None, :]).astype(np.float32)
    return torch.from_numpy(l).to(DEV)


def _noalloc(logits, K):
    T, E = logits.shape
    out = (torch.full((T, K), -7, dtype=torch.int32, device=DEV),
           torch.full((T, K), float("nan"), dtype=torch.float32, device=DEV),
           torch.full((E + 1,), -7, dtype=torch.int32, device=DEV),
           torch.full((T * K,), -7, dtype=torch.int32, device=DEV))
    p = [ctypes.c_void_p(t.data_ptr()) for t in out]
    st = moe.load().moe_route_noalloc(ctypes.c_void_p(logits.data_ptr()), T, E, K, *p,
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, moe.load().moe_last_error().decode()
    return out


def _same(a, b):
    ids, w, off, sp = a
    ids2, w2, off2, sp2 = b
    assert torch.equal(ids, ids2)
    assert torch.equal(w.view(torch.int32), w2.view(torch.int32))
    assert torch.equal(off, off2)
    assert torch.equal(sp, sp2)


def test_noalloc_route_equals_workspace_route_twice_second_smaller():
    moe.load()
    moe.moe_init()
    cases = [(8192, 128, 8, True),    # 65,536 pairs: 64 segments x 128 experts of scratch
             (700, 64, 7, False),     # 4,900 pairs: 5 segments x 64, smaller than the first
             (300, 32, 4, False)]     # 1,200 pairs: one-workgroup grouping, no scratch
    for i, (T, E, K, skew) in enumerate(cases):
        print(f"case T={T} E={E} K={K}", flush=True)
        l = _logits(T, E, 40 + i, skew)
        ref = moe.moe_route(l, K)
        got = _noalloc(l, K)
        torch.cuda.synchronize()
        _same(ref, got)
        counts = torch.diff(got[2].long())
        assert int(counts.sum()) == T * K and int(counts.min()) >= 0


def test_noalloc_route_binding_and_refusal():
    l = _logits(4100, 16, 7, False)            # 32,800 pairs
    K = 8
    T, E = l.shape
    outs = (torch.empty((T, K), dtype=torch.int32, device=DEV),
            torch.empty((T, K), dtype=torch.float32, device=DEV),
            torch.empty((E + 1,), dtype=torch.int32, device=DEV),
            torch.empty((T * K,), dtype=torch.int32, device=DEV))
    got = moe.moe_route_noalloc(l, K, *outs)
    _same(moe.moe_route(l, K), got)
    big = torch.empty((262145, 128), dtype=torch.float32, device=DEV)   # 2,097,160 pairs
    with pytest.raises(moe.MoeError, match="grouping scratch"):
        moe.moe_route_noalloc(big, 8, torch.empty((262145, 8), dtype=torch.int32, device=DEV),
                              torch.empty((262145, 8), dtype=torch.float32, device=DEV),
                              torch.empty((129,), dtype=torch.int32, device=DEV),
                              torch.empty((262145 * 8,), dtype=torch.int32, device=DEV))
