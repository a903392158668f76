"""GPU checks of the measurement micro-kernels (the HBM-read and MFMA
ceilings that the benchmark reports beside the datasheet peaks): each
computes what it claims, so its timing measures real work.

* The read probe's per-thread XORs combine to the XOR of every dword of the
  buffer, for sizes that are and are not multiples of the grid stride.
* The MFMA probe on small-integer operands (every sum exact in f32): the sum
  of a wavefront's outputs equals iters * sum over its four chains of
  sum_k colsum_A[k] * rowsum_B[k], with the operand of lane l of wave w,
  chain j taken from ops[(64 w + l) * 4 + j] (A) and
  ops[(64 w + l) * 4 + j + 2 n / 3] (B), both modulo n, and lane l holding
  row / column l % 32 at k = 8 (l / 32) .. + 8 of the 32 x 32 x 16 MFMA.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) + 16 * 77, 64 << 20])
def test_read_probe_xor(gpu_lib, nbytes):
    print(f"read probe {nbytes} bytes", flush=True)
    g = np.random.Generator(np.random.PCG64(nbytes))
    host = g.integers(0, 256, size=nbytes, dtype=np.uint8)
    buf = torch.from_numpy(host).to(DEV)
    out = gpu_lib.moe_probe_hbm_read(buf)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    exp = np.bitwise_xor.reduce(host.view(np.uint32))
    assert got == exp


@pytest.mark.parametrize("n_ops,iters", [(1000, 3), (262144 * 4, 2)])
def test_mfma_probe_exact(gpu_lib, n_ops, iters):
    print(f"mfma probe n_ops={n_ops} iters={iters}", flush=True)
    g = np.random.Generator(np.random.PCG64(n_ops + iters))
    vals = g.integers(-2, 3, size=(n_ops, 8)).astype(np.float32)
    ops = torch.from_numpy(vals).to(torch.bfloat16).reshape(-1).to(DEV)
    out = gpu_lib.moe_probe_mfma_bf16(ops, iters)
    torch.cuda.synchronize()
    per_wave = out.cpu().numpy().astype(np.float64).reshape(-1, 64).sum(axis=1)
    n_waves = per_wave.size
    assert n_waves == 4096
    lanes = np.arange(64)
    m = lanes % 32
    half = lanes // 32
    off = 2 * n_ops // 3
    for w in list(range(0, n_waves, 509)) + [n_waves - 1]:
        tot = 0.0
        for j in range(4):
            ia = ((64 * w + lanes) * 4 + j) % n_ops
            ib = ((64 * w + lanes) * 4 + j + off) % n_ops
            a = np.zeros((32, 16))
            b = np.zeros((16, 32))
            for ll in range(64):
                a[m[ll], 8 * half[ll]:8 * half[ll] + 8] = vals[ia[ll]]
                b[8 * half[ll]:8 * half[ll] + 8, m[ll]] = vals[ib[ll]]
            tot += float((a @ b).sum())
        assert per_wave[w] == iters * tot, (w, per_wave[w], iters * tot)
    assert gpu_lib.moe_probe_mfma_flops(iters) == n_waves * iters * 4 * 32 * 32 * 16 * 2
