"""The gate-up epilogue's SiLU table against the oracle, on the CPU.

The tile GEMM takes SiLU of a bf16 gate from a table of the 7,936 bf16
patterns without a closed form plus closed forms for the rest
(csrc/silu_table.h, built by the compiler). Here that header is compiled
into a small host program (g++, the same constexpr table and the same lookup
function the kernel calls) and, for every one of the 65,536 bf16 gate
patterns, its result is compared bit for bit with the oracle's SiLU of the
same f32 value (NaNs: the same positions). The table's own entries and its
zero padding are checked too, so a wrong index layout cannot hide behind the
closed forms.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from oracle import moe_oracle as O  # noqa: E402

CSRC = os.path.join(ROOT, "mixture_experts_ffn_expert_amd", "csrc")

PROGRAM = textwrap.dedent("""\
    #include <cstdio>
    #include <cstring>
    #include "silu_table.h"
    static constexpr moe::SiluTable kTab = moe::make_silu_table();
    int main() {
      for (int i = 0; i < moe::kSiluTabFloats; ++i) {
        unsigned u; std::memcpy(&u, &kTab.v[i], 4); std::printf("%08x\\n", u);
      }
      for (unsigned b = 0; b < 65536u; ++b) {
        const float v = moe::silu_bf16(b, kTab.v);
        unsigned u; std::memcpy(&u, &v, 4); std::printf("%08x\\n", u);
      }
      return 0;
    }
    """)


@pytest.fixture(scope="module")
def host_table(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    d = tmp_path_factory.mktemp("silu_table")
    src, exe = d / "dump.cpp", d / "dump"
    src.write_text(PROGRAM)
    subprocess.run(["g++", "-std=c++17", "-O2", "-ffp-contract=off", f"-I{CSRC}", str(src), "-o",
                    str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    vals = np.array([int(w, 16) for w in out], dtype=np.uint32)
    assert vals.size == 8192 + 65536
    return vals[:8192], vals[8192:]


def _oracle_silu_bits(bf16_bits):
    g = (bf16_bits.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(all="ignore"):
        return O.silu(g).view(np.uint32)


def _same(a, b):
    fa, fb = a.view(np.float32), b.view(np.float32)
    nan_a, nan_b = np.isnan(fa), np.isnan(fb)
    assert np.array_equal(nan_a, nan_b), "NaN positions differ"
    bad = np.nonzero((a != b) & ~nan_a)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first at index {bad[:5]}: {a[bad[:5]]} vs {b[bad[:5]]}"


def test_every_bf16_gate(host_table):
    _, lookup = host_table
    _same(lookup, _oracle_silu_bits(np.arange(65536, dtype=np.uint32)))


def test_table_entries_and_padding(host_table):
    tab, _ = host_table
    i = np.arange(7936, dtype=np.uint32)
    s, rem = i // 3968, i % 3968
    bits = (s << 15) | ((103 + rem // 128) << 7) | (rem % 128)
    _same(tab[:7936], _oracle_silu_bits(bits))
    assert not tab[7936:].any()
