"""CPU oracle for the BF16 MoE expert path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy code that states what each step of the
path computes. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path (the HIP
library and its Python binding) never does, and this package imports nothing
from it. See ``oracle/moe_oracle.py`` for the functions and their sources.

Parity status: every function is pinned by ``tests/test_oracle_*.py`` against
something other than itself (library routines, closed forms, invariants and a
brute-force dense evaluation). The GEMM values have no external printed
reference, so those are pinned only by the self-built checks listed there.
"""
from .moe_oracle import *  # noqa: F401,F403
from .keepquant import *  # noqa: F401,F403
from . import keepquant as _kq
from . import moe_oracle as _mo

__all__ = list(_mo.__all__) + list(_kq.__all__)
