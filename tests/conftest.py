import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; fails (never skips) without a GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test ran without a visible GPU")
    import mixture_experts_ffn_expert_amd as moe
    moe.load()
    return moe


_INPUTS = {}


def cached_inputs(n, **kw):
    """Workload inputs generated once per test session (they are large)."""
    import workloads
    key = (n, tuple(sorted(kw.items())))
    if key not in _INPUTS:
        if len(_INPUTS) >= 2:          # keep host memory bounded
            _INPUTS.pop(next(iter(_INPUTS)))
        _INPUTS[key] = workloads.make_inputs(n, **kw)
    return _INPUTS[key]
