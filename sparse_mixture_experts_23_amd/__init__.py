"""MI355X-native sparse Mixture-of-Experts layer forward.

The compute runs in hand-written HIP kernels for gfx950 behind the C-ABI in
include/moe.h (libmoe_mi355x.so, built by build.py); `api` wraps it for torch
tensors and `workloads` draws seeded synthetic inputs.
"""
from . import workloads  # noqa: F401

__all__ = ["workloads", "api", "_lib"]


def __getattr__(name):
    if name in ("api", "_lib"):
        import importlib
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
