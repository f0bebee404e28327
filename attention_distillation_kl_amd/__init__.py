"""StreamKL on MI355X: fused attention-KL divergence, forward and recompute backward.

The compute lives in hand-written HIP kernels for gfx950 behind a C ABI
(``libstreamkl.so``, declared in ``include/streamkl.h``); this package is the
thin Python binding over it.  Importing the package does not load the
library; the first call does, and it raises if the library is missing.
"""
from .inputs import WORKLOADS, Workload, make_inputs, workload_inputs  # noqa: F401

__all__ = ["WORKLOADS", "Workload", "make_inputs", "workload_inputs",
           "kl", "streamkl_fwd", "streamkl_bwd", "lib"]


def __getattr__(name):
    if name in ("kl", "streamkl_fwd", "streamkl_bwd", "StreamKLFunction"):
        from . import ops
        return getattr(ops, name)
    if name == "lib":
        from . import _lib
        return _lib
    raise AttributeError(name)
