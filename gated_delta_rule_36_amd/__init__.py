"""MI355X (gfx950) Kimi Delta Attention chunked forward pass.

``fwd(...)`` is the whole API: a thin binding over the C-ABI library
``libkda.so`` (declared in ``include/kda.h``), whose hand-written HIP kernels
run every step of the forward pass.  ``synth`` draws the seeded synthetic
inputs of the named workloads.
"""
from ._lib import KdaLibraryMissing
from .api import KdaArgumentError, KdaError, auto_segment_chunks, fwd, fwd_kernel

__all__ = ["fwd", "fwd_kernel", "auto_segment_chunks", "KdaError", "KdaArgumentError", "KdaLibraryMissing"]
