"""MI355X-native single-GPU hot path of DeepEP-style MoE dispatch / combine.

The work runs in hand-written HIP kernels for gfx950 behind the C ABI of
``libepx.so`` (include/epx.h); this package is the torch binding. Every call
loads the library first and raises ImportError if it has not been built --
there is no fallback implementation. (Importing the package itself does not
need the library, so ``python -m combine_get_dispatch_counts_amd.build`` can
run before it exists.)
"""
from ._lib import EpxError

from .api import (  # noqa: E402
    Dispatched,
    Layout,
    LowLatency,
    alloc_dispatch,
    alloc_layout,
    alloc_ll,
    calibrate_sweep_rate,
    combine,
    combine_final,
    combine_partial,
    dispatch,
    dispatch_fused,
    fused_launches,
    fused_workspace_size,
    get_dispatch_layout,
    get_dispatch_layout_noalloc,
    get_error,
    get_sweep_rate,
    ll_dispatch,
    ll_reset,
    ll_size_hint,
    Received,
    recv_permute,
    scale_stride,
    set_sweep_rate,
    workspace_size,
)

__all__ = ["EpxError", "Layout", "Dispatched", "LowLatency", "workspace_size", "ll_size_hint",
           "scale_stride", "get_error", "alloc_layout", "get_dispatch_layout",
           "get_dispatch_layout_noalloc", "alloc_dispatch",
           "dispatch", "combine", "combine_partial", "combine_final", "ll_reset", "alloc_ll",
           "ll_dispatch", "Received", "recv_permute", "fused_workspace_size",
           "fused_launches", "dispatch_fused", "set_sweep_rate", "get_sweep_rate",
           "calibrate_sweep_rate"]
