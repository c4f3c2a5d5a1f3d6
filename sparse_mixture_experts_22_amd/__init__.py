"""MI355X (gfx950) sparse mixture-of-experts layer.

A thin ctypes binding over libmoe.so (include/moe.h).  It only checks and
marshals arguments: every step of the layer runs in the HIP kernels.  PyTorch
supplies device memory and the current stream.  If the library has not been
built, every call raises; there is no CPU fallback.
"""
from ._binding import (  # noqa: F401
    MoEError,
    STATUS,
    check_dispatch,
    expert_capacity,
    expert_choice_capacity,
    forward,
    forward_capacity,
    forward_expert_choice,
    forward_q4,
    forward_f32,
    forward_traced,
    forward_noalloc,
    forward_packed,
    forward_packed_traced,
    pack_down,
    pack_up,
    noalloc_scratch_bytes,
    NOALLOC_SCRATCH_BYTES,
    last_error,
    lib,
    lib_path,
    quantize_q4,
    release,
    route,
    route_capacity,
    route_expert_choice,
    route_f32,
    route_stats,
    route_stats_f32,
    version,
    workspace_bytes,
)

__all__ = ["forward", "forward_traced", "forward_noalloc", "pack_up", "pack_down", "forward_packed",
           "forward_packed_traced", "noalloc_scratch_bytes", "NOALLOC_SCRATCH_BYTES", "forward_f32", "route", "route_f32", "route_stats", "route_stats_f32",
           "expert_capacity", "route_capacity", "forward_capacity", "check_dispatch",
           "quantize_q4", "forward_q4", "expert_choice_capacity", "route_expert_choice",
           "forward_expert_choice", "workspace_bytes", "release",
           "last_error", "version", "lib", "lib_path", "MoEError", "STATUS"]
