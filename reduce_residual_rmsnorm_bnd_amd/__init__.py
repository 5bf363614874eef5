"""libboundary for AMD Instinct MI355X: the layer-boundary completion path.

Per token row: sum the outstanding tensor-parallel partials (or finalize a
deferred MoE handoff), fold the sum into the bf16 residual stream, and produce
the consumer's RMSNorm-ed input as bf16 or as per-token-scaled fp8 e4m3. The
kernels are hand-written HIP for gfx950 behind a C ABI (include/boundary.h);
this package is its Python binding.
"""
from .boundary import *  # noqa: F401,F403
from .boundary import BoundaryError, Stream, lib, SYMBOLS  # noqa: F401

__all__ = [n for n in dir() if n.startswith(("bnd_", "BND_"))] + [
    "BoundaryError", "Stream", "lib", "SYMBOLS", "set_option", "get_option", "status_name",
    "last_launch_shape"]
