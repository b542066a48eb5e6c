"""BackLite attention hot path for AMD MI355X (gfx950).

Exact FlashAttention-style forward that records a log-sum-exp per (query row,
key tile); a mask pass that skips the smallest-weight key tiles per query tile
while their cumulative weight stays below ``negl_prob``; and a block-sparse
backward over the kept tiles.  Kernels are hand-written HIP in ``csrc/`` behind
the C ABI of ``include/backlite.h``; ``_lib`` is the ctypes binding.
``calibrate_negl_prob`` picks negl_prob for gradient-similarity targets.
"""
from . import _lib  # noqa: F401
from ._lib import BackliteError, bwd, fwd, mask  # noqa: F401
from .attention import BackLite, sparsity  # noqa: F401
from .calibrate import calibrate_negl_prob  # noqa: F401

__all__ = ["BackLite", "sparsity", "fwd", "mask", "bwd", "BackliteError", "calibrate_negl_prob"]
