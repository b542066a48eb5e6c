"""The BackLite attention module: exact forward, block-sparse backward.

Mirrors the interface the BackLite README describes ("Usage"):
``BackLite(negl_prob=0.05)`` is called as ``attn(query, key, value, scale=None,
return_softmax_lse=False, tile_stats=None)`` on (batch, seq_len, heads,
head_dim) bf16 tensors, with ``key``/``value`` carrying ``heads_k <= heads``.
With ``negl_prob > 0`` the forward records the per-row tile statistics in
``tile_stats`` (allocated here unless the caller passes one; it is only staging)
and reduces them to one log-weight per tile pair, which is all the module keeps
for the backward (128 rows to one value, 64x fewer bytes).  The backward builds
the tile mask from those and skips the masked tiles; with
``negl_prob == 0`` no statistics are recorded and the backward is dense.  A
``causal`` flag is added (the pages' LLM use is causal), and a ``window`` for
sliding-window layers (key j visible to query i iff i - window < j <= i).

Every step runs in the HIP library through ``_lib``; torch supplies device
memory, streams and autograd plumbing only.
"""
from __future__ import annotations

import math
import os

import torch

from . import _lib


class _BackLiteFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, scale, causal, negl_prob, tile_stats, stats_out, window, ws_cache, q_tile):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        tw = None
        if negl_prob > 0:
            B, n, H, _ = q.shape
            tw = torch.empty(_lib.tile_w_elems(B, H, n, causal), dtype=torch.float64, device=q.device)
        o, lse, _, olo = _lib.fwd(q, k, v, scale=scale, causal=causal, with_stats=negl_prob > 0,
                                  tile_lse=tile_stats if negl_prob > 0 else None, with_residual=True,
                                  window=window, tile_w=tw)
        # the compact statistics live as long as the graph (autograd frees them
        # with it), so a second backward through the same graph finds them too
        ctx.save_for_backward(q, k, v, o, olo, lse, tw)
        ctx.scale, ctx.causal, ctx.negl, ctx.window, ctx.q_tile = scale, causal, negl_prob, window, q_tile
        ctx.stats_out = stats_out
        ctx.ws_cache = ws_cache
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        q, k, v, o, olo, lse, tw = ctx.saved_tensors
        n = q.shape[1]
        B, _, H, _ = q.shape
        lists = _lib.mask_compact(tw, B, H, n, ctx.causal, ctx.negl, stats=ctx.stats_out,
                                  window=ctx.window, device=q.device, q_tile=ctx.q_tile)
        ws = ctx.ws_cache.get(q, k, ctx.causal, ctx.window, ctx.q_tile) if ctx.ws_cache is not None else None
        dq, dk, dv = _lib.bwd(q, k, v, o, do.contiguous(), lse, lists, scale=ctx.scale,
                              causal=ctx.causal, o_lo=olo, window=ctx.window, workspace=ws)
        return dq, dk, dv, None, None, None, None, None, None, None, None


class _WorkspaceCache:
    """One backward workspace per (device, shape), allocated on first use and
    reused by every later backward of that shape: no allocation and no device
    readback inside the backward.  Its G_S slots are sized from the candidate
    tile pairs, capped by a byte budget (None: an eighth of the device's
    memory); query tiles whose kept tiles do not all fit recompute G_Q."""

    def __init__(self, gs_budget_bytes=None):
        self.gs_budget_bytes = gs_budget_bytes
        self._ws = {}

    def get(self, q, k, causal, window, q_tile):
        key = (q.device, tuple(q.shape), k.shape[2], bool(causal), int(window), int(q_tile))
        ws = self._ws.get(key)
        if ws is None:
            ws = _lib.bwd_workspace(q, k, None, "auto", causal=causal, window=window,
                                    gs_budget_bytes=self.gs_budget_bytes, q_tile=q_tile)
            self._ws[key] = ws
        return ws

    def clear(self):
        self._ws.clear()


class BackLite(torch.nn.Module):
    """Attention with an exact forward and a block-sparse backward.

    negl_prob: tiles are skipped in the backward, smallest weight first, while
    their cumulative weight stays below this value (0 = dense backward).
    gs_budget_bytes: device memory for the stored-G_S slots of the backward
    workspace (None: an eighth of the device's memory, at most one slot per
    candidate tile pair).  The workspace is allocated on the first backward of
    a shape and reused.
    q_tile: rows of the backward's query tiles, 128 or 64 (half-height tiles
    give a finer mask: the README forms it "for each backward tile pair").
    """

    def __init__(self, negl_prob: float = 0.05, causal: bool = False, window: int = 0,
                 gs_budget_bytes: int | None = None, q_tile: int = 128):
        super().__init__()
        if q_tile not in (64, 128):
            raise ValueError("q_tile must be 64 or 128")
        self.q_tile = int(q_tile)
        if not (0.0 <= negl_prob < 1.0) or math.isnan(negl_prob):
            raise ValueError("negl_prob must be in [0, 1)")
        if window < 0 or (window > 0 and not causal):
            raise ValueError("window must be >= 0, and a window needs causal=True")
        self.negl_prob = float(negl_prob)
        self.causal = bool(causal)
        self.window = int(window)
        self.verbose = os.environ.get("BACKLITE_VERBOSE", "0") not in ("", "0")
        self.last_stats = None
        # the backward workspace, kept across steps (see _WorkspaceCache)
        self.workspaces = _WorkspaceCache(gs_budget_bytes)

    def forward(self, query, key, value, scale=None, return_softmax_lse=False, tile_stats=None,
                causal=None):
        causal = self.causal if causal is None else bool(causal)
        d = query.shape[-1]
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        stats = None
        if self.verbose:
            stats = torch.zeros(2, dtype=torch.int64, device=query.device)
            self.last_stats = stats
        o, lse = _BackLiteFn.apply(query, key, value, scale, causal, self.negl_prob, tile_stats, stats,
                                   self.window if causal else 0, self.workspaces, self.q_tile)
        if return_softmax_lse:
            return o, lse
        return o

    def extra_repr(self) -> str:
        return f"negl_prob={self.negl_prob}, causal={self.causal}, window={self.window}, q_tile={self.q_tile}"


def sparsity(stats: torch.Tensor) -> float:
    """1 - kept / candidate tile pairs from a stats buffer filled by the mask."""
    s = stats.tolist()
    return 1.0 - s[1] / s[0] if s[0] else 0.0


__all__ = ["BackLite", "sparsity"]
