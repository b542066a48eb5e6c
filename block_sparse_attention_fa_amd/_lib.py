"""ctypes binding of libbacklite.so (argument marshalling only).

Every function here takes torch CUDA tensors, checks dtype/shape/device on the
host, and passes raw device pointers and the current HIP stream to the C ABI
declared in include/backlite.h.  All computation happens in the library's HIP
kernels; there is no fallback: if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("BACKLITE_LIB", os.path.join(_PKG, "libbacklite.so"))
TILE = 128

_lib = None


class BackliteError(RuntimeError):
    pass


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise BackliteError(
            f"{LIB_PATH} not found: build it with `python -m block_sparse_attention_fa_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.backlite_tile_lse_elems.argtypes = [I, I, I, I]
    lib.backlite_tile_lse_elems.restype = Z
    lib.backlite_mask_elems.argtypes = [I, I, I, I]
    lib.backlite_mask_elems.restype = Z
    lib.backlite_count_elems.argtypes = [I, I, I, I]
    lib.backlite_count_elems.restype = Z
    lib.backlite_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.backlite_bwd_workspace_bytes.restype = Z
    lib.backlite_bwd_workspace_bytes_stored.argtypes = [I, I, I, I, I, I, ctypes.c_int64]
    lib.backlite_bwd_workspace_bytes_stored.restype = Z
    lib.backlite_bwd_state_offset.argtypes = [I, I, I, I, I]
    lib.backlite_bwd_state_offset.restype = Z
    lib.backlite_fwd.argtypes = [P, P, P, I, I, I, I, I, F, I, I, P, P, P, P, P, P]
    lib.backlite_fwd.restype = I
    lib.backlite_mask.argtypes = [P, P, I, I, I, I, I, I, F, P, P, P, P, P, P, P]
    lib.backlite_mask.restype = I
    lib.backlite_mask_compact.argtypes = [P, I, I, I, I, I, I, F, P, P, P, P, P, P, P]
    lib.backlite_mask_compact.restype = I
    lib.backlite_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, I, P, P, P, P, Z, P]
    lib.backlite_bwd.restype = I
    lib.backlite_bwd_atomic_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.backlite_bwd_atomic_workspace_bytes.restype = Z
    lib.backlite_bwd_atomic.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, P, P, P, P, Z, P]
    lib.backlite_bwd_atomic.restype = I
    lib.backlite_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, I, P, P, P, P]
    lib.backlite_bwd_noalloc.restype = I
    lib.backlite_bwd_noalloc_scratch_bytes.argtypes = []
    lib.backlite_bwd_noalloc_scratch_bytes.restype = Z
    lib.backlite_profile_enable.argtypes = [I]
    lib.backlite_profile_enable.restype = I
    lib.backlite_profile_reset.argtypes = []
    lib.backlite_profile_reset.restype = I
    lib.backlite_profile_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int64)]
    lib.backlite_profile_read.restype = I
    lib.backlite_check_lists.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_char_p, Z]
    lib.backlite_check_lists.restype = I
    lib.backlite_similarity_elems.argtypes = []
    lib.backlite_similarity_elems.restype = Z
    lib.backlite_similarity_sums.argtypes = [P, P, ctypes.c_int64, P, P]
    lib.backlite_similarity_sums.restype = I
    lib.backlite_status_string.argtypes = [I]
    lib.backlite_status_string.restype = ctypes.c_char_p
    lib.backlite_last_error.argtypes = []
    lib.backlite_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def lib():
    return _load()


def _check(rc: int, what: str):
    if rc != 0:
        L = _load()
        raise BackliteError(f"{what} failed: {L.backlite_status_string(rc).decode()} "
                            f"({L.backlite_last_error().decode()})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape=None):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def ntiles(n: int, tile: int = TILE) -> int:
    return (n + tile - 1) // tile


def tile_lse_elems(B, H, n, causal) -> int:
    return int(_load().backlite_tile_lse_elems(B, H, n, 1 if causal else 0))


def tile_w_elems(B, H, n, causal) -> int:
    """fp64 entries of the compact statistics: two per (b, h, tile pair), one per
    64-row half of the query tile."""
    return tile_lse_elems(B, H, n, causal) // 64


def fwd(q, k, v, scale=None, causal=False, with_stats=True, tile_lse=None, with_residual=False, window=0,
        tile_w=None):
    """O, lse_row [B,H,n] fp32, tile_lse (flat fp32 or None); with
    with_residual=True a fourth value, O_lo (bf16 rounding residual of O).
    window > 0 (causal only): key j visible to query i iff i - window < j <= i.
    tile_w: optional flat fp64 tensor of tile_w_elems() that receives the
    compact statistics (one log-weight per tile pair) for mask_compact."""
    B, n, H, d = q.shape
    Hk = k.shape[2]
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, n, Hk, d))
    _need(v, "v", torch.bfloat16, (B, n, Hk, d))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q)
    olo = torch.empty_like(q) if with_residual else None
    lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
    if with_stats and tile_lse is None:
        tile_lse = torch.empty(tile_lse_elems(B, H, n, causal), dtype=torch.float32, device=q.device)
    if tile_lse is not None:
        _need(tile_lse, "tile_lse", torch.float32, (tile_lse_elems(B, H, n, causal),))
    if tile_w is not None:
        _need(tile_w, "tile_w", torch.float64, (tile_w_elems(B, H, n, causal),))
    rc = _load().backlite_fwd(_ptr(q), _ptr(k), _ptr(v), B, n, H, Hk, d, scale, int(causal),
                              int(window), _ptr(o), _ptr(olo), _ptr(lse), _ptr(tile_lse), _ptr(tile_w),
                              _stream(q.device))
    _check(rc, "backlite_fwd")
    if with_residual:
        return o, lse, tile_lse, olo
    return o, lse, tile_lse


def _mask_outputs(B, H, n, q_tile, dev):
    T, Tq = ntiles(n), ntiles(n, q_tile)
    return {
        "keep": torch.empty((B, H, Tq, T), dtype=torch.uint8, device=dev),
        "qcnt": torch.empty((B, H, Tq), dtype=torch.int32, device=dev),
        "qidx": torch.empty((B, H, Tq, T), dtype=torch.int16, device=dev),
        "kcnt": torch.empty((B, H, T), dtype=torch.int32, device=dev),
        "kidx": torch.empty((B, H, T, Tq), dtype=torch.int16, device=dev),
        "q_tile": int(q_tile),
    }


def mask(tile_lse, lse, n, causal, negl_prob, stats=None, window=0, q_tile=TILE):
    """keep [B,H,Tq,T] u8, qcnt [B,H,Tq] i32, qidx [B,H,Tq,T] i16 (uint16 bits),
    kcnt [B,H,T], kidx [B,H,T,Tq], for query tiles of q_tile rows (128 or 64),
    and "q_tile" itself (bwd() reads it)."""
    B, H, nn = lse.shape
    assert nn == n
    _need(lse, "lse", torch.float32)
    if tile_lse is not None:
        _need(tile_lse, "tile_lse", torch.float32, (tile_lse_elems(B, H, n, causal),))
    dev = lse.device
    out = _mask_outputs(B, H, n, q_tile, dev)
    if stats is not None:
        _need(stats, "stats", torch.int64, (2,))
    rc = _load().backlite_mask(_ptr(tile_lse), _ptr(lse), B, H, n, int(causal), int(window), int(q_tile),
                               float(negl_prob), _ptr(out["keep"]), _ptr(out["qcnt"]), _ptr(out["qidx"]),
                               _ptr(out["kcnt"]), _ptr(out["kidx"]), _ptr(stats), _stream(dev))
    _check(rc, "backlite_mask")
    return out


def mask_compact(tile_w, B, H, n, causal, negl_prob, stats=None, window=0, device=None, q_tile=TILE):
    """As mask(), from the compact statistics fwd(..., tile_w=) wrote."""
    dev = tile_w.device if tile_w is not None else device
    if tile_w is not None:
        _need(tile_w, "tile_w", torch.float64, (tile_w_elems(B, H, n, causal),))
    out = _mask_outputs(B, H, n, q_tile, dev)
    if stats is not None:
        _need(stats, "stats", torch.int64, (2,))
    rc = _load().backlite_mask_compact(_ptr(tile_w), B, H, n, int(causal), int(window), int(q_tile),
                                       float(negl_prob), _ptr(out["keep"]), _ptr(out["qcnt"]), _ptr(out["qidx"]),
                                       _ptr(out["kcnt"]), _ptr(out["kidx"]), _ptr(stats), _stream(dev))
    _check(rc, "backlite_mask_compact")
    return out


def bwd_workspace_bytes(B, H, Hk, n, d) -> int:
    return int(_load().backlite_bwd_workspace_bytes(B, H, Hk, n, d))


def bwd_workspace_bytes_stored(B, H, Hk, n, d, max_tiles, q_tile=TILE) -> int:
    return int(_load().backlite_bwd_workspace_bytes_stored(B, H, Hk, n, d, int(q_tile), int(max_tiles)))


def bwd_state_offset(B, H, Hk, n, d) -> int:
    return int(_load().backlite_bwd_state_offset(B, H, Hk, n, d))


def bwd_stored_taken(workspace, B, H, Hk, n, d) -> tuple:
    """(every kept tile had a G_S slot, kept tile pairs) from the state words of
    a workspace the last backward used (synchronises with the device)."""
    w = bwd_state(workspace, B, H, Hk, n, d)
    return w[0], w[1]


def bwd_state(workspace, B, H, Hk, n, d) -> tuple:
    """(all kept tiles had a slot, kept tile pairs, kept tiles with a slot) from
    the state words of a workspace the last backward used (synchronises)."""
    off = bwd_state_offset(B, H, Hk, n, d)
    if workspace.numel() < off + 12:
        raise ValueError("bwd_state: the workspace has no G_S slots (a recompute-only workspace keeps no state words)")
    w = workspace[off:off + 12].view(torch.int32).tolist()
    return bool(w[0]), int(w[1]), int(w[2])


def check_lists(qcnt, qidx, kcnt, kidx, B, H, n, causal, window=0, q_tile=TILE):
    """Validate work lists held in host memory (numpy int32 / uint16 arrays)
    with backlite_check_lists; raises BackliteError with the first violation."""
    import numpy as np
    arrs = [np.ascontiguousarray(qcnt, dtype=np.int32), np.ascontiguousarray(qidx).view(np.uint16),
            np.ascontiguousarray(kcnt, dtype=np.int32), np.ascontiguousarray(kidx).view(np.uint16)]
    msg = ctypes.create_string_buffer(400)
    rc = _load().backlite_check_lists(*[a.ctypes.data_as(ctypes.c_void_p) for a in arrs], B, H, n, int(causal),
                                      int(window), int(q_tile), msg, 400)
    if rc != 0:
        raise BackliteError(f"backlite_check_lists: {msg.value.decode()}")


def candidate_pairs(n: int, causal: bool, window: int = 0, q_tile: int = TILE) -> int:
    """Candidate (query tile, key tile) pairs of one (batch, head): all Tq*T, or
    the causal triangle, or its band under a sliding window (integer bookkeeping
    for workspace sizes)."""
    T, Tq = ntiles(n), ntiles(n, q_tile)
    if not causal:
        return Tq * T
    w = window if 0 < window < n else 0
    tot = 0
    for qt in range(Tq):
        first = qt * q_tile
        last = min(n, first + q_tile) - 1
        lo = (first - w + 1) // TILE if (w and first - w + 1 > 0) else 0
        tot += last // TILE - lo + 1
    return tot


# Default share of device memory given to stored-G_S slots when the caller
# sets no budget.
GS_BUDGET_FRACTION = 1 / 8
def slot_bytes(q_tile: int = TILE) -> int:
    """Bytes of one stored tile: bf16 G_S of q_tile x 128 and 4 x q_tile fp32 sums."""
    return q_tile * TILE * 2 + 4 * q_tile * 4


SLOT_BYTES = slot_bytes(TILE)


def gs_slots_for_budget(B, H, n, causal, window, budget_bytes, device, q_tile=TILE) -> int:
    """Slots for a G_S budget in bytes (None: GS_BUDGET_FRACTION of the device's
    memory), never more than the candidate pairs: no device readback."""
    if budget_bytes is None:
        budget_bytes = int(torch.cuda.get_device_properties(device).total_memory * GS_BUDGET_FRACTION)
    return max(0, min(B * H * candidate_pairs(n, causal, window, q_tile), int(budget_bytes) // slot_bytes(q_tile)))


def bwd_workspace(q, k, lists=None, stored_tiles="auto", causal=False, window=0, gs_budget_bytes=None,
                  q_tile=None) -> torch.Tensor:
    """A backward workspace.  stored_tiles: "auto" gives G_S slots for every
    candidate tile pair, capped by gs_budget_bytes (default: an eighth of the
    device's memory), without reading anything back from the device; an int
    gives that many slots; 0 gives the base workspace (G_Q recomputes P and
    G_S).  When the kept tiles outnumber the slots, the query tiles past the
    slots recompute their G_Q (decided on the device).  q_tile: the lists'
    query-tile rows (default: lists["q_tile"], else 128)."""
    B, n, H, d = q.shape
    Hk = k.shape[2]
    if q_tile is None:
        q_tile = lists.get("q_tile", TILE) if lists is not None else TILE
    base = bwd_workspace_bytes(B, H, Hk, n, d)
    if stored_tiles == "auto":
        tiles = gs_slots_for_budget(B, H, n, causal, window, gs_budget_bytes, q.device, q_tile)
    else:
        tiles = int(stored_tiles or 0)
    size = bwd_workspace_bytes_stored(B, H, Hk, n, d, tiles, q_tile) if tiles > 0 else base
    return torch.empty(size, dtype=torch.uint8, device=q.device)


def _check_lists_shapes(lists, B, H, n) -> int:
    """The lists' query-tile rows (lists["q_tile"], default 128), after checking
    the four arrays' dtypes and shapes."""
    q_tile = int(lists.get("q_tile", TILE))
    T, Tq = ntiles(n), ntiles(n, q_tile)
    _need(lists["qcnt"], "qcnt", torch.int32, (B, H, Tq))
    _need(lists["kcnt"], "kcnt", torch.int32, (B, H, T))
    _need(lists["qidx"], "qidx", torch.int16, (B, H, Tq, T))
    _need(lists["kidx"], "kidx", torch.int16, (B, H, T, Tq))
    return q_tile


def bwd(q, k, v, o, do, lse, lists, scale=None, causal=False, workspace=None, out=None, o_lo=None,
        stored_tiles="auto", window=0):
    """G_Q, G_K, G_V (bf16) for the tile set in `lists` (qcnt/qidx/kcnt/kidx).
    o_lo: the forward's residual output (recommended; D then uses O + O_lo).
    workspace: reused if given (a larger one enables the stored-G_S path);
    otherwise one is allocated by bwd_workspace(stored_tiles=...), which reads
    nothing back from the device."""
    B, n, H, d = q.shape
    Hk = k.shape[2]
    for name, t, shp in (("q", q, (B, n, H, d)), ("k", k, (B, n, Hk, d)), ("v", v, (B, n, Hk, d)),
                         ("o", o, (B, n, H, d)), ("do", do, (B, n, H, d))):
        _need(t, name, torch.bfloat16, shp)
    _need(lse, "lse", torch.float32, (B, H, n))
    if o_lo is not None:
        _need(o_lo, "o_lo", torch.bfloat16, (B, n, H, d))
    q_tile = _check_lists_shapes(lists, B, H, n)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
    if workspace is None:
        workspace = bwd_workspace(q, k, lists, stored_tiles, causal=causal, window=window)
    rc = _load().backlite_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(o_lo), _ptr(do), _ptr(lse),
                              _ptr(lists["qcnt"]), _ptr(lists["qidx"]), _ptr(lists["kcnt"]),
                              _ptr(lists["kidx"]), B, n, H, Hk, d, scale, int(causal),
                              int(window), q_tile, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                              _stream(q.device))
    _check(rc, "backlite_bwd")
    return dq, dk, dv


def similarity_sums(a, b, out=None):
    """Device fp64 tensor whose first 4 entries become (sum a*b, sum a*a,
    sum b*b, sum (a-b)^2) of two bf16 tensors of equal size (the rest is the
    kernel's scratch)."""
    _need(a, "a", torch.bfloat16)
    _need(b, "b", torch.bfloat16, tuple(a.shape))
    if out is None:
        out = torch.empty(int(_load().backlite_similarity_elems()), dtype=torch.float64, device=a.device)
    _check(_load().backlite_similarity_sums(_ptr(a), _ptr(b), a.numel(), _ptr(out), _stream(a.device)),
           "backlite_similarity_sums")
    return out


def bwd_atomic_workspace(q, k) -> torch.Tensor:
    B, n, H, d = q.shape
    nb = int(_load().backlite_bwd_atomic_workspace_bytes(B, H, k.shape[2], n, d))
    return torch.empty(nb, dtype=torch.uint8, device=q.device)


def bwd_atomic(q, k, v, o, do, lse, lists, scale=None, causal=False, workspace=None, out=None, o_lo=None, window=0):
    """The fused single-pass backward with an fp32-atomic G_Q (backlite_bwd_atomic);
    128-row query tiles only."""
    B, n, H, d = q.shape
    Hk = k.shape[2]
    for name, t, shp in (("q", q, (B, n, H, d)), ("k", k, (B, n, Hk, d)), ("v", v, (B, n, Hk, d)),
                         ("o", o, (B, n, H, d)), ("do", do, (B, n, H, d))):
        _need(t, name, torch.bfloat16, shp)
    _need(lse, "lse", torch.float32, (B, H, n))
    if _check_lists_shapes(lists, B, H, n) != TILE:
        raise ValueError("the atomic G_Q backward takes 128-row query tiles")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq, dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    if workspace is None:
        workspace = bwd_atomic_workspace(q, k)
    rc = _load().backlite_bwd_atomic(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(o_lo), _ptr(do), _ptr(lse),
                                     _ptr(lists["qcnt"]), _ptr(lists["qidx"]), _ptr(lists["kcnt"]),
                                     _ptr(lists["kidx"]), B, n, H, Hk, d, scale, int(causal), int(window),
                                     _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                                     _stream(q.device))
    _check(rc, "backlite_bwd_atomic")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, do, lse, lists, out, scale=None, causal=False, o_lo=None, window=0):
    """The allocation-free backward (backlite_bwd_noalloc): the library's fixed
    per-GPU scratch serves as workspace and the caller supplies the outputs
    out = (dq, dk, dv); nothing is allocated by this call."""
    B, n, H, d = q.shape
    Hk = k.shape[2]
    for name, t, shp in (("q", q, (B, n, H, d)), ("k", k, (B, n, Hk, d)), ("v", v, (B, n, Hk, d)),
                         ("o", o, (B, n, H, d)), ("do", do, (B, n, H, d))):
        _need(t, name, torch.bfloat16, shp)
    _need(lse, "lse", torch.float32, (B, H, n))
    if o_lo is not None:
        _need(o_lo, "o_lo", torch.bfloat16, (B, n, H, d))
    dq, dk, dv = out
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _need(t, name, torch.bfloat16, tuple(ref.shape))
    q_tile = _check_lists_shapes(lists, B, H, n)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rc = _load().backlite_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(o_lo), _ptr(do), _ptr(lse),
                                      _ptr(lists["qcnt"]), _ptr(lists["qidx"]), _ptr(lists["kcnt"]),
                                      _ptr(lists["kidx"]), B, n, H, Hk, d, scale, int(causal), int(window),
                                      q_tile, _ptr(dq), _ptr(dk), _ptr(dv), _stream(q.device))
    _check(rc, "backlite_bwd_noalloc")
    return dq, dk, dv


PROFILE_KERNELS = ("fwd", "mask_select", "mask_transpose", "delta", "kmean", "dk_plan", "dkdv", "dk_reduce", "dq",
                   "gs_slots")


def profile_enable(on: bool = True):
    _check(_load().backlite_profile_enable(1 if on else 0), "backlite_profile_enable")


def profile_reset():
    _check(_load().backlite_profile_reset(), "backlite_profile_reset")


def profile_read() -> dict:
    """{kernel: (total_ms, launches)} accumulated since the last reset."""
    out = {}
    L = _load()
    for k in PROFILE_KERNELS:
        ms, cnt = ctypes.c_double(0.0), ctypes.c_int64(0)
        _check(L.backlite_profile_read(k.encode(), ctypes.byref(ms), ctypes.byref(cnt)), "backlite_profile_read")
        out[k] = (ms.value, cnt.value)
    return out
