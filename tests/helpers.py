"""Shared helpers for the parity tests: layout conversion between the library's
packed tile-LSE buffer and the oracle's [B, H, n, T] view, mask comparison with
the documented excuses, and tolerances."""
from __future__ import annotations

import numpy as np
import torch

from oracle import backlite_oracle as orc

TILE = 128
# acceptance bounds: O/LSE max-abs 2e-2 and rel-L2 1e-2; gradients rel-L2 1e-2
# and cosine 0.999 against the oracle on the same mask
O_MAXABS, O_REL = 2e-2, 1e-2
G_REL, G_COS = 1e-2, 0.999
THRESH_EXCUSE = 1e-6


def gpu_available() -> bool:
    try:
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def pair_index(qt, kt, T, causal):
    return qt * (qt + 1) // 2 + kt if causal else qt * T + kt


def packed_to_rows(flat, B, H, n, causal):
    """library tile-LSE layout -> [B, H, n, T] fp64 (non-candidates -inf)."""
    T = (n + TILE - 1) // TILE
    pairs = T * (T + 1) // 2 if causal else T * T
    a = np.asarray(flat, dtype=np.float64).reshape(B, H, pairs, TILE)
    out = np.full((B, H, T * TILE, T), -np.inf)
    for qt in range(T):
        for kt in range(qt + 1 if causal else T):
            out[:, :, qt * TILE:(qt + 1) * TILE, kt] = a[:, :, pair_index(qt, kt, T, causal), :]
    return out[:, :, :n]


def rows_to_packed(rows, B, H, n, causal):
    """[B, H, n, T] -> library layout (rows >= n set to -inf), float32."""
    T = (n + TILE - 1) // TILE
    pairs = T * (T + 1) // 2 if causal else T * T
    full = np.full((B, H, T * TILE, T), -np.inf)
    full[:, :, :n] = rows
    out = np.empty((B, H, pairs, TILE), np.float32)
    for qt in range(T):
        for kt in range(qt + 1 if causal else T):
            out[:, :, pair_index(qt, kt, T, causal), :] = full[:, :, qt * TILE:(qt + 1) * TILE, kt]
    return out.reshape(-1)


def lists_to_torch(keep, device, q_tile=TILE):
    qcnt, qidx, kcnt, kidx = orc.lists_from_keep(keep)
    return {
        "qcnt": torch.from_numpy(qcnt).to(device),
        "qidx": torch.from_numpy(qidx.view(np.int16)).to(device),
        "kcnt": torch.from_numpy(kcnt).to(device),
        "kidx": torch.from_numpy(kidx.view(np.int16)).to(device),
        "q_tile": q_tile,
    }


def check_lists(m, keep_ref):
    """The library's lists must equal the ones derived from keep_ref."""
    keep = m["keep"].cpu().numpy().astype(bool)
    assert (keep == keep_ref).all()
    qcnt, qidx, kcnt, kidx = orc.lists_from_keep(keep_ref)
    gq = m["qcnt"].cpu().numpy()
    gk = m["kcnt"].cpu().numpy()
    assert (gq == qcnt).all() and (gk == kcnt).all()
    gqi = m["qidx"].cpu().numpy().view(np.uint16)
    gki = m["kidx"].cpu().numpy().view(np.uint16)
    B, H, Tq, Tk = keep_ref.shape
    for b in range(B):
        for h in range(H):
            for t in range(Tq):
                assert (gqi[b, h, t, :qcnt[b, h, t]] == qidx[b, h, t, :qcnt[b, h, t]]).all()
            for t in range(Tk):
                assert (gki[b, h, t, :kcnt[b, h, t]] == kidx[b, h, t, :kcnt[b, h, t]]).all()


def excused_mismatches(keep_gpu, keep_ref, a_ref, cand, negl):
    """Tiles where the GPU mask differs from the oracle's.  Returns (bad, excused):
    a mismatch is excused when, in the oracle's own order, the tile's prefix sum
    lies within 1e-6 of negl_prob, or its weight is within 1e-6 (relative to the
    row's largest weight) of a weight on the other side of the cut."""
    diff = np.argwhere(keep_gpu != keep_ref)
    bad, exc = [], []
    for b, h, qt, kt in diff:
        idx = np.nonzero(cand[qt])[0]
        av = a_ref[b, h, qt, idx]
        order = np.lexsort((idx, av))
        w = np.exp(av[order])
        c = np.add.accumulate(w)
        pos = int(np.nonzero(idx[order] == kt)[0][0])
        near_cut = abs(c[pos] - negl) <= THRESH_EXCUSE
        kept_ref = keep_ref[b, h, qt, idx[order]]
        other = w[kept_ref != keep_ref[b, h, qt, kt]]
        near_tie = other.size > 0 and np.min(np.abs(other - w[pos])) <= THRESH_EXCUSE * w.max()
        (exc if (near_cut or near_tie) else bad).append((int(b), int(h), int(qt), int(kt)))
    return bad, exc


def assert_close_out(name, got, ref, maxabs=O_MAXABS, rel=O_REL):
    g = orc.to_f64(got)
    r = orc.to_f64(ref)
    ma = float(np.max(np.abs(g - r))) if g.size else 0.0
    rl = orc.rel_l2(g, r)
    assert ma <= maxabs and rl <= rel, f"{name}: max-abs {ma:.3e} (<= {maxabs}), rel-L2 {rl:.3e} (<= {rel})"
    return ma, rl


def assert_close_grad(name, got, ref):
    rl = orc.rel_l2(got, ref)
    cs = orc.cosine(got, ref)
    assert rl <= G_REL and cs >= G_COS, f"{name}: rel-L2 {rl:.3e} (<= {G_REL}), cosine {cs:.6f} (>= {G_COS})"
    return rl, cs


def flush_print(*a):
    print(*a, flush=True)

