"""Plain fp64 CPU oracle for BackLite's forward / mask / sparse-backward path.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
bench's CPU-baseline leg may import or run this module; the product path never
does, and this module imports nothing from the GPU package.

It computes, slowly and directly, what the pages define:

* Attention forward S = scale*Q K^T, P = row-softmax(S), O = P V, with the row
  log-sum-exp kept for the backward ("Introducing BackLite", section
  "Backpropagation for attention", forward equations; safe softmax with the
  row maximum subtracted, FlashAttention tutorial, "Safe Softmax Algorithm").
* A log-sum-exp per (query row, key tile) recorded by the forward, and the tile
  probability p_tile = exp(LSE_tile - LSE_row) (BackLite README, "How It Works /
  Sparse Backward Masking", phases 1 and 2).
* The tile weight of a (query tile, key tile) pair = the maximum of p_tile over
  the valid rows of the query tile (our reading: the blog's "sum of P over the
  tile" and the README's per-tile LSE are both aggregations of the same
  per-row numbers; the max is the conservative one, since it bounds every row's
  neglected mass).
* For each query tile, the smallest-weight key tiles whose cumulative weight
  stays strictly below negl_prob are skipped ("Introducing BackLite", "Using
  Sparsity"; README "Overview" and "Usage": cumulative weight < negl_prob).
* The backward G_V = P^T G_O, G_P = G_O V^T, D = rowsum(G_O * O),
  G_S = P * (G_P - D), G_Q = scale G_S K, G_K = scale G_S^T Q ("Introducing
  BackLite", backward equations; D as the row sum, FlashAttention tutorial,
  "Flash Attention Backward Pass"), with every skipped tile's entries of P and
  G_S set to zero ("Using Sparsity": the mask on P carries over to G_S).

Readings where the pages are silent (each also listed in the design notes):
natural-log LSEs; strict "<"; ties among equal weights broken by the lower key
tile index first; the order is taken on the exact exponent a = log(w) (equal
a <=> equal w); prefix sums are sequential fp64 adds in sorted order; causally
empty tiles are not candidates; padded rows/columns of a ragged last tile never
enter any sum or maximum; D uses the full (unmasked) output row.

Layouts: Q, O, G_O, G_Q are [B, n, H, d]; K, V, G_K, G_V are [B, n, Hk, d];
LSE is [B, H, n]; the oracle's tile LSE is [B, H, n, T] (row-major by query
row), T = ceil(n / tile).  Query head h reads kv head h // (H // Hk).
"""
from __future__ import annotations

import numpy as np

TILE = 128


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def to_f64(x) -> np.ndarray:
    """bf16/fp32 torch tensor or numpy array -> float64 numpy (exact upcast)."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # local: only to convert torch inputs
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def ntiles(n: int, tile: int = TILE) -> int:
    return (n + tile - 1) // tile


def kv_head(h: int, H: int, Hk: int) -> int:
    return h // (H // Hk)


def candidates(n: int, causal: bool, tile: int = TILE, window: int = 0, q_tile: int | None = None) -> np.ndarray:
    """cand[qt, kt]: the key tile holds at least one (i, j) with i, j < n that the
    causal rule (j <= i) allows.  Causally empty tiles are never candidates.

    window > 0 (causal only): a sliding window of `window` keys, key j visible to
    query i iff i - window < j <= i (our reading of the blog's Nanochat windows of
    1024 / 2048 tokens, "Training Nanochat").  A tile pair is then a candidate iff
    its first key is <= its last row and its last key is > its first row - window.

    q_tile: rows per query tile (default: tile).  The BackLite README forms the
    mask "for each backward tile pair" ("How It Works / Sparse Backward
    Masking"), and a backward's query tiles may be smaller than the forward's key
    tiles; the result is then [ceil(n / q_tile), ceil(n / tile)].
    """
    q_tile = tile if q_tile is None else q_tile
    Tq, Tk = ntiles(n, q_tile), ntiles(n, tile)
    qt = np.arange(Tq)[:, None]
    kt = np.arange(Tk)[None, :]
    i_lo, i_hi = qt * q_tile, np.minimum(n, (qt + 1) * q_tile) - 1
    k_lo, k_hi = kt * tile, np.minimum(n, (kt + 1) * tile) - 1
    if window:
        assert causal, "a sliding window is causal"
        return (k_lo <= i_hi) & (k_hi > i_lo - window)
    if causal:
        return np.broadcast_to(k_lo <= i_hi, (Tq, Tk)).copy()   # first key <= last row
    return np.ones((Tq, Tk), bool)


def _score_block(qh, kh, rows, scale, causal, window=0):
    """S for query rows `rows` against all keys, -inf where causally masked
    (and, with a sliding window, where j <= i - window)."""
    S = scale * (qh[rows] @ kh.T)
    if causal:
        j = np.arange(kh.shape[0])[None, :]
        ok = j <= rows[:, None]
        if window:
            ok &= j > rows[:, None] - window
        S = np.where(ok, S, -np.inf)
    return S


def _row_lse(S):
    """Safe log-sum-exp per row: m + log(sum exp(S - m))."""
    m = S.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(S - m).sum(axis=1, keepdims=True)))[:, 0]


def _tile_lse(S, n, tile):
    """log-sum-exp of S over each key tile's columns; -inf if none is finite."""
    T = ntiles(n, tile)
    pad = np.full((S.shape[0], T * tile), -np.inf)
    pad[:, :n] = S
    Z = pad.reshape(S.shape[0], T, tile)
    m = Z.max(axis=2)
    fin = np.isfinite(m)
    msafe = np.where(fin, m, 0.0)
    with np.errstate(divide="ignore"):
        s = np.log(np.exp(Z - msafe[:, :, None]).sum(axis=2))
    return np.where(fin, msafe + s, -np.inf)


# ----------------------------------------------------------------------------
# forward with per-(row, key tile) statistics
# ----------------------------------------------------------------------------
def forward(q, k, v, scale=None, causal=False, tile=TILE, heads=None, rows=None, block=128, window=0):
    """Exact attention forward plus tile statistics.

    Returns dict with O [B, nr, H', d], lse [B, H', nr], tile_lse [B, H', nr, T]
    where nr = len(rows) (all rows by default) and H' = len(heads).
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, n, H, d = q.shape
    Hk = k.shape[2]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    heads = list(range(H)) if heads is None else list(heads)
    rows = np.arange(n) if rows is None else np.asarray(rows)
    T = ntiles(n, tile)
    O = np.zeros((B, len(rows), len(heads), d))
    lse = np.zeros((B, len(heads), len(rows)))
    tl = np.zeros((B, len(heads), len(rows), T))
    for b in range(B):
        for hi, h in enumerate(heads):
            g = kv_head(h, H, Hk)
            qh, kh, vh = q[b, :, h], k[b, :, g], v[b, :, g]
            for s in range(0, len(rows), block):
                r = rows[s:s + block]
                S = _score_block(qh, kh, r, scale, causal, window)
                L = _row_lse(S)
                P = np.exp(S - L[:, None])
                O[b, s:s + block, hi] = P @ vh
                lse[b, hi, s:s + block] = L
                tl[b, hi, s:s + block] = _tile_lse(S, n, tile)
    return {"O": O, "lse": lse, "tile_lse": tl}


# ----------------------------------------------------------------------------
# mask from statistics
# ----------------------------------------------------------------------------
def tile_log_weights(tile_lse, lse, n, causal, tile=TILE, window=0, q_tile=None):
    """a[b, h, qt, kt] = max over valid rows i of the query tile of
    (LSE_tile[i, kt] - LSE_row[i]), in fp64; the tile weight is w = exp(a)
    (README phase 2: p_tile = exp(LSE_tile - LSE_row)).  -inf off-candidate.

    tile_lse: [B, H, n, T] (fp32 or fp64 values); lse: [B, H, n].  The query
    tiles have q_tile rows (default: tile), so a is [B, H, ceil(n/q_tile), T].
    """
    q_tile = tile if q_tile is None else q_tile
    tl = np.asarray(tile_lse, dtype=np.float64)
    ls = np.asarray(lse, dtype=np.float64)
    B, H, nn, T = tl.shape
    assert nn == n
    Tq = ntiles(n, q_tile)
    diff = tl - ls[..., None]
    pad = np.full((B, H, Tq * q_tile, T), -np.inf)
    pad[:, :, :n] = diff
    a = pad.reshape(B, H, Tq, q_tile, T).max(axis=3)
    cand = candidates(n, causal, tile, window, q_tile)
    return np.where(cand[None, None], a, -np.inf)


def select_keep(a, cand, negl_prob):
    """keep[b, h, qt, kt] from log-weights a.

    Per query tile: order the candidate key tiles by (a ascending, kt ascending),
    form sequential fp64 prefix sums c_r of w = exp(a) in that order, and skip
    position r iff c_r < negl_prob.  Weights are >= 0 so the skipped set is a
    prefix of the order.  Everything else among the candidates is kept.
    """
    a = np.asarray(a, dtype=np.float64)
    B, H, Tq, Tk = a.shape
    keep = np.zeros((B, H, Tq, Tk), bool)
    for b in range(B):
        for h in range(H):
            for qt in range(Tq):
                idx = np.nonzero(cand[qt])[0]
                if idx.size == 0:
                    continue
                av = a[b, h, qt, idx]
                order = np.lexsort((idx, av))          # primary a, then kt
                c = np.add.accumulate(np.exp(av[order]))  # sequential left-to-right
                skipped = idx[order][c < negl_prob]
                kp = np.ones(idx.size, bool)
                kp[np.isin(idx, skipped)] = False
                keep[b, h, qt, idx[kp]] = True
    return keep


def mask_from_stats(tile_lse, lse, n, causal, negl_prob, tile=TILE, window=0, q_tile=None):
    a = tile_log_weights(tile_lse, lse, n, causal, tile, window, q_tile)
    cand = candidates(n, causal, tile, window, q_tile)
    return select_keep(a, cand, negl_prob)


def lists_from_keep(keep):
    """Compacted work lists.  q-list(qt) = kept kt ascending; k-list(kt) = kept
    qt ascending.  Returns (qcnt [B,H,Tq], qidx [B,H,Tq,Tk], kcnt [B,H,Tk],
    kidx [B,H,Tk,Tq]); rows of qidx/kidx hold the list in their first cnt
    entries and zeros after."""
    keep = np.asarray(keep, bool)
    B, H, Tq, Tk = keep.shape
    qcnt = keep.sum(axis=3).astype(np.int32)
    kcnt = keep.sum(axis=2).astype(np.int32)
    qidx = np.zeros((B, H, Tq, Tk), np.uint16)
    kidx = np.zeros((B, H, Tk, Tq), np.uint16)
    for b in range(B):
        for h in range(H):
            for t in range(Tq):
                r = np.nonzero(keep[b, h, t])[0]
                qidx[b, h, t, :r.size] = r
            for t in range(Tk):
                c = np.nonzero(keep[b, h, :, t])[0]
                kidx[b, h, t, :c.size] = c
    return qcnt, qidx, kcnt, kidx


# ----------------------------------------------------------------------------
# D and the (masked) backward
# ----------------------------------------------------------------------------
def delta(do, o):
    """D[b, h, i] = sum_c G_O[b, i, h, c] * O[b, i, h, c]."""
    do, o = to_f64(do), to_f64(o)
    return np.einsum("bihc,bihc->bhi", do, o)


def backward(q, k, v, do, keep=None, scale=None, causal=False, tile=TILE,
             heads=None, q_rows=None, window=0, q_tile=None):
    """Masked attention backward in fp64.

    keep: [B, H, Tq, T] bool tile mask over *all* heads (None = every candidate);
    its query tiles have q_tile rows (default: tile), its key tiles tile keys.
    heads: restrict to these query heads (G_K/G_V then sum over those heads only).
    q_rows: restrict the query rows that contribute (G_Q is returned for those
    rows only; G_K/G_V then hold only those rows' contributions).
    Returns dict dQ [B, nr, H', d], dK, dV [B, n, Hk, d], plus O, lse, D.
    """
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    B, n, H, d = q.shape
    Hk = k.shape[2]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    heads = list(range(H)) if heads is None else list(heads)
    rows = np.arange(n) if q_rows is None else np.asarray(q_rows)
    q_tile = tile if q_tile is None else q_tile
    cand = candidates(n, causal, tile, window, q_tile)
    dQ = np.zeros((B, len(rows), len(heads), d))
    dK = np.zeros((B, n, Hk, d))
    dV = np.zeros((B, n, Hk, d))
    Oall = np.zeros((B, len(rows), len(heads), d))
    Lall = np.zeros((B, len(heads), len(rows)))
    Dall = np.zeros((B, len(heads), len(rows)))
    kt_of_col = np.arange(n) // tile
    for b in range(B):
        for hi, h in enumerate(heads):
            g = kv_head(h, H, Hk)
            qh, kh, vh, doh = q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h]
            km = cand if keep is None else np.asarray(keep[b, h], bool)
            for s in range(0, len(rows), tile):
                r = rows[s:s + tile]
                S = _score_block(qh, kh, r, scale, causal, window)
                L = _row_lse(S)
                P = np.exp(S - L[:, None])
                O = P @ vh
                D = (doh[r] * O).sum(axis=1)           # full-row D
                M = km[(r // q_tile)[:, None], kt_of_col[None, :]]
                Ph = np.where(M, P, 0.0)
                dP = doh[r] @ vh.T
                dS = Ph * (dP - D[:, None])
                dQ[b, s:s + tile, hi] = scale * (dS @ kh)
                dK[b, :, g] += scale * (dS.T @ qh[r])
                dV[b, :, g] += Ph.T @ doh[r]
                Oall[b, s:s + tile, hi] = O
                Lall[b, hi, s:s + tile] = L
                Dall[b, hi, s:s + tile] = D
    return {"dQ": dQ, "dK": dK, "dV": dV, "O": Oall, "lse": Lall, "D": Dall}


# ----------------------------------------------------------------------------
# comparison metrics (rel-L2 and cosine on the flattened tensors)
# ----------------------------------------------------------------------------
def rel_l2(a, ref):
    a, ref = to_f64(a).ravel(), to_f64(ref).ravel()
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / (den if den > 0 else 1.0))


def cosine(a, ref):
    a, ref = to_f64(a).ravel(), to_f64(ref).ravel()
    na, nr = np.linalg.norm(a), np.linalg.norm(ref)
    if na == 0 and nr == 0:
        return 1.0
    return float(a @ ref / (na * nr))


# ----------------------------------------------------------------------------
# sampled evaluation for long sequences
# ----------------------------------------------------------------------------
def sampled_head_group(q, k, v, do, heads, negl_prob, causal=False, q_tiles=(), k_tiles=(),
                       scale=None, tile=TILE, block=TILE, all_rows=True, stats=None, window=0, threads=1,
                       q_tile=None):
    """The same definitions as forward / mask_from_stats / backward, evaluated
    for one group of query heads sharing a kv head, but only for selected
    outputs, so that long sequences stay tractable on the CPU.

    For every query head h in `heads` (all must read the same kv head):
      * pass 1, over every row when all_rows (else over the rows of q_tiles
        only): row LSE, tile LSE and D = rowsum(G_O * O);
      * the tile mask of the head from those statistics (rows of the query
        tiles pass 1 did not visit stay all-False);
      * O and G_Q of the rows of `q_tiles`;
      * the head's contribution to G_K, G_V of the key rows of `k_tiles`
        (requires all_rows), summed over `heads`.
    `stats` (the "stats" entry of a previous call with the same inputs) skips
    pass 1, e.g. to evaluate several negl_prob values.  `window` is the sliding
    window of `candidates` / `forward` (causal only).  `threads` > 1 runs the
    query tiles of pass 1 on that many threads (each tile's arithmetic is the
    same; numpy releases the interpreter lock inside its array operations).
    `q_tile`: rows per query tile of the mask (default: tile); q_tiles and
    k_tiles stay in units of `tile` rows / keys, and out["keep"] is
    [ceil(n / q_tile), T].
    """
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    B, n, H, d = q.shape
    Hk = k.shape[2]
    assert B == 1, "sampled evaluation takes one sequence"
    assert all_rows or not k_tiles, "key-tile gradients need every row's statistics"
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    g = kv_head(heads[0], H, Hk)
    assert all(kv_head(h, H, Hk) == g for h in heads)
    T = ntiles(n, tile)
    q_tile = tile if q_tile is None else q_tile
    assert tile % q_tile == 0, "query tiles subdivide the statistics' row blocks"
    cand = candidates(n, causal, tile, window, q_tile)
    kh, vh = k[0, :, g], v[0, :, g]
    q_tiles, k_tiles = list(q_tiles), list(k_tiles)
    out = {"keep": [], "lse": [], "tile_lse": [], "D": [], "O": [], "dQ": [], "stats": []}
    dK = {kt: np.zeros((min(n, (kt + 1) * tile) - kt * tile, d)) for kt in k_tiles}
    dV = {kt: np.zeros_like(dK[kt]) for kt in k_tiles}
    p1_tiles = range(T) if all_rows else sorted(set(q_tiles))
    for hi, h in enumerate(heads):
        qh, doh = q[0, :, h], do[0, :, h]
        if stats is None:
            # pass 1: row statistics over the full key range
            L = np.full(n, np.nan)
            TL = np.full((n, T), -np.inf)
            Dr = np.full(n, np.nan)
            Oq = {}

            def pass1(qt):
                r = np.arange(qt * tile, min(n, (qt + 1) * tile))
                S = _score_block(qh, kh, r, scale, causal, window)
                L[r] = _row_lse(S)
                TL[r] = _tile_lse(S, n, tile)
                O = np.exp(S - L[r][:, None]) @ vh
                Dr[r] = (doh[r] * O).sum(axis=1)
                if qt in q_tiles:
                    Oq[qt] = O

            if threads > 1:
                from concurrent.futures import ThreadPoolExecutor

                from threadpoolctl import threadpool_limits
                with threadpool_limits(1), ThreadPoolExecutor(threads) as ex:  # one BLAS thread per tile
                    list(ex.map(pass1, p1_tiles))
            else:
                for qt in p1_tiles:
                    pass1(qt)
            st = {"L": L, "TL": TL, "D": Dr, "O": Oq}
        else:
            st = stats[hi]
        L, TL, Dr, Oq = st["L"], st["TL"], st["D"], st["O"]
        out["stats"].append(st)
        # mask of the visited query tiles
        a = tile_log_weights(np.where(np.isfinite(TL), TL, -np.inf)[None, None],
                             np.where(np.isfinite(L), L, 0.0)[None, None], n, causal, tile, window, q_tile)
        cv = cand.copy()
        visited = np.zeros(T, bool)
        visited[list(p1_tiles)] = True
        cv[~np.repeat(visited, tile // q_tile)[:cv.shape[0]]] = False
        kp = select_keep(a, cv, negl_prob)[0, 0]
        out["keep"].append(kp)
        out["lse"].append(L)
        out["tile_lse"].append(TL)
        out["D"].append(Dr)
        out["O"].append([Oq[qt] for qt in q_tiles])
        # pass 2: G_Q rows of q_tiles, G_K/G_V contributions to k_tiles
        for qt in q_tiles:
            r = np.arange(qt * tile, min(n, (qt + 1) * tile))
            S = _score_block(qh, kh, r, scale, causal, window)
            P = np.exp(S - L[r][:, None])
            M = kp[(r // q_tile)[:, None], (np.arange(n) // tile)[None, :]]
            dS = np.where(M, P, 0.0) * (doh[r] @ vh.T - Dr[r][:, None])
            out["dQ"].append((h, qt, scale * (dS @ kh)))
        for kt in k_tiles:
            c = np.arange(kt * tile, min(n, (kt + 1) * tile))
            for qt in np.nonzero(kp[:, kt])[0]:
                r = np.arange(qt * q_tile, min(n, (qt + 1) * q_tile))
                Sc = scale * (qh[r] @ kh[c].T)
                if causal:
                    ok = c[None, :] <= r[:, None]
                    if window:
                        ok &= c[None, :] > r[:, None] - window
                    Sc = np.where(ok, Sc, -np.inf)
                Pc = np.exp(Sc - L[r][:, None])
                dSc = Pc * (doh[r] @ vh[c].T - Dr[r][:, None])
                dK[kt] += scale * (dSc.T @ qh[r])
                dV[kt] += Pc.T @ doh[r]
    out["dK"] = dK
    out["dV"] = dV
    return out


# ----------------------------------------------------------------------------
# negl_prob calibration
# ----------------------------------------------------------------------------
GRADS = ("dQ", "dK", "dV")


def gradient_agreement(g, ref):
    """(cosine, rel-L2) of each of G_Q, G_K, G_V against the reference
    gradients: the two similarity metrics the blog compares BackLite's
    gradients with exact FlashAttention's by ("Introducing BackLite",
    "Experiments")."""
    return {nm: (cosine(g[nm], ref[nm]), rel_l2(g[nm], ref[nm])) for nm in GRADS}


def within_targets(agree, cos_min, rel_max):
    """Every gradient has cosine > cos_min and rel-L2 < rel_max (the blog's
    calibration targets are strict: cosine similarity > 0.99, relative L2
    difference < 0.1; "Preliminary results with Wan 2.1 1.3b", Fig. 4)."""
    return all(c > cos_min and r < rel_max for c, r in agree.values())


def calibrate(q, k, v, do, causal=False, scale=None, cos_min=0.99, rel_max=0.1, pi_max=0.5, iters=8,
              tile=TILE, window=0):
    """The largest negl_prob in [0, pi_max] (to the bisection's resolution) whose
    masked gradients stay within the targets of the dense (negl_prob = 0) ones.

    The pages describe a tool that picks the neglected weight to meet a minimum
    cosine similarity and a maximum relative L2 difference ("Introducing
    BackLite", "Preliminary results with Wan 2.1 1.3b"; README "Overview",
    Tunable).  They do not give its search; this reading bisects, which relies
    on the keep sets shrinking as negl_prob grows: pi_max is tried first, then
    `iters` halvings of [lo, hi] with lo always within the targets (lo = 0 is
    the dense backward itself).

    Returns negl_prob (the last value within the targets), upper (the smallest
    value tried that was not, or pi_max), its keep mask, the gradient agreement
    and the sparsity (1 - kept / candidate tile pairs), plus every probe
    (negl_prob, within) in order.  `window`: a sliding window (causal only),
    as in `candidates`; the dense reference then has the same window.
    """
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    B, n, H, _ = q.shape
    f = forward(q, k, v, scale=scale, causal=causal, tile=tile, window=window)
    dense = backward(q, k, v, do, keep=None, scale=scale, causal=causal, tile=tile, window=window)
    cand = candidates(n, causal, tile, window)
    ncand = B * H * int(cand.sum())

    def probe(pi):
        keep = mask_from_stats(f["tile_lse"], f["lse"], n, causal, pi, tile, window)
        g = backward(q, k, v, do, keep=keep, scale=scale, causal=causal, tile=tile, window=window)
        agree = gradient_agreement(g, dense)
        return within_targets(agree, cos_min, rel_max), keep, agree

    probes = []
    ok, keep, agree = probe(pi_max)
    probes.append((pi_max, ok))
    if ok:
        return dict(negl_prob=pi_max, upper=pi_max, keep=keep, agreement=agree,
                    sparsity=1.0 - keep.sum() / ncand, probes=probes)
    lo, hi = 0.0, pi_max
    best_keep = np.broadcast_to(cand, (B, H) + cand.shape).copy()
    best_agree = gradient_agreement(dense, dense)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        ok, keep, agree = probe(mid)
        probes.append((mid, ok))
        if ok:
            lo, best_keep, best_agree = mid, keep, agree
        else:
            hi = mid
    return dict(negl_prob=lo, upper=hi, keep=best_keep, agreement=best_agree,
                sparsity=1.0 - best_keep.sum() / ncand, probes=probes)
