"""Parity at the full workload sizes, in the launch configuration the bench
times: the 8k causal GQA LLM, the 32k and 75k video-DiT grids and the 128k
causal LLM, and the two LLM shapes with sliding windows of 1024 and 2048 keys.  The oracle evaluates sampled heads and tiles (rows of sampled
query tiles: forward outputs, mask rows, G_Q; columns of sampled key tiles:
G_K, G_V, where every row's statistics are affordable); properties that hold
at any size are checked on every head.  GPU only."""
import os
import time

import numpy as np
import pytest
import torch

from helpers import (TILE, assert_close_grad, assert_close_out, excused_mismatches, flush_print,
                     gpu_available, pair_index)
from oracle import backlite_oracle as orc
from workloads import DIT480, DIT720, LLM8K, LLM128K, make_inputs

pytestmark = pytest.mark.gpu

# host threads for the oracle's row statistics (16: the CPU share of a one-GPU host)
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))

LARGE = {
    # GQA: the whole group of kv head 0 (query heads 0-3), every row
    "llm-8k-causal-gqa": dict(w=LLM8K, heads=[0, 1, 2, 3], q_tiles=[0, 31, 63], k_tiles=[0, 1, 31, 62, 63],
                              all_rows=True),
    "dit-480p-32k": dict(w=DIT480, heads=[0], q_tiles=[0, 128, 255], k_tiles=[0, 128, 255], all_rows=True),
    "dit-720p-75k": dict(w=DIT720, heads=[0], q_tiles=[0, 295, 590], k_tiles=[0, 295, 590], all_rows=True),
    # key tile 0 holds the attention sinks: every query tile keeps it, so its
    # G_K/G_V list is split over many workgroups and summed by the reduction
    "llm-128k-causal": dict(w=LLM128K, heads=[0], q_tiles=[0, 511, 1023], k_tiles=[0, 511, 1023],
                            all_rows=True),
    "llm-8k-causal-gqa-window1024": dict(w=LLM8K, heads=[0, 1, 2, 3], q_tiles=[0, 8, 31, 63],
                                         k_tiles=[0, 1, 31, 62, 63], all_rows=True, window=1024),
    "llm-128k-causal-window2048": dict(w=LLM128K, heads=[0], q_tiles=[0, 15, 16, 511, 1023],
                                       k_tiles=[0, 1, 511, 1023], all_rows=True, window=2048),
}


def _tile_rows(tl, B, H, n, causal, h, qt):
    """GPU tile-LSE rows of query tile qt of head h -> [rows, T] (-inf off-candidate)."""
    T = (n + TILE - 1) // TILE
    pairs = T * (T + 1) // 2 if causal else T * T
    nk = qt + 1 if causal else T
    base = (h * pairs + pair_index(qt, 0, T, causal)) * TILE
    blk = tl[base: base + nk * TILE].view(nk, TILE).t().cpu().numpy().astype(np.float64)
    out = np.full((TILE, T), -np.inf)
    out[:, :nk] = blk
    return out[: min(TILE, n - qt * TILE)]


@pytest.mark.parametrize("name", list(LARGE))
def test_full_size(name):
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    cfg = LARGE[name]
    w = cfg["w"]
    B, H, Hk, n, d, causal = w.B, w.H, w.Hk, w.n, w.d, w.causal
    T = (n + TILE - 1) // TILE
    heads, q_tiles, k_tiles = cfg["heads"], cfg["q_tiles"], cfg["k_tiles"]
    win = cfg.get("window", 0)
    flush_print(f"[case] {name}: B={B} H={H} Hk={Hk} n={n} d={d} causal={causal} window={win}")
    t0 = time.time()
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    xg = {k_: v_.to(dev) for k_, v_ in x.items()}
    o, lse, tl, olo = bl.fwd(xg["q"], xg["k"], xg["v"], causal=causal, with_residual=True, window=win)
    torch.cuda.synchronize()
    flush_print(f"  inputs + forward {time.time() - t0:.1f} s")

    g = orc.kv_head(heads[0], H, Hk)
    sl = {nm: x[nm][:, :, heads] for nm in ("q", "do")}
    sl.update({nm: x[nm][:, :, g:g + 1] for nm in ("k", "v")})
    hidx = list(range(len(heads)))
    stats = None
    for negl in w.negl_probs:
        t1 = time.time()
        m = bl.mask(tl if negl > 0 else None, lse, n, causal, negl, window=win)
        dq, dk, dv = bl.bwd(xg["q"], xg["k"], xg["v"], o, xg["do"], lse, m, causal=causal, o_lo=olo, window=win)
        torch.cuda.synchronize()
        ref = orc.sampled_head_group(sl["q"], sl["k"], sl["v"], sl["do"], hidx, negl, causal,
                                     q_tiles=q_tiles, k_tiles=k_tiles, all_rows=cfg["all_rows"], stats=stats,
                                     window=win, threads=ORACLE_THREADS)
        first = stats is None
        stats = ref["stats"]
        keep_all = m["keep"].cpu().numpy().astype(bool)
        # ---- properties on every head: lists agree with the bitmap, every query
        # tile keeps at least one key tile, causal pairs above the diagonal absent
        qcnt, kcnt = m["qcnt"].cpu().numpy(), m["kcnt"].cpu().numpy()
        assert (qcnt == keep_all.sum(axis=3)).all() and (kcnt == keep_all.sum(axis=2)).all()
        assert qcnt.min() >= 1
        cand = orc.candidates(n, causal, window=win)
        assert not (keep_all & ~cand).any()      # causal (and window) non-candidates are never kept
        cand_total = cand.sum() * B * H
        flush_print(f"  negl={negl}: sparsity {1 - keep_all.sum() / cand_total:.4f}")
        # ---- forward rows (once)
        if first:
            Og, Or, Lg, Lr, TLg, TLr = [], [], [], [], [], []
            for hi, h in enumerate(heads):
                for j, qt in enumerate(q_tiles):
                    r = slice(qt * TILE, min(n, (qt + 1) * TILE))
                    Og.append(orc.to_f64(o[0, r, h].cpu()))
                    Or.append(ref["O"][hi][j])
                    Lg.append(lse[0, h, r].cpu().numpy())
                    Lr.append(ref["lse"][hi][r])
                    got = _tile_rows(tl, B, H, n, causal, h, qt)
                    want = ref["tile_lse"][hi][r]
                    sel = np.isfinite(want) & (want - ref["lse"][hi][r][:, None] > -60.0)
                    TLg.append(got[sel])
                    TLr.append(want[sel])
            assert_close_out("O", np.concatenate(Og), np.concatenate(Or))
            assert_close_out("lse", np.concatenate(Lg), np.concatenate(Lr))
            assert_close_out("tile_lse", np.concatenate(TLg), np.concatenate(TLr))
        # ---- mask of the sampled heads
        visited = np.arange(T) if cfg["all_rows"] else np.array(sorted(set(q_tiles)))
        nexc = 0
        for hi, h in enumerate(heads):
            kg = keep_all[0, h]
            kr = ref["keep"][hi]
            if negl == 0:
                assert (kg == cand).all()
                continue
            L = ref["lse"][hi]
            TL = ref["tile_lse"][hi]
            a = orc.tile_log_weights(np.where(np.isfinite(TL), TL, -np.inf)[None, None],
                                     np.where(np.isfinite(L), L, 0.0)[None, None], n, causal, window=win)
            bad, exc = excused_mismatches(kg[visited][None, None], kr[visited][None, None],
                                          a[:, :, visited], cand[visited], negl)
            assert not bad, f"head {h}: unexcused mask mismatches {bad[:5]}"
            nexc += len(exc)
        # ---- G_Q rows of sampled query tiles (where both masks agree on the row)
        G, R = [], []
        for (hi, qt, dqr) in ref["dQ"]:
            h = heads[hi]
            if not (keep_all[0, h, qt] == ref["keep"][hi][qt]).all():
                continue
            r = slice(qt * TILE, min(n, (qt + 1) * TILE))
            G.append(orc.to_f64(dq[0, r, h].cpu()))
            R.append(dqr)
        assert G, "no comparable G_Q rows"
        rl, cs = assert_close_grad("dQ", np.concatenate(G), np.concatenate(R))
        msg = f"    dQ rel-L2 {rl:.2e} cos {cs:.6f}"
        # ---- G_K, G_V rows of sampled key tiles
        if k_tiles:
            GK, RK, GV, RV = [], [], [], []
            for kt in k_tiles:
                if not all((keep_all[0, h, :, kt] == ref["keep"][hi][:, kt]).all() for hi, h in enumerate(heads)):
                    continue
                r = slice(kt * TILE, min(n, (kt + 1) * TILE))
                GK.append(orc.to_f64(dk[0, r, g].cpu()))
                RK.append(ref["dK"][kt])
                GV.append(orc.to_f64(dv[0, r, g].cpu()))
                RV.append(ref["dV"][kt])
            assert GK, "no comparable G_K/G_V rows"
            rk, ck = assert_close_grad("dK", np.concatenate(GK), np.concatenate(RK))
            rv, cv = assert_close_grad("dV", np.concatenate(GV), np.concatenate(RV))
            msg += f"  dK rel-L2 {rk:.2e} cos {ck:.6f}  dV rel-L2 {rv:.2e} cos {cv:.6f}"
        flush_print(msg + f"  (excused mask tiles {nexc}, {time.time() - t1:.1f} s)")
