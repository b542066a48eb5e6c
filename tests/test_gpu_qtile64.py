"""Half-height (64-row) backward query tiles: the README forms the mask "for
each backward tile pair" ("How It Works / Sparse Backward Masking"), and the
backward's tiles need not match the forward's 128-row ones.  The per-row tile
statistics are aggregated over 64 rows instead of 128, the lists hold 64-row
query tiles against 128-key tiles, and all three backward passes work on
them.  Parity against the oracle's masks and gradients with q_tile = 64, on
small cases and sampled at full size.  GPU only."""
import numpy as np
import pytest
import torch

from helpers import (assert_close_grad, check_lists, excused_mismatches, flush_print, gpu_available,
                     lists_to_torch, packed_to_rows, rows_to_packed)
from oracle import backlite_oracle as orc
from workloads import DIT480, LLM128K, TINY, make_inputs, small

pytestmark = pytest.mark.gpu

Q = 64
NEGL = 0.05
CASES = [
    TINY,
    small(1000, H=4, Hk=2, d=128, causal=True, kind="blocks", seed=1),
    small(300, H=2, Hk=1, d=64, causal=False, kind="gaussian", seed=2),
    small(129, H=1, d=128, causal=True, kind="gaussian", seed=3),
    small(1, H=2, Hk=1, d=64, causal=False, seed=4),
    small(640, H=2, d=128, causal=False, kind="blocks", B=2, seed=5),
    small(383, H=3, Hk=1, d=128, causal=False, kind="gaussian", seed=6),
]
IDS = [w.name for w in CASES]
PATHS = ("recompute", "stored")
_cache = {}


def _setup(w, window=0):
    key = (w.name, window)
    if key in _cache:
        return _cache[key]
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    flush_print(f"[case] {w.name} window={window} q_tile={Q}")
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    xg = {k: v.to(dev) for k, v in x.items()}
    ref = orc.forward(x["q"], x["k"], x["v"], causal=w.causal, window=window)
    o, lse, tl, olo = bl.fwd(xg["q"], xg["k"], xg["v"], causal=w.causal, with_residual=True, window=window)
    torch.cuda.synchronize()
    r = dict(w=w, x=x, xg=xg, ref=ref, o=o, olo=olo, lse=lse, tl=tl, bl=bl, dev=dev, win=window)
    _cache[key] = r
    return r


def _bwd(r, lists, path):
    bl, xg, w = r["bl"], r["xg"], r["w"]
    ws = bl._lib.bwd_workspace(xg["q"], xg["k"], lists, stored_tiles=0 if path == "recompute" else "auto",
                               causal=w.causal, window=r["win"])
    out = bl.bwd(xg["q"], xg["k"], xg["v"], r["o"], xg["do"], r["lse"], lists, causal=w.causal, o_lo=r["olo"],
                 workspace=ws, window=r["win"])
    if path == "stored":
        taken, kept = bl._lib.bwd_stored_taken(ws, w.B, w.H, w.Hk, w.n, w.d)
        assert taken and kept == int(lists["qcnt"].sum().item())
    return out


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_mask_q64_same_inputs_bit_exact(w):
    """The oracle's statistics rounded to fp32 into the library's mask with
    64-row query tiles: keep bitmap and lists equal the oracle's selection."""
    r = _setup(w)
    bl, dev = r["bl"], r["dev"]
    B, H, n = w.B, w.H, w.n
    tl32 = rows_to_packed(r["ref"]["tile_lse"], B, H, n, w.causal)
    lse32 = r["ref"]["lse"].astype(np.float32)
    for negl in (0.0, 0.01, NEGL, 0.3, 0.9):
        m = bl.mask(torch.from_numpy(tl32).to(dev), torch.from_numpy(lse32).to(dev), n, w.causal, negl, q_tile=Q)
        keep_ref = orc.mask_from_stats(packed_to_rows(tl32, B, H, n, w.causal), lse32, n, w.causal,
                                       np.float64(np.float32(negl)), q_tile=Q)
        check_lists(m, keep_ref)


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_mask_q64_end_to_end(w):
    r = _setup(w)
    bl, n = r["bl"], w.n
    cand = orc.candidates(n, w.causal, q_tile=Q)
    a_ref = orc.tile_log_weights(r["ref"]["tile_lse"], r["ref"]["lse"], n, w.causal, q_tile=Q)
    for negl in (0.01, NEGL, 0.1):
        m = bl.mask(r["tl"], r["lse"], n, w.causal, negl, q_tile=Q)
        keep_ref = orc.select_keep(a_ref, cand, negl)
        keep = m["keep"].cpu().numpy().astype(bool)
        bad, exc = excused_mismatches(keep, keep_ref, a_ref, cand, negl)
        assert not bad, f"unexcused mask mismatches {bad[:5]}"
        check_lists(m, keep)
        # never less sparse than the 128-row mask: each half keeps at most what its tile keeps
        m128 = bl.mask(r["tl"], r["lse"], n, w.causal, negl)
        assert int(m["qcnt"].sum()) <= 2 * int(m128["qcnt"].sum())
        flush_print(f"  negl={negl}: kept {keep.sum()} (64-row) vs {int(m128['qcnt'].sum())} (128-row), "
                    f"excused {len(exc)}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_backward_q64_on_oracle_mask(w, path):
    r = _setup(w)
    x = r["x"]
    keep = orc.mask_from_stats(r["ref"]["tile_lse"], r["ref"]["lse"], w.n, w.causal, NEGL, q_tile=Q)
    lists = lists_to_torch(keep, r["dev"], q_tile=Q)
    dq, dk, dv = _bwd(r, lists, path)
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=w.causal, q_tile=Q)
    for name, got, ref in (("dQ", dq, g["dQ"]), ("dK", dk, g["dK"]), ("dV", dv, g["dV"])):
        rl, cs = assert_close_grad(name, got.cpu(), ref)
        flush_print(f"  {path} {name}: rel-L2 {rl:.2e} cos {cs:.6f}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("w", [CASES[1], CASES[2], CASES[6]], ids=[IDS[1], IDS[2], IDS[6]])
def test_backward_q64_dense_equals_dense(w, path):
    """negl_prob = 0 with 64-row query tiles keeps every candidate: the dense
    gradients, as with 128-row tiles."""
    r = _setup(w)
    x = r["x"]
    m = r["bl"].mask(None, r["lse"], w.n, w.causal, 0.0, q_tile=Q)
    check_lists(m, np.broadcast_to(orc.candidates(w.n, w.causal, q_tile=Q), (w.B, w.H) + m["keep"].shape[-2:]))
    dq, dk, dv = _bwd(r, m, path)
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], causal=w.causal)
    for name, got, ref in (("dQ", dq, g["dQ"]), ("dK", dk, g["dK"]), ("dV", dv, g["dV"])):
        assert_close_grad(name, got.cpu(), ref)


@pytest.mark.parametrize("w", [CASES[1], CASES[2], CASES[6]], ids=[IDS[1], IDS[2], IDS[6]])
def test_q64_stored_matches_recompute_and_repeats(w):
    r = _setup(w)
    m = r["bl"].mask(r["tl"], r["lse"], w.n, w.causal, NEGL, q_tile=Q)
    a = _bwd(r, m, "recompute")
    b = _bwd(r, m, "stored")
    b2 = _bwd(r, m, "stored")
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))
    assert torch.equal(a[2].view(torch.int16), b[2].view(torch.int16))
    for u, v in zip(b, b2):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))
    rl = orc.rel_l2(b[0].cpu(), orc.to_f64(a[0].cpu()))
    flush_print(f"  dQ stored vs recompute rel-L2 {rl:.2e}")
    assert rl <= 2e-3


@pytest.mark.parametrize("frac", [0.3, 0.9])
def test_q64_slot_budget(frac):
    """Fewer slots than kept 64-row tiles: a prefix of the query tiles takes G_Q
    from stored G_S, the rest is recomputed (per 64-row half inside the
    recompute pass's 128-row workgroups); matches the oracle."""
    w = CASES[1]
    r = _setup(w)
    bl, x, xg = r["bl"], r["x"], r["xg"]
    keep = orc.mask_from_stats(r["ref"]["tile_lse"], r["ref"]["lse"], w.n, w.causal, NEGL, q_tile=Q)
    m = lists_to_torch(keep, r["dev"], q_tile=Q)
    qcnt = m["qcnt"].cpu().numpy().reshape(-1)
    slots = max(1, int(frac * qcnt.sum()))
    ws = bl._lib.bwd_workspace(xg["q"], xg["k"], m, stored_tiles=slots)
    a = bl.bwd(xg["q"], xg["k"], xg["v"], r["o"], xg["do"], r["lse"], m, causal=True, o_lo=r["olo"], workspace=ws)
    all_in, counted, slotted = bl._lib.bwd_state(ws, w.B, w.H, w.Hk, w.n, w.d)
    assert not all_in and counted == int(qcnt.sum()) and slotted == slots
    b = _bwd(r, m, "recompute")
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))
    stored = (np.cumsum(qcnt) <= slots).reshape(w.B, w.H, -1)
    ga, gb = a[0].cpu(), b[0].cpu()
    for h in range(w.H):
        for qt in range(stored.shape[-1]):
            rows = slice(qt * Q, min(w.n, qt * Q + Q))
            if not stored[0, h, qt]:
                assert torch.equal(ga[0, rows, h].view(torch.int16), gb[0, rows, h].view(torch.int16))
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=w.causal, q_tile=Q)
    for name, got, ref in (("dQ", a[0], g["dQ"]), ("dK", a[1], g["dK"]), ("dV", a[2], g["dV"])):
        assert_close_grad(name, got.cpu(), ref)


SINK = small(1536, H=4, Hk=1, d=64, causal=True, kind="positional", seed=9, period=512.0)


@pytest.mark.parametrize("path", PATHS)
def test_backward_q64_split_lists(path, monkeypatch):
    """Attention sinks with 64-row query tiles: the sink key tile's list (every
    64-row tile of every head) is split over workgroups."""
    w = SINK
    r = _setup(w)
    x = r["x"]
    keep = orc.mask_from_stats(r["ref"]["tile_lse"], r["ref"]["lse"], w.n, w.causal, NEGL, q_tile=Q)
    lists = lists_to_torch(keep, r["dev"], q_tile=Q)
    monkeypatch.setenv("BACKLITE_DKDV_MIN_CHUNK", "16")
    dq, dk, dv = _bwd(r, lists, path)
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=w.causal, q_tile=Q)
    for name, got, ref in (("dQ", dq, g["dQ"]), ("dK", dk, g["dK"]), ("dV", dv, g["dV"])):
        rl, cs = assert_close_grad(name, got.cpu(), ref)
        flush_print(f"  split {path} {name}: rel-L2 {rl:.2e}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("win", [300, 128])
def test_backward_q64_window(win, path):
    w = small(1000, H=4, Hk=2, d=128, causal=True, kind="blocks", seed=1)
    r = _setup(w, window=win)
    x = r["x"]
    keep = orc.mask_from_stats(r["ref"]["tile_lse"], r["ref"]["lse"], w.n, True, NEGL, window=win, q_tile=Q)
    m = r["bl"].mask(r["tl"], r["lse"], w.n, True, NEGL, window=win, q_tile=Q)
    a_ref = orc.tile_log_weights(r["ref"]["tile_lse"], r["ref"]["lse"], w.n, True, window=win, q_tile=Q)
    bad, exc = excused_mismatches(m["keep"].cpu().numpy().astype(bool), keep, a_ref,
                                  orc.candidates(w.n, True, window=win, q_tile=Q), NEGL)
    assert not bad
    dq, dk, dv = _bwd(r, lists_to_torch(keep, r["dev"], q_tile=Q), path)
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=True, window=win, q_tile=Q)
    for name, got, ref in (("dQ", dq, g["dQ"]), ("dK", dk, g["dK"]), ("dV", dv, g["dV"])):
        assert_close_grad(name, got.cpu(), ref)


def test_module_q64_matches_oracle():
    """BackLite(q_tile=64): forward + loss.backward() against the oracle."""
    w = small(500, H=4, Hk=2, d=128, causal=True, kind="blocks", seed=7)
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (x[nm].to(dev).requires_grad_() for nm in ("q", "k", "v"))
    attn = bl.BackLite(negl_prob=NEGL, causal=True, q_tile=Q)
    attn(q, k, v).backward(x["do"].to(dev))
    ref = orc.forward(x["q"], x["k"], x["v"], causal=True)
    keep = orc.mask_from_stats(ref["tile_lse"], ref["lse"], w.n, True, NEGL, q_tile=Q)
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=True, q_tile=Q)
    for name, got, rr in (("dQ", q.grad, g["dQ"]), ("dK", k.grad, g["dK"]), ("dV", v.grad, g["dV"])):
        assert_close_grad(name, got.cpu(), rr)


@pytest.mark.parametrize("w,heads,q_tiles,k_tiles,win", [
    (DIT480, [0], [0, 128, 255], [0, 128, 255], 0),
    (LLM128K, [0], [0, 511, 1023], [0, 511, 1023], 0),
], ids=["dit-480p-32k", "llm-128k-causal"])
def test_full_size_q64(w, heads, q_tiles, k_tiles, win):
    """Full size, in the bench's launch configuration, with 64-row query tiles:
    the sampled head's whole mask against the oracle's, G_Q rows of sampled
    128-row blocks and G_K/G_V of sampled key tiles, on both G_Q paths."""
    if not gpu_available():
        pytest.skip("no GPU")
    import os
    import block_sparse_attention_fa_amd as bl
    flush_print(f"[case] {w.name} q_tile={Q}")
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    xg = {k_: v_.to(dev) for k_, v_ in x.items()}
    B, H, Hk, n, causal = w.B, w.H, w.Hk, w.n, w.causal
    o, lse, tl, olo = bl.fwd(xg["q"], xg["k"], xg["v"], causal=causal, with_residual=True, window=win)
    negl = next(p for p in w.negl_probs if p > 0)   # the workload's sparse setting
    m = bl.mask(tl, lse, n, causal, negl, window=win, q_tile=Q)
    m128 = bl.mask(tl, lse, n, causal, negl, window=win)
    g = orc.kv_head(heads[0], H, Hk)
    sl = {nm: x[nm][:, :, heads] for nm in ("q", "do")}
    sl.update({nm: x[nm][:, :, g:g + 1] for nm in ("k", "v")})
    ref = orc.sampled_head_group(sl["q"], sl["k"], sl["v"], sl["do"], list(range(len(heads))), negl, causal,
                                 q_tiles=q_tiles, k_tiles=k_tiles, all_rows=True, window=win, q_tile=Q,
                                 threads=max(1, min(16, len(os.sched_getaffinity(0)))))
    keep_all = m["keep"].cpu().numpy().astype(bool)
    kg, kr = keep_all[0, heads[0]], ref["keep"][0]
    L, TL = ref["lse"][0], ref["tile_lse"][0]
    a = orc.tile_log_weights(TL[None, None], L[None, None], n, causal, window=win, q_tile=Q)
    bad, exc = excused_mismatches(kg[None, None], kr[None, None], a, orc.candidates(n, causal, window=win, q_tile=Q),
                                  negl)
    assert not bad, bad[:5]
    cand = orc.candidates(n, causal, window=win, q_tile=Q)
    sp64 = 1 - keep_all.sum() / (cand.sum() * B * H)
    sp128 = 1 - int(m128["qcnt"].sum()) / (orc.candidates(n, causal, window=win).sum() * B * H)
    flush_print(f"  negl={negl}: sparsity {sp64:.4f} with 64-row query tiles, {sp128:.4f} with 128-row ones; "
                f"kept work {int(m['qcnt'].sum()) / 2:.0f} vs {int(m128['qcnt'].sum())} 128x128 tiles; "
                f"excused {len(exc)}")
    assert sp64 >= sp128
    for path in PATHS:
        ws = bl._lib.bwd_workspace(xg["q"], xg["k"], m, stored_tiles=0 if path == "recompute" else "auto",
                                   causal=causal, window=win)
        dq, dk, dv = bl.bwd(xg["q"], xg["k"], xg["v"], o, xg["do"], lse, m, causal=causal, o_lo=olo, window=win,
                            workspace=ws)
        torch.cuda.synchronize()
        G, R = [], []
        for (hi, qt, dqr) in ref["dQ"]:
            rows = slice(qt * 128, min(n, qt * 128 + 128))
            if (keep_all[0, heads[hi], 2 * qt:2 * qt + 2] == kr[2 * qt:2 * qt + 2]).all():
                G.append(orc.to_f64(dq[0, rows, heads[hi]].cpu()))
                R.append(dqr)
        assert G
        rl, cs = assert_close_grad("dQ", np.concatenate(G), np.concatenate(R))
        GK, RK, GV, RV = [], [], [], []
        for kt in k_tiles:
            if (keep_all[0, heads[0], :, kt] == kr[:, kt]).all():
                rows = slice(kt * 128, min(n, kt * 128 + 128))
                GK.append(orc.to_f64(dk[0, rows, g].cpu()))
                RK.append(ref["dK"][kt])
                GV.append(orc.to_f64(dv[0, rows, g].cpu()))
                RV.append(ref["dV"][kt])
        assert GK
        rk, _ = assert_close_grad("dK", np.concatenate(GK), np.concatenate(RK))
        rv, _ = assert_close_grad("dV", np.concatenate(GV), np.concatenate(RV))
        flush_print(f"  {path}: dQ rel-L2 {rl:.2e}, dK {rk:.2e}, dV {rv:.2e}")
        del ws
