"""Sliding-window attention (causal, key j visible to query i iff
i - window < j <= i): parity of the HIP forward, mask and backward with the
fp64 oracle on small seeded cases.  Windows narrower than a tile, windows that
cut tiles in the middle, ragged tails, GQA and both head sizes.  GPU only."""
import numpy as np
import pytest
import torch

from helpers import (assert_close_grad, assert_close_out, check_lists, excused_mismatches,
                     flush_print, gpu_available, lists_to_torch, packed_to_rows, rows_to_packed)
from oracle import backlite_oracle as orc
from workloads import make_inputs, small

pytestmark = pytest.mark.gpu

# (workload, window)
CASES = [
    (small(1000, H=4, Hk=2, d=128, causal=True, kind="blocks", seed=11), 300),
    (small(700, H=2, Hk=1, d=64, causal=True, kind="gaussian", seed=12), 128),
    (small(513, H=2, d=128, causal=True, kind="gaussian", seed=13), 1),
    (small(900, H=2, Hk=1, d=64, causal=True, kind="positional", seed=14, period=256.0), 200),
    (small(300, H=2, d=64, causal=True, kind="gaussian", seed=15), 1000),   # window >= n: plain causal
]
IDS = [f"{w.name}-w{win}" for w, win in CASES]
NEGL = 0.05

_cache = {}


def _setup(case):
    w, win = case
    key = (w.name, win)
    if key in _cache:
        return _cache[key]
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    flush_print(f"[case] {w.name} window={win}")
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    xg = {k: v.to(dev) for k, v in x.items()}
    ref = orc.forward(x["q"], x["k"], x["v"], causal=True, window=win)
    o, lse, tl, olo = bl.fwd(xg["q"], xg["k"], xg["v"], causal=True, with_residual=True, window=win)
    torch.cuda.synchronize()
    r = dict(w=w, win=win, x=x, xg=xg, ref=ref, o=o, olo=olo, lse=lse, tl=tl, bl=bl, dev=dev)
    _cache[key] = r
    return r


def _cand_rows(n, win):
    """[n, T] bool: row i's tile is a candidate of key tile kt."""
    cand = orc.candidates(n, True, window=win)
    return cand[np.arange(n) // 128]


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_window_forward_outputs(case):
    r = _setup(case)
    assert_close_out("O", r["o"].cpu(), r["ref"]["O"])
    assert_close_out("lse", r["lse"].cpu(), r["ref"]["lse"])


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_window_forward_tile_lse(case):
    """Candidate tiles only: the layout keeps the causal triangle and pairs
    outside the window are never written."""
    r = _setup(case)
    w, win = r["w"], r["win"]
    B, H, n = w.B, w.H, w.n
    got = packed_to_rows(r["tl"].cpu().numpy(), B, H, n, True)
    ref = r["ref"]["tile_lse"]
    cr = np.broadcast_to(_cand_rows(n, win), got.shape)
    lse = r["ref"]["lse"][..., None]
    sel = cr & np.isfinite(ref) & (ref - lse > -60.0)
    assert_close_out("tile_lse", got[sel], ref[sel])
    # a row of a candidate tile that sees none of its keys gets exactly -inf
    assert not np.isnan(got[cr]).any()
    assert (got[cr & ~np.isfinite(ref)] == -np.inf).all()
    # logsumexp over the candidate tiles of the GPU's own output = lse_row
    g = np.where(cr & np.isfinite(got), got, -np.inf)
    m = g.max(-1, keepdims=True)
    lse_tiles = (m + np.log(np.exp(g - m).sum(-1, keepdims=True)))[..., 0]
    np.testing.assert_allclose(lse_tiles, r["lse"].cpu().numpy(), atol=2e-5, rtol=0)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_window_mask_same_inputs_bit_exact(case):
    r = _setup(case)
    w, win, bl, dev = r["w"], r["win"], r["bl"], r["dev"]
    B, H, n = w.B, w.H, w.n
    tl32 = rows_to_packed(r["ref"]["tile_lse"], B, H, n, True)
    lse32 = r["ref"]["lse"].astype(np.float32)
    for negl in (0.0, 0.01, NEGL, 0.3):
        m = bl.mask(torch.from_numpy(tl32).to(dev), torch.from_numpy(lse32).to(dev), n, True, negl, window=win)
        keep_ref = orc.mask_from_stats(packed_to_rows(tl32, B, H, n, True), lse32, n, True,
                                       np.float64(np.float32(negl)), window=win)
        check_lists(m, keep_ref)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_window_mask_end_to_end(case):
    r = _setup(case)
    w, win, bl = r["w"], r["win"], r["bl"]
    n = w.n
    cand = orc.candidates(n, True, window=win)
    a_ref = orc.tile_log_weights(r["ref"]["tile_lse"], r["ref"]["lse"], n, True, window=win)
    for negl in (0.01, NEGL):
        m = bl.mask(r["tl"], r["lse"], n, True, negl, window=win)
        keep_ref = orc.select_keep(a_ref, cand, negl)
        keep = m["keep"].cpu().numpy().astype(bool)
        bad, exc = excused_mismatches(keep, keep_ref, a_ref, cand, negl)
        flush_print(f"  negl={negl}: kept {keep.sum()}/{keep_ref.sum()} ref, excused {len(exc)}")
        assert not bad, f"unexcused mask mismatches {bad[:5]}"
        check_lists(m, keep)


def _check_grad(name, got, ref):
    """assert_close_grad, except for an all-zero reference: with window = 1
    every row's softmax is one-hot on its own key, so G_S = P * (G_P - D) = 0
    and G_Q = G_K = 0 exactly; the GPU's bf16 O and D leave only rounding
    residue there, checked in absolute terms."""
    if not np.any(orc.to_f64(ref)):
        ma = float(np.abs(orc.to_f64(got)).max())
        assert ma <= 1e-3, f"{name}: max-abs {ma:.3e} against an exactly zero gradient"
        return ma, 1.0
    return assert_close_grad(name, got, ref)


def _bwd(r, lists, path):
    bl, xg, w = r["bl"], r["xg"], r["w"]
    ws = bl._lib.bwd_workspace(xg["q"], xg["k"], lists, stored_tiles=0 if path == "recompute" else "auto")
    out = bl.bwd(xg["q"], xg["k"], xg["v"], r["o"], xg["do"], r["lse"], lists, causal=True,
                 o_lo=r["olo"], workspace=ws, window=r["win"])
    if path == "stored":
        taken, kept = bl._lib.bwd_stored_taken(ws, w.B, w.H, w.Hk, w.n, w.d)
        assert taken and kept == int(lists["qcnt"].sum().item())
    return out


@pytest.mark.parametrize("path", ("recompute", "stored"))
@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_window_backward_on_oracle_mask(case, path):
    r = _setup(case)
    w, win, x = r["w"], r["win"], r["x"]
    keep = orc.mask_from_stats(r["ref"]["tile_lse"], r["ref"]["lse"], w.n, True, NEGL, window=win)
    dq, dk, dv = _bwd(r, lists_to_torch(keep, r["dev"]), path)
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=True, window=win)
    for name, got, ref in (("dQ", dq, g["dQ"]), ("dK", dk, g["dK"]), ("dV", dv, g["dV"])):
        rl, cs = _check_grad(name, got.cpu(), ref)
        flush_print(f"  {path} {name}: rel-L2 {rl:.2e} cos {cs:.6f}")


@pytest.mark.parametrize("path", ("recompute", "stored"))
@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_window_backward_dense(case, path):
    """negl_prob = 0: the lists hold every candidate of the window."""
    r = _setup(case)
    w, win, x, bl = r["w"], r["win"], r["x"], r["bl"]
    m = bl.mask(None, r["lse"], w.n, True, 0.0, window=win)
    T = m["keep"].shape[-1]
    check_lists(m, np.broadcast_to(orc.candidates(w.n, True, window=win), (w.B, w.H, T, T)))
    dq, dk, dv = _bwd(r, m, path)
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], causal=True, window=win)
    for name, got, ref in (("dQ", dq, g["dQ"]), ("dK", dk, g["dK"]), ("dV", dv, g["dV"])):
        _check_grad(name, got.cpu(), ref)


def test_window_module_autograd():
    """The autograd module with a window, dense backward, against the oracle."""
    w, win = CASES[1]
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev).requires_grad_(True) for n in ("q", "k", "v"))
    attn = bl.BackLite(negl_prob=0.0, causal=True, window=win)
    o = attn(q, k, v)
    o.backward(x["do"].to(dev))
    ref = orc.forward(x["q"], x["k"], x["v"], causal=True, window=win)
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], causal=True, window=win)
    assert_close_out("O", o.detach().cpu(), ref["O"])
    for name, t in (("dQ", q), ("dK", k), ("dV", v)):
        assert_close_grad(name, t.grad.cpu(), g[name])


def test_window_requires_causal():
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    with pytest.raises(ValueError):
        bl.BackLite(causal=False, window=64)
    q = torch.zeros((1, 128, 1, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(bl.BackliteError):
        bl.fwd(q, q, q, causal=False, window=64)


@pytest.mark.parametrize("n,win", [(131072, 2048), (65536, 300), (20000, 129)])
def test_window_dense_mask_many_tiles(n, win):
    """negl_prob = 0 with a window on sequences of many tiles: the keep bitmap is
    exactly the window's candidate set (the candidate range then starts far from
    tile 0, so the flags are set by other threads than those that cleared them)."""
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    lse = torch.zeros((1, 2, n), dtype=torch.float32, device="cuda:0")
    m = bl.mask(None, lse, n, True, 0.0, window=win)
    T = m["keep"].shape[-1]
    check_lists(m, np.broadcast_to(orc.candidates(n, True, window=win), (1, 2, T, T)))
