"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on small
seeded cases that span several tiles, ragged tails, causal masking, GQA, both
head sizes and batch > 1.  GPU only."""
import numpy as np
import pytest
import torch

from helpers import (assert_close_grad, assert_close_out, check_lists, excused_mismatches,
                     flush_print, gpu_available, lists_to_torch, packed_to_rows, rows_to_packed)
from oracle import backlite_oracle as orc
from workloads import TINY, make_inputs, small

pytestmark = pytest.mark.gpu

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
NEGL = 0.05

_cache = {}


def _setup(w):
    if w.name in _cache:
        return _cache[w.name]
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    flush_print(f"[case] {w.name}")
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    xg = {k: v.to(dev) for k, v in x.items()}
    ref = orc.forward(x["q"], x["k"], x["v"], causal=w.causal)
    o, lse, tl, olo = bl.fwd(xg["q"], xg["k"], xg["v"], causal=w.causal, with_residual=True)
    torch.cuda.synchronize()
    r = dict(w=w, x=x, xg=xg, ref=ref, o=o, olo=olo, lse=lse, tl=tl, bl=bl, dev=dev)
    _cache[w.name] = r
    return r


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_forward_outputs(w):
    r = _setup(w)
    assert_close_out("O", r["o"].cpu(), r["ref"]["O"])
    assert_close_out("lse", r["lse"].cpu(), r["ref"]["lse"])
    # O_lo is the rounding residual of the fp32 output: at most half a bf16 ulp
    # of O, and O + O_lo is closer to the exact output than O alone
    o1 = orc.to_f64(r["o"].cpu())
    lo = orc.to_f64(r["olo"].cpu())
    half_ulp = np.where(o1 != 0, 2.0 ** (np.floor(np.log2(np.abs(np.where(o1 != 0, o1, 1.0)))) - 8), 2.0 ** -133)
    assert (np.abs(lo) <= half_ulp).all()
    if w.n > 1:
        assert orc.rel_l2(o1 + lo, r["ref"]["O"]) < orc.rel_l2(o1, r["ref"]["O"])


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_forward_tile_lse(w):
    r = _setup(w)
    B, H, n = w.B, w.H, w.n
    got = packed_to_rows(r["tl"].cpu().numpy(), B, H, n, w.causal)
    ref = r["ref"]["tile_lse"]
    cand = orc.candidates(n, w.causal)
    T = cand.shape[0]
    # compare where the tile carries non-negligible probability (fp32 range)
    lse = r["ref"]["lse"][..., None]
    sel = np.isfinite(ref) & (ref - lse > -60.0)
    assert_close_out("tile_lse", got[sel], ref[sel])
    # every row of a candidate tile sees at least one key: no NaN anywhere
    rows = np.arange(n)
    for kt in range(T):
        c = cand[rows // 128, kt]
        assert not np.isnan(got[:, :, c, kt]).any()
    # identity on the GPU's own output: logsumexp_kt tile_lse = lse_row
    g = np.where(np.isfinite(got), got, -np.inf)
    m = g.max(-1, keepdims=True)
    lse_tiles = (m + np.log(np.exp(g - m).sum(-1, keepdims=True)))[..., 0]
    np.testing.assert_allclose(lse_tiles, r["lse"].cpu().numpy(), atol=2e-5, rtol=0)


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_mask_same_inputs_bit_exact(w):
    """Selection logic alone: the oracle's tile statistics, rounded to fp32, go
    into the library's mask call; keep bitmap and lists must equal the oracle's
    selection on those same fp32 values, bit for bit."""
    r = _setup(w)
    bl, dev = r["bl"], r["dev"]
    B, H, n = w.B, w.H, w.n
    tl32 = rows_to_packed(r["ref"]["tile_lse"], B, H, n, w.causal)
    lse32 = r["ref"]["lse"].astype(np.float32)
    for negl in (0.0, 0.01, NEGL, 0.3, 0.9):
        m = bl.mask(torch.from_numpy(tl32).to(dev), torch.from_numpy(lse32).to(dev), n, w.causal, negl)
        keep_ref = orc.mask_from_stats(packed_to_rows(tl32, B, H, n, w.causal), lse32, n, w.causal,
                                       np.float64(np.float32(negl)))
        check_lists(m, keep_ref)


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_mask_end_to_end(w):
    """GPU forward statistics -> GPU mask versus the oracle's own statistics and
    selection: equal except tiles within 1e-6 of the cut (reported)."""
    r = _setup(w)
    bl = r["bl"]
    n = w.n
    cand = orc.candidates(n, w.causal)
    a_ref = orc.tile_log_weights(r["ref"]["tile_lse"], r["ref"]["lse"], n, w.causal)
    for negl in (0.01, NEGL, 0.1):
        m = bl.mask(r["tl"], r["lse"], n, w.causal, negl)
        keep_ref = orc.select_keep(a_ref, cand, negl)
        keep = m["keep"].cpu().numpy().astype(bool)
        bad, exc = excused_mismatches(keep, keep_ref, a_ref, cand, negl)
        flush_print(f"  negl={negl}: kept {keep.sum()}/{keep_ref.sum()} ref, excused {len(exc)}")
        assert not bad, f"unexcused mask mismatches {bad[:5]}"
        check_lists(m, keep)


PATHS = ("recompute", "stored")


def _bwd_path(r, lists, path, o_lo=True):
    """Backward through the C ABI on the given G_Q path: "recompute" (base
    workspace) or "stored" (slots for every kept tile; the state words must
    show the stored path taken)."""
    bl, xg, w = r["bl"], r["xg"], r["w"]
    ws = bl._lib.bwd_workspace(xg["q"], xg["k"], lists, stored_tiles=0 if path == "recompute" else "auto")
    out = bl.bwd(xg["q"], xg["k"], xg["v"], r["o"], xg["do"], r["lse"], lists, causal=w.causal,
                 o_lo=r["olo"] if o_lo else None, workspace=ws)
    if path == "stored":
        taken, kept = bl._lib.bwd_stored_taken(ws, w.B, w.H, w.Hk, w.n, w.d)
        assert taken and kept == int(lists["qcnt"].sum().item())
    return out


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_backward_on_oracle_mask(w, path):
    r = _setup(w)
    dev, x = r["dev"], r["x"]
    keep = orc.mask_from_stats(r["ref"]["tile_lse"], r["ref"]["lse"], w.n, w.causal, NEGL)
    lists = lists_to_torch(keep, dev)
    dq, dk, dv = _bwd_path(r, lists, path)
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=w.causal)
    for name, got, ref in (("dQ", dq, g["dQ"]), ("dK", dk, g["dK"]), ("dV", dv, g["dV"])):
        rl, cs = assert_close_grad(name, got.cpu(), ref)
        flush_print(f"  {path} {name}: rel-L2 {rl:.2e} cos {cs:.6f}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_backward_dense(w, path):
    """negl_prob = 0 without statistics: every candidate tile, dense gradients."""
    r = _setup(w)
    bl, x = r["bl"], r["x"]
    m = bl.mask(None, r["lse"], w.n, w.causal, 0.0)
    check_lists(m, np.broadcast_to(orc.candidates(w.n, w.causal), (w.B, w.H) + (m["keep"].shape[-1],) * 2))
    dq, dk, dv = _bwd_path(r, m, path)
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], causal=w.causal)
    for name, got, ref in (("dQ", dq, g["dQ"]), ("dK", dk, g["dK"]), ("dV", dv, g["dV"])):
        assert_close_grad(name, got.cpu(), ref)


@pytest.mark.parametrize("w", [CASES[0], CASES[1], CASES[2]], ids=IDS[:3])
def test_stored_path_matches_recompute(w):
    """Both G_Q paths: G_K, G_V bit-identical (same pass, with or without the
    G_S stores); G_Q equal to the recompute path up to fp32 summation order."""
    r = _setup(w)
    m = r["bl"].mask(r["tl"], r["lse"], w.n, w.causal, NEGL)
    a = _bwd_path(r, m, "recompute")
    b = _bwd_path(r, m, "stored")
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))
    assert torch.equal(a[2].view(torch.int16), b[2].view(torch.int16))
    rl = orc.rel_l2(b[0].cpu(), orc.to_f64(a[0].cpu()))
    flush_print(f"  dQ stored vs recompute rel-L2 {rl:.2e}")
    assert rl <= 2e-3


@pytest.mark.parametrize("frac", [0.0, 0.4, 0.999])
def test_stored_path_with_a_slot_budget(frac):
    """Fewer G_S slots than kept tiles (a byte budget): slots go to the kept
    tiles in query-tile order, the query tiles whose kept tiles all got one take
    G_Q from the stored tiles and the rest recompute, decided on the device.
    State words: not all stored, kept count, slotted count.  G_K/G_V equal the
    recompute path's bit for bit; G_Q of the recomputed query tiles equals it
    bit for bit, the stored ones agree to fp32 summation order; all match the
    oracle."""
    r = _setup(CASES[1])
    bl, x, xg, w = r["bl"], r["x"], r["xg"], r["w"]
    keep = orc.mask_from_stats(r["ref"]["tile_lse"], r["ref"]["lse"], w.n, w.causal, NEGL)
    m = lists_to_torch(keep, r["dev"])
    qcnt = m["qcnt"].cpu().numpy().reshape(-1)
    kept = int(qcnt.sum())
    slots = max(1, int(frac * kept))
    ws = bl._lib.bwd_workspace(xg["q"], xg["k"], m, stored_tiles=slots)
    a = bl.bwd(xg["q"], xg["k"], xg["v"], r["o"], xg["do"], r["lse"], m, causal=True, o_lo=r["olo"],
               workspace=ws)
    all_in, counted, slotted = bl._lib.bwd_state(ws, w.B, w.H, w.Hk, w.n, w.d)
    assert not all_in and counted == kept and slotted == slots
    b = _bwd_path(r, m, "recompute")
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))
    assert torch.equal(a[2].view(torch.int16), b[2].view(torch.int16))
    # query tiles (b, h, qt) in slot order; stored iff exclusive prefix + count <= slots
    stored = (np.cumsum(qcnt) <= slots).reshape(w.B, w.H, -1)
    T = stored.shape[-1]
    ga, gb = a[0].cpu(), b[0].cpu()
    for bb in range(w.B):
        for h in range(w.H):
            for qt in range(T):
                rows = slice(qt * 128, min(w.n, qt * 128 + 128))
                u, v = ga[bb, rows, h], gb[bb, rows, h]
                if stored[bb, h, qt]:
                    assert orc.rel_l2(u, orc.to_f64(v)) <= 2e-3
                else:
                    assert torch.equal(u.view(torch.int16), v.view(torch.int16))
    flush_print(f"  slots {slots}/{kept}: {int(stored.sum())} of {stored.size} query tiles stored")
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=w.causal)
    for name, got, ref in (("dQ", a[0], g["dQ"]), ("dK", a[1], g["dK"]), ("dV", a[2], g["dV"])):
        assert_close_grad(name, got.cpu(), ref)


@pytest.mark.parametrize("w", [CASES[0], CASES[1], CASES[2], CASES[5]], ids=[IDS[0], IDS[1], IDS[2], IDS[5]])
def test_delta_buffer(w):
    """The D preprocess on its own: the backward leaves D = rowsum(G_O * O) in
    fp32 at the start of its workspace ([B, H, n]).  Against the oracle's
    delta() of the same bf16 operands (O + O_lo when the residual is passed, O
    alone when not) it agrees to fp32 rounding; against the oracle's fp64 D from
    its own forward, the residual brings it closer."""
    r = _setup(w)
    bl, x, xg = r["bl"], r["x"], r["xg"]
    m = bl.mask(r["tl"], r["lse"], w.n, w.causal, NEGL)
    B, H, n = w.B, w.H, w.n
    ref64 = orc.delta(x["do"], r["ref"]["O"])
    errs = {}
    for with_lo in (True, False):
        ws = bl._lib.bwd_workspace(xg["q"], xg["k"], m, stored_tiles=0)
        bl.bwd(xg["q"], xg["k"], xg["v"], r["o"], xg["do"], r["lse"], m, causal=w.causal,
               o_lo=r["olo"] if with_lo else None, workspace=ws)
        D = ws[:B * H * n * 4].view(torch.float32).view(B, H, n).cpu().numpy().astype(np.float64)
        o_used = orc.to_f64(r["o"].cpu()) + (orc.to_f64(r["olo"].cpu()) if with_lo else 0.0)
        want = orc.delta(x["do"], o_used)
        scale = orc.delta(np.abs(orc.to_f64(x["do"])), np.abs(o_used))  # sum of |terms| per row
        assert np.all(np.abs(D - want) <= 2e-6 * scale + 1e-30), f"O_lo={with_lo}: D off by more than fp32 rounding"
        errs[with_lo] = orc.rel_l2(D, ref64)
    flush_print(f"  D rel-L2 vs fp64 oracle: with O_lo {errs[True]:.2e}, O alone {errs[False]:.2e}")
    assert errs[True] <= 1e-2 and errs[False] <= 1e-2
    if n > 1:
        assert errs[True] < errs[False]


# 128 query heads on one kv head: every key tile's G_K/G_V list holds 128 x 17 =
# 2176 items, more than the 2048-item window the G_K/G_V pass keeps in LDS
WIDE = small(2176, H=128, Hk=1, d=64, causal=False, kind="gaussian", seed=12)


@pytest.mark.parametrize("path", PATHS)
def test_backward_item_window_refill(path, monkeypatch):
    """A G_K/G_V chunk longer than the LDS item window (2048 items): with the
    minimum chunk set above the list length no list is split and the pass
    refills its item window mid-chunk.  Gradients match the oracle (dense, every
    pair kept) and the split run (chunks of 16); G_Q, untouched by the chunking,
    is identical bit for bit."""
    w = WIDE
    r = _setup(w)
    bl, x, xg = r["bl"], r["x"], r["xg"]
    m = bl.mask(None, r["lse"], w.n, w.causal, 0.0)
    T = orc.ntiles(w.n)
    items = int(m["kcnt"].cpu().numpy().reshape(w.B, w.Hk, w.H // w.Hk, T).sum(axis=2).max())
    assert items > 2048
    monkeypatch.setenv("BACKLITE_DKDV_MIN_CHUNK", "4096")
    whole = _bwd_path(r, m, path)
    monkeypatch.setenv("BACKLITE_DKDV_MIN_CHUNK", "16")
    split = _bwd_path(r, m, path)
    assert torch.equal(whole[0].view(torch.int16), split[0].view(torch.int16))
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], causal=w.causal)
    for name, got, alt, ref in (("dQ", whole[0], split[0], g["dQ"]), ("dK", whole[1], split[1], g["dK"]),
                                ("dV", whole[2], split[2], g["dV"])):
        rl, cs = assert_close_grad(name, got.cpu(), ref)
        assert_close_grad(name + " (split)", alt.cpu(), ref)
        flush_print(f"  {path} {name}: rel-L2 {rl:.2e} cos {cs:.6f}; whole vs split "
                    f"{orc.rel_l2(got.cpu(), orc.to_f64(alt.cpu())):.1e}")


# attention sinks: every query tile keeps key tile 0, whose list (48 items over
# the 4 heads of the group) is several times the average list
SINK = small(1536, H=4, Hk=1, d=64, causal=True, kind="positional", seed=9, period=512.0)


def _expected_split(lists, B, Hk, G, T, chmin):
    """Host-side copy of the chunk-length rule, to check that a case splits."""
    kc = lists["kcnt"].cpu().numpy().reshape(B, Hk, G, T).sum(axis=2)
    ch = max(chmin, -(-2 * int(kc.sum()) // (B * Hk * T)))
    return int(kc.max()), ch


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("chmin", [1, 16])
def test_backward_split_lists(chmin, path, monkeypatch):
    """G_K/G_V lists split over several workgroups (the sink key tile's list is
    split into chunks whose fp32 partials are summed in order): gradients match
    the oracle, G_Q is unchanged by the split, and results repeat bit for bit."""
    w = SINK
    r = _setup(w)
    x = r["x"]
    keep = orc.mask_from_stats(r["ref"]["tile_lse"], r["ref"]["lse"], w.n, w.causal, NEGL)
    lists = lists_to_torch(keep, r["dev"])
    longest, ch = _expected_split(lists, w.B, w.Hk, w.H // w.Hk, orc.ntiles(w.n), chmin)
    flush_print(f"  longest list {longest} items, chunk length {ch}")
    assert longest > ch, "the case must split a list"
    monkeypatch.setenv("BACKLITE_DKDV_MIN_CHUNK", str(chmin))
    dq, dk, dv = _bwd_path(r, lists, path)
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=w.causal)
    for name, got, ref in (("dQ", dq, g["dQ"]), ("dK", dk, g["dK"]), ("dV", dv, g["dV"])):
        rl, cs = assert_close_grad(name, got.cpu(), ref)
        flush_print(f"  split {path} {name}: rel-L2 {rl:.2e} cos {cs:.6f}")
    again = _bwd_path(r, lists, path)
    for u, v in zip((dq, dk, dv), again):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))


# non-causal with a ragged last key tile (1000 = 7 x 128 + 104 keys), used
# with a constructed keep pattern: the diagonal, and the ragged tile kept by
# every query tile, so that tile's list (4 heads x 8 query tiles) is several
# times the chunk length
RAGGED_COL = small(1000, H=4, Hk=1, d=128, causal=False, kind="gaussian", seed=13)


@pytest.mark.parametrize("path", PATHS)
def test_backward_split_ragged_tile(path, monkeypatch):
    """The ragged last key tile's G_K/G_V list split into chunks (chunk minimum
    1): on the stored path these chunks run in the instance that masks the
    padded keys, launched over the ragged tiles' chunks only.  Gradients match
    the oracle on the same keep pattern and repeat bit for bit."""
    w = RAGGED_COL
    r = _setup(w)
    x = r["x"]
    T = orc.ntiles(w.n)
    keep = np.zeros((w.B, w.H, T, T), dtype=bool)
    keep[:, :, np.arange(T), np.arange(T)] = True
    keep[:, :, :, T - 1] = True
    lists = lists_to_torch(keep, r["dev"])
    longest, ch = _expected_split(lists, w.B, w.Hk, w.H // w.Hk, T, 1)
    flush_print(f"  ragged tile list {longest} items, chunk length {ch}")
    assert longest > 2 * ch, "the ragged tile's list must split into several chunks"
    monkeypatch.setenv("BACKLITE_DKDV_MIN_CHUNK", "1")
    dq, dk, dv = _bwd_path(r, lists, path)
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=w.causal)
    for name, got, ref in (("dQ", dq, g["dQ"]), ("dK", dk, g["dK"]), ("dV", dv, g["dV"])):
        rl, cs = assert_close_grad(name, got.cpu(), ref)
        flush_print(f"  ragged split {path} {name}: rel-L2 {rl:.2e} cos {cs:.6f}")
    again = _bwd_path(r, lists, path)
    for u, v in zip((dq, dk, dv), again):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))


@pytest.mark.parametrize("path", PATHS)
def test_backward_plan_mixed_lists(path, monkeypatch):
    """A keep pattern that exercises the G_K/G_V chunk plan's ordering: most
    key tiles (the ragged last one included) have empty lists, one is kept by
    every query tile of every head (32 items, split into four chunks at chunk
    minimum 1), two have short lists, so the tiles fall in several length
    classes and the chunk table holds zero-length chunks.  Gradients match
    the oracle on the same pattern and repeat bit for bit."""
    w = RAGGED_COL
    r = _setup(w)
    x = r["x"]
    T = orc.ntiles(w.n)
    keep = np.zeros((w.B, w.H, T, T), dtype=bool)
    keep[:, :, :, 2] = True
    keep[:, 0, 3, 5] = True
    keep[:, 1, :4, 6] = True
    lists = lists_to_torch(keep, r["dev"])
    longest, ch = _expected_split(lists, w.B, w.Hk, w.H // w.Hk, T, 1)
    assert longest > 2 * ch, "the long list must split into several chunks"
    monkeypatch.setenv("BACKLITE_DKDV_MIN_CHUNK", "1")
    dq, dk, dv = _bwd_path(r, lists, path)
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=w.causal)
    for name, got, ref in (("dQ", dq, g["dQ"]), ("dK", dk, g["dK"]), ("dV", dv, g["dV"])):
        rl, cs = assert_close_grad(name, got.cpu(), ref)
        flush_print(f"  mixed lists {path} {name}: rel-L2 {rl:.2e} cos {cs:.6f}")
    # key tiles no query tile keeps get exactly zero gradients
    dk_c, dv_c = dk.cpu().float(), dv.cpu().float()  # [B, n, H_k, d]
    for kt in (0, 1, 3, 4, 7):
        rows = slice(kt * 128, min(w.n, (kt + 1) * 128))
        assert (dk_c[:, rows] == 0).all() and (dv_c[:, rows] == 0).all()
    again = _bwd_path(r, lists, path)
    for u, v in zip((dq, dk, dv), again):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))


def test_backward_nothing_kept():
    """Lists that keep no tile at all (a caller may build them): every
    gradient is exactly zero."""
    w = RAGGED_COL
    r = _setup(w)
    bl, xg = r["bl"], r["xg"]
    T = orc.ntiles(w.n)
    lists = lists_to_torch(np.zeros((w.B, w.H, T, T), dtype=bool), r["dev"])
    dq, dk, dv = bl.bwd(xg["q"], xg["k"], xg["v"], r["o"], xg["do"], r["lse"], lists, causal=w.causal,
                        o_lo=r["olo"])
    torch.cuda.synchronize()
    for name, t in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert (t.float() == 0).all(), name


@pytest.mark.parametrize("path", PATHS)
def test_backward_deterministic(path):
    r = _setup(CASES[1])
    bl, w = r["bl"], r["w"]
    m = bl.mask(r["tl"], r["lse"], w.n, w.causal, NEGL)
    a = _bwd_path(r, m, path)
    b = _bwd_path(r, m, path)
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))


def test_module_autograd_matches_oracle():
    """BackLite module: forward + loss.backward() against the oracle end to end."""
    w = small(500, H=4, Hk=2, d=128, causal=True, kind="blocks", seed=7)
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev).requires_grad_() for n in ("q", "k", "v"))
    attn = bl.BackLite(negl_prob=NEGL, causal=True)
    o, lse = attn(q, k, v, return_softmax_lse=True)
    o.backward(x["do"].to(dev))
    ref = orc.forward(x["q"], x["k"], x["v"], causal=True)
    keep = orc.mask_from_stats(ref["tile_lse"], ref["lse"], w.n, True, NEGL)
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=True)
    assert_close_out("O", o.detach().cpu(), ref["O"])
    assert_close_out("lse", lse.cpu(), ref["lse"])
    for name, got, rr in (("dQ", q.grad, g["dQ"]), ("dK", k.grad, g["dK"]), ("dV", v.grad, g["dV"])):
        assert_close_grad(name, got.cpu(), rr)


def test_module_backward_twice_with_retained_graph():
    """Two backward passes through one graph (retain_graph=True): the compact
    statistics live with the graph, so the second pass runs the same sparse
    backward and accumulates exactly the first one's gradients again."""
    w = small(500, H=4, Hk=2, d=128, causal=True, kind="blocks", seed=7)
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev).requires_grad_() for n in ("q", "k", "v"))
    attn = bl.BackLite(negl_prob=NEGL, causal=True)
    o = attn(q, k, v)
    do = x["do"].to(dev)
    o.backward(do, retain_graph=True)
    first = [t.grad.clone() for t in (q, k, v)]
    for t in (q, k, v):
        t.grad = None
    o.backward(do)
    for a, t in zip(first, (q, k, v)):
        assert torch.equal(a.view(torch.int16), t.grad.view(torch.int16))


def test_backward_without_residual_gaussian():
    """O_lo is optional: on inputs without a large shared key component the
    bf16 O alone already meets the bound."""
    r = _setup(CASES[2])
    bl, x, xg, w = r["bl"], r["x"], r["xg"], r["w"]
    keep = orc.mask_from_stats(r["ref"]["tile_lse"], r["ref"]["lse"], w.n, w.causal, NEGL)
    dq, dk, dv = bl.bwd(xg["q"], xg["k"], xg["v"], r["o"], xg["do"], r["lse"], lists_to_torch(keep, r["dev"]),
                        causal=w.causal)
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=w.causal)
    for name, got, ref in (("dQ", dq, g["dQ"]), ("dK", dk, g["dK"]), ("dV", dv, g["dV"])):
        assert_close_grad(name, got.cpu(), ref)


def test_stats_counters():
    r = _setup(CASES[0])
    bl, w = r["bl"], r["w"]
    st = torch.zeros(2, dtype=torch.int64, device=r["dev"])
    m = bl.mask(r["tl"], r["lse"], w.n, w.causal, NEGL, stats=st)
    s = st.cpu().tolist()
    assert s[0] == w.B * w.H * 64 and s[1] == int(m["keep"].sum().item())


@pytest.mark.parametrize("w", [CASES[0], CASES[1], CASES[2], CASES[5]], ids=[IDS[0], IDS[1], IDS[2], IDS[5]])
def test_backward_atomic_gq_variant(w):
    """The fused single-pass variant with an fp32-atomic G_Q: G_K and G_V equal
    the two-pass backward's bit for bit (the same G_K/G_V pass), G_Q matches the
    oracle on the same mask and the two-pass G_Q to fp32 summation order."""
    r = _setup(w)
    bl, x, xg = r["bl"], r["x"], r["xg"]
    keep = orc.mask_from_stats(r["ref"]["tile_lse"], r["ref"]["lse"], w.n, w.causal, NEGL)
    lists = lists_to_torch(keep, r["dev"])
    a = bl._lib.bwd_atomic(xg["q"], xg["k"], xg["v"], r["o"], xg["do"], r["lse"], lists, causal=w.causal,
                           o_lo=r["olo"])
    b = _bwd_path(r, lists, "recompute")
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))
    assert torch.equal(a[2].view(torch.int16), b[2].view(torch.int16))
    g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=w.causal)
    rl, cs = assert_close_grad("dQ", a[0].cpu(), g["dQ"])
    flush_print(f"  atomic dQ rel-L2 {rl:.2e} cos {cs:.6f}; vs two-pass {orc.rel_l2(a[0].cpu(), orc.to_f64(b[0].cpu())):.1e}")
