"""Compact tile statistics: the forward's tile_w output (one fp64 log-weight
per tile pair, reduced from the per-row tile LSEs in the forward's epilogue)
and backlite_mask_compact.  tile_w must equal the oracle's tile_log_weights
applied to the forward's own fp32 outputs, bit for bit (the same fp64
subtraction and maximum), and the compact mask must select exactly the tiles
the per-row mask selects.  GPU only."""
import numpy as np
import pytest
import torch

from helpers import TILE, check_lists, flush_print, gpu_available, packed_to_rows, pair_index
from oracle import backlite_oracle as orc
from workloads import DIT480, LLM128K, TINY, make_inputs, small

pytestmark = pytest.mark.gpu

# (workload, window)
CASES = [
    (TINY, 0),
    (small(1000, H=4, Hk=2, d=128, causal=True, kind="blocks", seed=1), 0),
    (small(300, H=2, Hk=1, d=64, causal=False, kind="gaussian", seed=2), 0),
    (small(640, H=2, d=128, causal=False, kind="blocks", B=2, seed=5), 0),
    (small(1000, H=4, Hk=2, d=128, causal=True, kind="blocks", seed=11), 300),
    (small(513, H=2, d=64, causal=True, kind="gaussian", seed=13), 1),
]
IDS = [f"{w.name}-w{win}" for w, win in CASES]


def _unpack_w(tw, B, H, n, causal, cand):
    """[B*H*pairs*2] fp64 -> [B, H, ceil(n/64), T]: the value of 64-row half j of
    query tile qt at row 2 qt + j; -inf where the 128-row pair is no candidate."""
    T = (n + TILE - 1) // TILE
    pairs = T * (T + 1) // 2 if causal else T * T
    a = np.asarray(tw, dtype=np.float64).reshape(B, H, pairs, 2)
    out = np.full((B, H, 2 * T, T), -np.inf)
    for qt in range(T):
        for kt in range(T):
            if cand[qt, kt]:
                out[:, :, 2 * qt:2 * qt + 2, kt] = a[:, :, pair_index(qt, kt, T, causal), :]
    return out[:, :, :(n + 63) // 64]


def _run(bl, w, win):
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (x[nm].to(dev) for nm in ("q", "k", "v"))
    B, H, n = w.B, w.H, w.n
    tw = torch.empty(bl._lib.tile_w_elems(B, H, n, w.causal), dtype=torch.float64, device=dev)
    o, lse, tl = bl.fwd(q, k, v, causal=w.causal, window=win, tile_w=tw)
    o2, lse2, tl2 = bl.fwd(q, k, v, causal=w.causal, window=win)
    torch.cuda.synchronize()
    return o, lse, tl, tw, o2, lse2


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_compact_statistics_bit_exact(case):
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    w, win = case
    B, H, n, causal = w.B, w.H, w.n, w.causal
    flush_print(f"[case] {w.name} window={win}")
    o, lse, tl, tw, o2, lse2 = _run(bl, w, win)
    # asking for the compact statistics changes nothing else
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    cand = orc.candidates(n, causal, window=win)
    rows = packed_to_rows(tl.cpu().numpy(), B, H, n, causal)
    rows = np.where(np.broadcast_to(cand[np.arange(n) // TILE], rows.shape), rows, -np.inf)
    # one value per 64-row half: the oracle's log-weights over 64-row query tiles
    want = orc.tile_log_weights(rows, lse.cpu().numpy(), n, causal, window=win, q_tile=64)
    got = _unpack_w(tw.cpu().numpy(), B, H, n, causal, cand)
    assert np.array_equal(got, want)
    # the compact mask selects exactly what the per-row mask selects, for both
    # query-tile heights
    for q_tile in (128, 64):
        for negl in (0.0, 0.01, 0.05, 0.3):
            m1 = bl.mask(tl, lse, n, causal, negl, window=win, q_tile=q_tile)
            m2 = bl._lib.mask_compact(tw, B, H, n, causal, negl, window=win, q_tile=q_tile)
            check_lists(m2, m1["keep"].cpu().numpy().astype(bool))
    # and dense without statistics
    m0 = bl._lib.mask_compact(None, B, H, n, causal, 0.0, window=win, device=tw.device)
    T = m0["keep"].shape[-1]
    check_lists(m0, np.broadcast_to(cand, (B, H, T, T)))


@pytest.mark.parametrize("w,win", [(DIT480, 0), (LLM128K, 2048)], ids=["dit-480p-32k", "llm-128k-causal-w2048"])
def test_compact_mask_full_size(w, win):
    """At full size, in the bench's launch configuration: the compact mask's
    lists equal the per-row mask's for every head."""
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    flush_print(f"[case] {w.name} window={win}")
    B, H, n, causal = w.B, w.H, w.n, w.causal
    o, lse, tl, tw, o2, lse2 = _run(bl, w, win)
    assert torch.equal(o, o2)
    sparse = next(p for p in w.negl_probs if p > 0)
    for negl, q_tile in [(p, 128) for p in w.negl_probs] + [(sparse, 64)]:
        m1 = bl.mask(tl, lse, n, causal, negl, window=win, q_tile=q_tile)
        m2 = bl._lib.mask_compact(tw, B, H, n, causal, negl, window=win, q_tile=q_tile)
        for key in ("keep", "qcnt", "qidx", "kcnt", "kidx"):
            if key in ("qidx", "kidx"):
                # compare only the listed prefix of each row
                cnt = m1["qcnt" if key == "qidx" else "kcnt"]
                idx = torch.arange(m1[key].shape[-1], device=cnt.device)
                sel = idx[None, None, None, :] < cnt[..., None]
                assert torch.equal(m1[key][sel], m2[key][sel]), key
            else:
                assert torch.equal(m1[key], m2[key]), key
        flush_print(f"  negl={negl} q_tile={q_tile}: kept {int(m1['qcnt'].sum())} tiles, identical")
    flush_print(f"  tile_lse {tl.numel() * 4 / 1e9:.3f} GB, tile_w {tw.numel() * 8 / 1e9:.4f} GB")


@pytest.mark.parametrize("causal,win", [(False, 0), (True, 0), (True, 300)], ids=["noncausal", "causal", "window300"])
def test_module_compact_path_equals_per_row_path(causal, win):
    """The autograd module (which keeps only the compact statistics) gives the
    same gradients, bit for bit, as fwd -> mask on the per-row statistics ->
    bwd through the C ABI."""
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    w = small(1000, H=4, Hk=2, d=128, causal=causal, kind="blocks", seed=31)
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (x[nm].to(dev) for nm in ("q", "k", "v", "do"))
    qg, kg, vg = (t.clone().requires_grad_(True) for t in (q, k, v))
    attn = bl.BackLite(negl_prob=0.05, causal=causal, window=win)
    attn(qg, kg, vg).backward(do)
    o, lse, tl, olo = bl.fwd(q, k, v, causal=causal, with_residual=True, window=win)
    m = bl.mask(tl, lse, w.n, causal, 0.05, window=win)
    ws = bl._lib.bwd_workspace(q, k, m)
    dq, dk, dv = bl.bwd(q, k, v, o, do, lse, m, causal=causal, o_lo=olo, window=win, workspace=ws)
    kept = int(m["qcnt"].sum())
    flush_print(f"  kept {kept} tiles")
    assert kept < m["keep"].numel()
    for name, a, b in (("dQ", qg.grad, dq), ("dK", kg.grad, dk), ("dV", vg.grad, dv)):
        assert torch.equal(a, b), name
