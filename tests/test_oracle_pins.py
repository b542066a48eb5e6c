"""Pins of the fp64 oracle against things other than itself.

Each test fixes the oracle to a library routine, a closed form, a value the
pages print, brute force on a tiny input, or an invariant the pages state, so
that a dropped term, a wrong sign or index, or a transposed operand in the
oracle fails at least one of them.  CPU only.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import backlite_oracle as orc
from workloads import TINY, make_inputs, small


def _rand(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return scale * g.standard_normal(shape)


def _torch_attention(q, k, v, scale, causal):
    """Reference via torch fp64 library ops on CPU: [B,n,H,d] layout, GQA by repeat."""
    B, n, H, d = q.shape
    Hk = k.shape[2]
    G = H // Hk
    qt = q.permute(0, 2, 1, 3)
    kt = k.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vt = v.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    S = scale * torch.matmul(qt, kt.transpose(-1, -2).contiguous())
    if causal:
        m = torch.ones(n, n, dtype=torch.bool).tril()
        S = S.masked_fill(~m, float("-inf"))
    lse = torch.logsumexp(S, dim=-1)
    P = torch.softmax(S, dim=-1)
    O = torch.matmul(P, vt).permute(0, 2, 1, 3)
    return O, lse, S, P


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n,H,Hk,d,causal", [(200, 2, 2, 16, False), (200, 4, 2, 16, True),
                                              (129, 2, 1, 8, True), (1, 1, 1, 4, False)])
def test_forward_matches_torch_library(n, H, Hk, d, causal):
    q, k, v = _rand((1, n, H, d), 1), _rand((1, n, Hk, d), 2), _rand((1, n, Hk, d), 3)
    sc = 0.37
    out = orc.forward(q, k, v, scale=sc, causal=causal, tile=64)
    O, lse, _, _ = _torch_attention(*(torch.from_numpy(x) for x in (q, k, v)), sc, causal)
    np.testing.assert_allclose(out["O"], O.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["lse"], lse.numpy(), rtol=0, atol=1e-12)


def test_softmax_overflow_case(golden_dir):
    vals = {}
    for line in open(os.path.join(golden_dir, "softmax_overflow.txt")):
        if line.startswith("#") or not line.strip():
            continue
        key, *nums = line.split()
        vals[key] = [float(x) for x in nums]
    # one query, three keys, d = 1, scale 1: S = q * k = [1000, 1001, 1002]
    q = np.ones((1, 1, 1, 1))
    k = np.array(vals["scores"]).reshape(1, 3, 1, 1)
    v = np.array([1.0, 0.0, 0.0]).reshape(1, 3, 1, 1)
    # pad the query to 3 rows so the shapes agree; only row 0 is examined
    qq = np.ones((1, 3, 1, 1))
    out = orc.forward(qq, k, v, scale=1.0, causal=False, tile=4)
    assert np.isfinite(out["lse"]).all()
    assert out["lse"][0, 0, 0] == pytest.approx(vals["lse"][0], abs=1e-12)
    # O with V = e_0 picks P[0]; check all three probabilities with three one-hot V's
    for c in range(3):
        vc = np.zeros((1, 3, 1, 1))
        vc[0, c, 0, 0] = 1.0
        o = orc.forward(qq, k, vc, scale=1.0, tile=4)["O"][0, 0, 0, 0]
        # exp(S - LSE) with S ~ 1e3 carries the rounding of LSE (ulp 1.1e-13)
        assert o == pytest.approx(vals["p"][c], rel=1e-12)
    del q


def test_tile_lse_identities():
    """logsumexp over a row's tile LSEs equals the row LSE; p_tile sums to 1."""
    for causal in (False, True):
        q, k, v = _rand((1, 300, 2, 8), 4, 2.0), _rand((1, 300, 1, 8), 5, 2.0), _rand((1, 300, 1, 8), 6)
        out = orc.forward(q, k, v, causal=causal, tile=64)
        tl, L = out["tile_lse"], out["lse"]
        m = tl.max(axis=-1, keepdims=True)
        lse_of_tiles = (m + np.log(np.exp(tl - m).sum(-1, keepdims=True)))[..., 0]
        np.testing.assert_allclose(lse_of_tiles, L, atol=1e-12)
        np.testing.assert_allclose(np.exp(tl - L[..., None]).sum(-1), 1.0, atol=1e-12)
        if causal:
            # a tile that lies entirely above the diagonal has no valid key: -inf
            rows = np.arange(300)
            for kt in range(tl.shape[-1]):
                empty = rows < 64 * kt
                assert np.isneginf(tl[0, :, empty, kt]).all()
                assert np.isfinite(tl[0, :, ~empty, kt]).all()


def test_tile_lse_brute_force_small():
    """Per-element brute force with Python loops on a tiny ragged causal case."""
    n, d, t = 11, 3, 4
    q, k, v = _rand((1, n, 1, d), 7), _rand((1, n, 1, d), 8), _rand((1, n, 1, d), 9)
    sc = 0.5
    out = orc.forward(q, k, v, scale=sc, causal=True, tile=t)
    for i in range(n):
        for kt in range((n + t - 1) // t):
            terms = [math.exp(sc * float(q[0, i, 0] @ k[0, j, 0]))
                     for j in range(kt * t, min(n, kt * t + t)) if j <= i]
            ref = math.log(sum(terms)) if terms else -math.inf
            got = out["tile_lse"][0, 0, i, kt]
            if terms:
                assert got == pytest.approx(ref, abs=1e-12)
            else:
                assert got == -math.inf


def test_causal_block_classification(golden_dir):
    """The page's N=16, block-4 worked example: which query blocks see key block 1."""
    rows = [l.split() for l in open(os.path.join(golden_dir, "causal_blocks_n16_t4.txt"))
            if l.strip() and not l.startswith("#")]
    n, t = 16, 4
    cand = orc.candidates(n, True, t)
    q = _rand((1, n, 1, 2), 10)
    k = _rand((1, n, 1, 2), 11)
    tl = orc.forward(q, k, k, causal=True, tile=t)["tile_lse"][0, 0]   # [n, T]
    for qb, r0, r1, cls in rows:
        qb, r0, r1 = int(qb), int(r0), int(r1)
        valid = np.array([[j <= i for j in range(4, 8)] for i in range(r0, r1 + 1)])
        if cls == "empty":
            assert not cand[qb, 1] and not valid.any()
            assert np.isneginf(tl[r0:r1 + 1, 1]).all()
        elif cls == "partial":
            assert cand[qb, 1] and valid.any() and not valid.all()
        else:
            assert cand[qb, 1] and valid.all()
        if cls != "empty":
            assert np.isfinite(tl[r0:r1 + 1, 1]).all()


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------
def test_selection_closed_form_uniform():
    """Q = 0 => S = 0 => every tile weight is 1/8 (n = 1024, 8 key tiles)."""
    n, d = 1024, 64
    q = np.zeros((1, n, 1, d))
    k = _rand((1, n, 1, d), 12)
    v = _rand((1, n, 1, d), 13)
    out = orc.forward(q, k, v)
    assert out["lse"] == pytest.approx(math.log(1024.0), abs=1e-12)
    assert out["tile_lse"] == pytest.approx(math.log(128.0), abs=1e-12)
    np.testing.assert_allclose(out["O"][0, :, 0], np.broadcast_to(v[0, :, 0].mean(0), (n, d)), atol=1e-12)
    a = orc.tile_log_weights(out["tile_lse"], out["lse"], n, False)
    np.testing.assert_allclose(np.exp(a), 0.125, rtol=1e-15)
    cand = orc.candidates(n, False)
    expect = {0.05: [], 0.3: [0, 1], 0.9: [0, 1, 2, 3, 4, 5, 6]}
    for pi, skipped in expect.items():
        keep = orc.select_keep(a, cand, pi)
        for qt in range(8):
            assert sorted(set(range(8)) - set(np.nonzero(keep[0, 0, qt])[0])) == skipped


def test_selection_strictness_and_ties():
    """Exact weights 1/4 (exp(log 0.25) == 0.25 in fp64): the prefix sums are
    0.25, 0.5, 0.75, 1.0 exactly, so negl_prob = 0.5 skips only the first tile
    (0.5 is not < 0.5), and among equal weights the lower kt goes first."""
    assert math.exp(math.log(0.25)) == 0.25
    a = np.full((1, 1, 4, 4), math.log(0.25))
    cand = orc.candidates(4 * 128, False)
    keep = orc.select_keep(a, cand, 0.5)
    assert (keep[0, 0] == np.array([False, True, True, True])).all()
    keep = orc.select_keep(a, cand, np.nextafter(0.5, 1.0))
    assert (keep[0, 0] == np.array([False, False, True, True])).all()
    keep = orc.select_keep(a, cand, 0.0)
    assert keep.all()


def _brute_keep(w, pi):
    """Brute force: tile t is skipped iff the total weight of every tile that
    precedes-or-equals it in the (w, kt) order is < pi (pairwise comparisons,
    no sort)."""
    T = len(w)
    out = np.ones(T, bool)
    for t in range(T):
        le = [u for u in range(T) if (w[u], u) <= (w[t], t)]
        if math.fsum(w[u] for u in le) < pi:
            out[t] = False
    return out


def test_selection_brute_force():
    g = np.random.default_rng(14)
    for trial in range(300):
        T = int(g.integers(1, 8))
        w = g.dirichlet(np.ones(T) * 0.5)
        if trial % 5 == 0:
            w = np.round(w * 8) / 8 + 1e-3          # force equal weights
        pi = float(g.uniform(0, 1))
        a = np.log(w).reshape(1, 1, 1, T)
        a = np.broadcast_to(a, (1, 1, T, T)).copy()
        keep = orc.select_keep(a, orc.candidates(T * 128, False), pi)[0, 0, 0]
        ref = _brute_keep(np.exp(np.log(w)), pi)
        # a sum within 1e-12 of pi may round either way between fsum and the
        # sequential sum; skip those draws
        cs = np.sort(w)
        if np.min(np.abs(np.cumsum(cs) - pi)) < 1e-12:
            continue
        assert (keep == ref).all(), (w, pi, keep, ref)


def test_selection_invariants_on_block_workload():
    """I3: skipped mass per row < negl_prob; I5: every query tile keeps >= 1;
    I6: the keep set shrinks as negl_prob grows; off-diagonal tiles of the
    block-structured workload are negligible so only the diagonal is kept."""
    x = make_inputs(TINY)
    out = orc.forward(x["q"], x["k"], x["v"])
    a = orc.tile_log_weights(out["tile_lse"], out["lse"], TINY.n, False)
    cand = orc.candidates(TINY.n, False)
    prev = None
    p = np.exp(out["tile_lse"] - out["lse"][..., None])     # [B,H,n,T]
    for pi in (0.0, 1e-12, 0.01, 0.05, 0.1, 0.5, 0.99):
        keep = orc.select_keep(a, cand, pi)
        assert keep.sum(axis=3).min() >= 1
        if prev is not None:
            assert not (keep & ~prev).any()
        prev = keep
        for qt in range(8):
            skip = ~keep[0, :, qt, :]                        # [H, T]
            w = np.exp(a[0, :, qt, :])
            assert ((w * skip).sum(-1) < pi + 0.0).all() or pi == 0.0
            rows = p[0, :, qt * 128:(qt + 1) * 128, :]
            assert ((rows * skip[:, None, :]).sum(-1) < max(pi, 1e-300)).all() or pi == 0.0
        if pi >= 1e-6:      # the largest off-diagonal weight here is ~4e-10
            assert (keep[0, :] == np.eye(8, dtype=bool)[None]).all()


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def _loss_fd(q, k, v, do, scale, causal):
    O = orc.forward(q, k, v, scale=scale, causal=causal, tile=16)["O"]
    return float((do * O).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_dense_grads_central_differences(causal):
    """n = 64, d = 16: central differences of L = sum(G_O * O), step 1e-6."""
    n, d = 64, 16
    q, k, v, do = (_rand((1, n, 1, d), s, 0.7) for s in (20, 21, 22, 23))
    sc = 1.0 / math.sqrt(d)
    g = orc.backward(q, k, v, do, scale=sc, causal=causal, tile=16)
    h = 1e-6
    rng = np.random.default_rng(24)
    for name, X, G in (("q", q, g["dQ"]), ("k", k, g["dK"]), ("v", v, g["dV"])):
        for _ in range(40):
            i, c = int(rng.integers(n)), int(rng.integers(d))
            Xp, Xm = X.copy(), X.copy()
            Xp[0, i, 0, c] += h
            Xm[0, i, 0, c] -= h
            args = {"q": q, "k": k, "v": v}
            fp = _loss_fd(*(Xp if nm == name else args[nm] for nm in ("q", "k", "v")), do, sc, causal)
            fm = _loss_fd(*(Xm if nm == name else args[nm] for nm in ("q", "k", "v")), do, sc, causal)
            fd = (fp - fm) / (2 * h)
            an = G[0, i, 0, c]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, i, c, fd, an)


@pytest.mark.parametrize("n,H,Hk,causal", [(200, 2, 2, False), (200, 4, 1, True), (130, 4, 2, False)])
def test_dense_grads_torch_autograd(n, H, Hk, causal):
    d = 16
    q, k, v, do = _rand((1, n, H, d), 30), _rand((1, n, Hk, d), 31), _rand((1, n, Hk, d), 32), _rand((1, n, H, d), 33)
    sc = 0.3
    g = orc.backward(q, k, v, do, scale=sc, causal=causal, tile=64)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    O, _, _, _ = _torch_attention(tq, tk, tv, sc, causal)
    O.backward(torch.from_numpy(do))
    np.testing.assert_allclose(g["dQ"], tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(g["dK"], tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(g["dV"], tv.grad.numpy(), atol=1e-11)


def test_masked_grads_torch_autograd():
    """A mask that drops heavy tiles.  Independent route: dS_dense from torch
    autograd through softmax, restricted by the element mask; G_Q, G_K from
    autograd of S = scale Q K^T fed that restricted dS; G_V from autograd of
    (masked P, held constant) @ V."""
    n, d, t = 192, 8, 64
    q, k, v, do = _rand((1, n, 1, d), 40, 1.5), _rand((1, n, 1, d), 41, 1.5), _rand((1, n, 1, d), 42), _rand((1, n, 1, d), 43)
    sc = 0.5
    for causal in (False, True):
        keep = orc.candidates(n, causal, t).copy()
        keep[2, 0] = False
        keep[1, 1] = False
        keep[0, 0] = True
        g = orc.backward(q, k, v, do, keep=keep[None, None], scale=sc, causal=causal, tile=t)
        tq, tk, tv = (torch.from_numpy(x[0, :, 0]).requires_grad_() for x in (q, k, v))
        tdo = torch.from_numpy(do[0, :, 0])
        S = sc * tq @ tk.T
        if causal:
            S = S.masked_fill(~torch.ones(n, n, dtype=torch.bool).tril(), float("-inf"))
        P = torch.softmax(S, -1)
        O = P @ tv
        dS_dense, = torch.autograd.grad(O, S, tdo, retain_graph=True)
        M = torch.from_numpy(np.kron(keep, np.ones((t, t), bool))[:n, :n])
        dQ, dK = torch.autograd.grad(S, (tq, tk), torch.where(M, dS_dense, 0.0))
        dV, = torch.autograd.grad(torch.where(M, P, 0.0).detach() @ tv, tv, tdo)
        np.testing.assert_allclose(g["dQ"][0, :, 0], dQ.numpy(), atol=1e-11)
        np.testing.assert_allclose(g["dK"][0, :, 0], dK.numpy(), atol=1e-11)
        np.testing.assert_allclose(g["dV"][0, :, 0], dV.numpy(), atol=1e-11)


def test_all_keep_and_zero_negl_are_dense():
    """I4/I7: negl_prob = 0 keeps every candidate; the all-keep mask reproduces
    the dense backward exactly."""
    w = small(300, H=2, Hk=1, d=16, causal=True, kind="blocks")
    x = make_inputs(w)
    out = orc.forward(x["q"], x["k"], x["v"], causal=True)
    keep = orc.mask_from_stats(out["tile_lse"], out["lse"], w.n, True, 0.0)
    assert (keep == orc.candidates(w.n, True)[None, None]).all()
    g0 = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=None, causal=True)
    g1 = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=True)
    for key in ("dQ", "dK", "dV"):
        assert np.array_equal(g0[key], g1[key])


def test_block_diagonal_limit():
    """With the tiny block workload every off-diagonal tile weight is below
    ~4e-10, so the sparse gradients differ from the dense ones by no more than
    about that much, relative."""
    x = make_inputs(TINY)
    out = orc.forward(x["q"], x["k"], x["v"])
    keep = orc.mask_from_stats(out["tile_lse"], out["lse"], TINY.n, False, 0.05)
    assert keep.sum() == 2 * 8
    a = orc.tile_log_weights(out["tile_lse"], out["lse"], TINY.n, False)
    wmax = float(np.exp(a[~keep]).max())
    assert wmax < 1e-9
    gd = orc.backward(x["q"], x["k"], x["v"], x["do"])
    gs = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep)
    for key in ("dQ", "dK", "dV"):
        r = orc.rel_l2(gs[key], gd[key])
        assert 0 < r < 10 * wmax


def test_gqa_equals_repeated_mha():
    n, H, Hk, d = 160, 4, 2, 8
    q, k, v, do = _rand((1, n, H, d), 50), _rand((1, n, Hk, d), 51), _rand((1, n, Hk, d), 52), _rand((1, n, H, d), 53)
    keep = np.random.default_rng(54).random((1, H, 3, 3)) < 0.6
    keep[..., 0] = True
    g = orc.backward(q, k, v, do, keep=keep, causal=False, tile=64)
    kr, vr = np.repeat(k, 2, axis=2), np.repeat(v, 2, axis=2)
    gr = orc.backward(q, kr, vr, do, keep=keep, causal=False, tile=64)
    np.testing.assert_allclose(g["dQ"], gr["dQ"], atol=1e-13)
    np.testing.assert_allclose(g["dK"], gr["dK"].reshape(1, n, Hk, 2, d).sum(3), atol=1e-13)
    np.testing.assert_allclose(g["dV"], gr["dV"].reshape(1, n, Hk, 2, d).sum(3), atol=1e-13)


def test_lists_from_keep():
    keep = np.zeros((1, 1, 3, 3), bool)
    keep[0, 0] = [[1, 0, 1], [0, 0, 1], [1, 1, 1]]
    qcnt, qidx, kcnt, kidx = orc.lists_from_keep(keep)
    assert qcnt.tolist() == [[[2, 1, 3]]]
    assert qidx[0, 0, 0, :2].tolist() == [0, 2] and qidx[0, 0, 1, :1].tolist() == [2]
    assert kcnt.tolist() == [[[2, 1, 3]]]
    assert kidx[0, 0, 0, :2].tolist() == [0, 2] and kidx[0, 0, 2, :3].tolist() == [0, 1, 2]


@pytest.mark.parametrize("causal", [False, True])
def test_delta_brute_force_identity(causal):
    """D_i = sum_c G_O[i,c] O[i,c] must equal sum_j P_ij (G_O_i . V_j), since
    O_i = sum_j P_ij V_j: the FlashAttention tutorial's row sum
    ("Flash Attention Backward Pass") written out with Python loops over the
    oracle's own P on a tiny GQA input.  A transposed operand, a sum over the
    wrong axis or a head mix-up in delta() fails it."""
    B, n, H, Hk, d = 2, 7, 4, 2, 3
    q, k, v, do = (_rand((B, n, hh, d), s) for s, hh in ((1, H), (2, Hk), (3, Hk), (4, H)))
    f = orc.forward(q, k, v, causal=causal, tile=4)
    D = orc.delta(do, f["O"])
    assert D.shape == (B, H, n)
    scale = 1.0 / math.sqrt(d)
    for b in range(B):
        for h in range(H):
            g = orc.kv_head(h, H, Hk)
            for i in range(n):
                s = [scale * sum(q[b, i, h, c] * k[b, j, g, c] for c in range(d)) if (not causal or j <= i)
                     else -math.inf for j in range(n)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = sum(e)
                want = sum(e[j] / z * sum(do[b, i, h, c] * v[b, j, g, c] for c in range(d)) for j in range(n))
                assert D[b, h, i] == pytest.approx(want, rel=1e-12, abs=1e-13)
    # the backward's own full-row D is the same definition
    g = orc.backward(q, k, v, do, causal=causal, tile=4)
    np.testing.assert_allclose(g["D"], D, rtol=1e-12, atol=1e-13)


def test_metrics():
    a = np.array([1.0, 2.0, 3.0])
    assert orc.rel_l2(a, a) == 0.0 and orc.cosine(a, a) == pytest.approx(1.0)
    assert orc.rel_l2(2 * a, a) == pytest.approx(1.0)
    assert orc.cosine(-a, a) == pytest.approx(-1.0)


def test_sampled_head_group_matches_full_oracle():
    """The sampled evaluation reproduces the full oracle's rows and tiles (also
    with a sliding window of 90 keys, which cuts 64-wide tiles mid-way)."""
    for causal, (H, Hk), win in ((False, (2, 1), 0), (True, (3, 3), 0), (True, (2, 1), 90)):
        n, d = 300, 16
        q, k, v, do = _rand((1, n, H, d), 60, 1.5), _rand((1, n, Hk, d), 61, 1.5), _rand((1, n, Hk, d), 62), _rand((1, n, H, d), 63)
        heads = [0, 1] if Hk == 1 else [1]
        f = orc.forward(q, k, v, causal=causal, tile=64, window=win)
        keep = orc.mask_from_stats(f["tile_lse"], f["lse"], n, causal, 0.2, tile=64, window=win)
        g = orc.backward(q, k, v, do, keep=keep, causal=causal, tile=64, heads=heads, window=win)
        sp = orc.sampled_head_group(q, k, v, do, heads, 0.2, causal, q_tiles=[0, 2, 4], k_tiles=[0, 3, 4],
                                    tile=64, block=64, window=win)
        for hi, h in enumerate(heads):
            assert (sp["keep"][hi] == keep[0, h]).all()
            np.testing.assert_allclose(sp["lse"][hi], f["lse"][0, h], atol=1e-12)
            np.testing.assert_allclose(sp["tile_lse"][hi], f["tile_lse"][0, h], atol=1e-12)
            for j, qt in enumerate([0, 2, 4]):
                r = slice(qt * 64, min(n, qt * 64 + 64))
                np.testing.assert_allclose(sp["O"][hi][j], f["O"][0, r, h], atol=1e-12)
        for (h, qt, dq) in sp["dQ"]:
            r = slice(qt * 64, min(n, qt * 64 + 64))
            np.testing.assert_allclose(dq, g["dQ"][0, r, heads.index(h)], atol=1e-11)
        gk = orc.kv_head(heads[0], H, Hk)
        for kt in (0, 3, 4):
            r = slice(kt * 64, min(n, kt * 64 + 64))
            np.testing.assert_allclose(sp["dK"][kt], g["dK"][0, r, gk], atol=1e-11)
            np.testing.assert_allclose(sp["dV"][kt], g["dV"][0, r, gk], atol=1e-11)
        # pass 1 spread over threads: the same numbers, bit for bit
        sp4 = orc.sampled_head_group(q, k, v, do, heads, 0.2, causal, q_tiles=[0, 2, 4], k_tiles=[0, 3, 4],
                                     tile=64, block=64, window=win, threads=4)
        for hi in range(len(heads)):
            assert np.array_equal(sp4["lse"][hi], sp["lse"][hi])
            assert np.array_equal(sp4["tile_lse"][hi], sp["tile_lse"][hi])
            assert np.array_equal(sp4["D"][hi], sp["D"][hi]) and (sp4["keep"][hi] == sp["keep"][hi]).all()
        for kt in (0, 3, 4):
            assert np.array_equal(sp4["dK"][kt], sp["dK"][kt]) and np.array_equal(sp4["dV"][kt], sp["dV"][kt])


def test_sampled_rows_only_mode_and_stats_reuse():
    n, d = 260, 8
    q, k, v, do = _rand((1, n, 1, d), 70, 1.5), _rand((1, n, 1, d), 71, 1.5), _rand((1, n, 1, d), 72), _rand((1, n, 1, d), 73)
    full = orc.sampled_head_group(q, k, v, do, [0], 0.1, True, q_tiles=[1, 4], k_tiles=[0], tile=64)
    rows = orc.sampled_head_group(q, k, v, do, [0], 0.1, True, q_tiles=[1, 4], tile=64, all_rows=False)
    for qt in (1, 4):
        assert (rows["keep"][0][qt] == full["keep"][0][qt]).all()
    for (h1, t1, a), (h2, t2, b) in zip(full["dQ"], rows["dQ"]):
        assert t1 == t2
        np.testing.assert_allclose(a, b, atol=1e-12)
    again = orc.sampled_head_group(q, k, v, do, [0], 0.1, True, q_tiles=[1, 4], k_tiles=[0], tile=64,
                                   stats=full["stats"])
    np.testing.assert_allclose(again["dK"][0], full["dK"][0], atol=1e-12)


# ----------------------------------------------------------------------------
# negl_prob calibration
# ----------------------------------------------------------------------------
def test_calibrate_block_diagonal_limit_takes_pi_max():
    """Block-structured inputs: off-diagonal tile weights are ~1e-19, so every
    negl_prob in [1e-15, 1) keeps exactly the diagonal tiles, whose masked
    gradients differ from the dense ones by ~1e-10 relative (the skipped
    tiles' own weight): the first probe, pi_max, is within any target."""
    x = make_inputs(TINY)
    r = orc.calibrate(x["q"], x["k"], x["v"], x["do"], causal=False, pi_max=0.9, iters=4)
    assert r["negl_prob"] == 0.9 and r["probes"] == [(0.9, True)]
    assert r["sparsity"] == 1.0 - 1.0 / 8
    for c, rl in r["agreement"].values():
        assert c > 1 - 1e-12 and rl < 1e-8


def test_calibrate_trivial_targets():
    """Targets every gradient meets -> pi_max; a cosine above 1 that nothing
    meets (strict) -> 0, bracketed by the first bisection step."""
    w = small(384, H=1, d=64, causal=True, kind="gaussian", seed=31)
    x = make_inputs(w)
    r = orc.calibrate(x["q"], x["k"], x["v"], x["do"], causal=True, cos_min=-2.0, rel_max=np.inf, pi_max=0.5)
    assert r["negl_prob"] == 0.5 and len(r["probes"]) == 1
    r = orc.calibrate(x["q"], x["k"], x["v"], x["do"], causal=True, cos_min=1.0, rel_max=np.inf, pi_max=0.5,
                      iters=3)
    assert r["negl_prob"] == 0.0 and r["upper"] == 0.0625 and r["sparsity"] == 0.0
    assert [p for p, _ in r["probes"]] == [0.5, 0.25, 0.125, 0.0625]


def test_calibrate_with_window():
    """With a sliding window the bisection uses the windowed forward, mask and
    dense backward: negl_prob and `upper` re-checked with those functions, the
    kept tiles inside the window's candidates, and the sparsity counted over
    them."""
    w = small(900, H=2, Hk=1, d=64, causal=True, kind="gaussian", seed=24)
    x = make_inputs(w)
    win, iters = 256, 6
    r = orc.calibrate(x["q"], x["k"], x["v"], x["do"], causal=True, iters=iters, window=win)
    f = orc.forward(x["q"], x["k"], x["v"], causal=True, window=win)
    dense = orc.backward(x["q"], x["k"], x["v"], x["do"], causal=True, window=win)

    def within(pi):
        keep = orc.mask_from_stats(f["tile_lse"], f["lse"], w.n, True, pi, window=win)
        g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=True, window=win)
        ok = True
        for nm in ("dQ", "dK", "dV"):
            a, b = g[nm].ravel(), dense[nm].ravel()
            cos = float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))
            rel = float(np.linalg.norm(a - b) / np.linalg.norm(b))
            ok &= cos > 0.99 and rel < 0.1
        return keep, ok

    keep, ok = within(r["negl_prob"])
    assert ok and (keep == r["keep"]).all()
    if r["upper"] > r["negl_prob"]:
        assert not within(r["upper"])[1]
    cand = orc.candidates(w.n, True, window=win)
    assert not (r["keep"] & ~cand[None, None]).any()
    assert r["sparsity"] == pytest.approx(1.0 - r["keep"].sum() / (w.B * w.H * cand.sum()), abs=1e-15)


def test_calibrate_brackets_the_largest_value_within_targets():
    """On unstructured inputs the bisection ends with negl_prob within the
    targets and `upper` (pi_max / 2^iters above it) outside them, each checked
    here by recomputing mask, gradients and metrics; the keep sets of the
    probed values are nested (larger negl_prob keeps a subset)."""
    w = small(640, H=2, Hk=1, d=64, causal=True, kind="gaussian", seed=22)
    x = make_inputs(w)
    iters = 6
    r = orc.calibrate(x["q"], x["k"], x["v"], x["do"], causal=True, cos_min=0.99, rel_max=0.1, pi_max=0.5,
                      iters=iters)
    assert 0.0 < r["negl_prob"] < r["upper"] < 0.5
    assert r["upper"] - r["negl_prob"] == 0.5 / 2 ** iters
    f = orc.forward(x["q"], x["k"], x["v"], causal=True)
    dense = orc.backward(x["q"], x["k"], x["v"], x["do"], causal=True)

    def agree(pi):
        keep = orc.mask_from_stats(f["tile_lse"], f["lse"], w.n, True, pi)
        g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=True)
        out = {}
        for nm in ("dQ", "dK", "dV"):
            a, b = g[nm].ravel(), dense[nm].ravel()
            out[nm] = (float(a @ b / np.linalg.norm(a) / np.linalg.norm(b)),
                       float(np.linalg.norm(a - b) / np.linalg.norm(b)))
        return keep, out

    keep_lo, a_lo = agree(r["negl_prob"])
    assert all(c > 0.99 and rl < 0.1 for c, rl in a_lo.values())
    assert (keep_lo == r["keep"]).all()
    _, a_hi = agree(r["upper"])
    assert not all(c > 0.99 and rl < 0.1 for c, rl in a_hi.values())
    pis = sorted(p for p, _ in r["probes"])
    keeps = [orc.mask_from_stats(f["tile_lse"], f["lse"], w.n, True, p) for p in pis]
    for k0, k1 in zip(keeps, keeps[1:]):
        assert not (k1 & ~k0).any()


# ----------------------------------------------------------------------------
# sliding window (causal, `window` keys: i - window < j <= i)
# ----------------------------------------------------------------------------
def _torch_window_attention(q, k, v, scale, window):
    """torch fp64 attention with an explicit boolean band mask (library ops)."""
    B, n, H, d = q.shape
    G = H // k.shape[2]
    qt = q.permute(0, 2, 1, 3)
    kt = k.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vt = v.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    band = (j <= i) & (j > i - window)
    S = (scale * torch.matmul(qt, kt.transpose(-1, -2).contiguous())).masked_fill(~band, float("-inf"))
    P = torch.softmax(S, dim=-1)
    return torch.matmul(P, vt).permute(0, 2, 1, 3), torch.logsumexp(S, dim=-1)


@pytest.mark.parametrize("n,tile,window", [(50, 8, 1), (50, 8, 7), (50, 8, 8), (50, 8, 13), (37, 4, 5)])
def test_window_candidates_brute_force(n, tile, window):
    """A tile pair is a candidate iff it holds a visible (i, j): every pair enumerated."""
    T = orc.ntiles(n, tile)
    ref = np.zeros((T, T), bool)
    for i in range(n):
        for j in range(max(0, i - window + 1), i + 1):
            ref[i // tile, j // tile] = True
    assert (orc.candidates(n, True, tile, window) == ref).all()


def test_window_at_least_n_is_plain_causal():
    n = 300
    q, k, v, do = (_rand((1, n, h, 16), s) for s, h in ((1, 4), (2, 2), (3, 2), (4, 4)))
    for w in (n, n + 50):
        a = orc.forward(q, k, v, causal=True, tile=64, window=w)
        b = orc.forward(q, k, v, causal=True, tile=64)
        for key in ("O", "lse", "tile_lse"):
            assert np.array_equal(a[key], b[key])
        ga = orc.backward(q, k, v, do, causal=True, tile=64, window=w)
        gb = orc.backward(q, k, v, do, causal=True, tile=64)
        for key in ("dQ", "dK", "dV"):
            assert np.array_equal(ga[key], gb[key])
        assert (orc.candidates(n, True, 64, w) == orc.candidates(n, True, 64)).all()


def test_window_one_is_self_attention():
    """window = 1: each row sees only itself, so O = V (of its kv head),
    LSE_i = s_ii, G_S = 0 (P = I and G_P_ii = D_i), hence G_Q = G_K = 0, and
    G_V = G_O summed over the query heads of each kv head."""
    n, H, Hk, d = 200, 4, 2, 16
    q, k, v, do = _rand((1, n, H, d), 5), _rand((1, n, Hk, d), 6), _rand((1, n, Hk, d), 7), _rand((1, n, H, d), 8)
    sc = 0.25
    f = orc.forward(q, k, v, scale=sc, causal=True, tile=64, window=1)
    g = orc.backward(q, k, v, do, scale=sc, causal=True, tile=64, window=1)
    G = H // Hk
    for h in range(H):
        kv = h // G
        np.testing.assert_array_equal(f["O"][0, :, h], v[0, :, kv])
        np.testing.assert_allclose(f["lse"][0, h], sc * (q[0, :, h] * k[0, :, kv]).sum(-1), rtol=0, atol=1e-12)
    assert np.abs(g["dQ"]).max() < 1e-12 and np.abs(g["dK"]).max() < 1e-12
    np.testing.assert_allclose(g["dV"][0], do[0].reshape(n, Hk, G, d).sum(2), rtol=0, atol=1e-12)
    # only the diagonal tiles are candidates
    assert (orc.candidates(n, True, 64, 1) == np.eye(orc.ntiles(n, 64), dtype=bool)).all()


@pytest.mark.parametrize("n,window", [(300, 100), (257, 64), (200, 129)])
def test_window_matches_torch_library(n, window):
    """Forward against torch fp64 with an explicit band mask; gradients against
    torch autograd through the same masked attention."""
    H, Hk, d = 4, 2, 16
    q, k, v, do = _rand((1, n, H, d), 11), _rand((1, n, Hk, d), 12), _rand((1, n, Hk, d), 13), _rand((1, n, H, d), 14)
    sc = 0.3
    f = orc.forward(q, k, v, scale=sc, causal=True, tile=64, window=window)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    O, lse = _torch_window_attention(tq, tk, tv, sc, window)
    np.testing.assert_allclose(f["O"], O.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(f["lse"][0], lse.detach().numpy()[0], rtol=0, atol=1e-12)
    O.backward(torch.from_numpy(do))
    g = orc.backward(q, k, v, do, scale=sc, causal=True, tile=64, window=window)
    for name, t in (("dQ", tq), ("dK", tk), ("dV", tv)):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=0, atol=1e-10)
    # logsumexp over the tile LSEs is the row LSE (identity I1 under the window)
    tl = f["tile_lse"][0]
    m = tl.max(-1, keepdims=True)
    np.testing.assert_allclose(m[..., 0] + np.log(np.exp(tl - m).sum(-1)), f["lse"][0], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# backward query tiles smaller than the key tiles ("for each backward tile
# pair", BackLite README, "How It Works / Sparse Backward Masking")
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n,tile,q_tile,causal,window", [(50, 8, 4, False, 0), (50, 8, 4, True, 0),
                                                         (45, 8, 2, True, 0), (50, 8, 4, True, 7),
                                                         (37, 4, 2, True, 5), (64, 8, 8, True, 0)])
def test_candidates_query_tiles_brute_force(n, tile, q_tile, causal, window):
    """cand[qt, kt] with q_tile-row query tiles: some (i, j) with i in the query
    tile, j in the key tile, both < n, that the causal rule (and window) allow."""
    cand = orc.candidates(n, causal, tile, window, q_tile)
    Tq, Tk = -(-n // q_tile), -(-n // tile)
    assert cand.shape == (Tq, Tk)
    for qt in range(Tq):
        for kt in range(Tk):
            want = any((not causal or j <= i) and (not window or j > i - window)
                       for i in range(qt * q_tile, min(n, (qt + 1) * q_tile))
                       for j in range(kt * tile, min(n, (kt + 1) * tile)))
            assert cand[qt, kt] == want, (qt, kt)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 11)])
def test_tile_log_weights_query_tiles_brute_force(causal, window):
    """a[qt, kt] over q_tile-row query tiles, by loops over the rows; and the
    tile-row weight is exactly the larger of its two half-tile weights."""
    n, tile, q = 45, 8, 4
    g = np.random.default_rng(5)
    qq, kk, vv = (g.standard_normal((1, n, 2, 4)) * 2 for _ in range(3))
    f = orc.forward(qq, kk, vv, causal=causal, tile=tile, window=window)
    a = orc.tile_log_weights(f["tile_lse"], f["lse"], n, causal, tile, window, q_tile=q)
    cand = orc.candidates(n, causal, tile, window, q)
    for h in range(2):
        for qt in range(a.shape[2]):
            for kt in range(a.shape[3]):
                rows = range(qt * q, min(n, (qt + 1) * q))
                want = max(f["tile_lse"][0, h, i, kt] - f["lse"][0, h, i] for i in rows) if cand[qt, kt] else -np.inf
                assert a[0, h, qt, kt] == want
    a8 = orc.tile_log_weights(f["tile_lse"], f["lse"], n, causal, tile, window)
    a4 = np.concatenate([a, np.full(a.shape[:2] + (a8.shape[2] * 2 - a.shape[2], a.shape[3]), -np.inf)], axis=2)
    halves = np.maximum(a4[:, :, 0::2], a4[:, :, 1::2])
    np.testing.assert_array_equal(np.where(np.isfinite(a8), a8, -np.inf), np.where(np.isfinite(a8), halves, -np.inf))


def test_lists_from_rectangular_keep():
    keep = np.zeros((1, 1, 4, 2), bool)
    keep[0, 0] = [[1, 0], [1, 1], [0, 1], [0, 0]]
    qcnt, qidx, kcnt, kidx = orc.lists_from_keep(keep)
    assert qidx.shape == (1, 1, 4, 2) and kidx.shape == (1, 1, 2, 4)
    assert qcnt.tolist() == [[[1, 2, 1, 0]]] and kcnt.tolist() == [[[2, 2]]]
    assert qidx[0, 0, 1, :2].tolist() == [0, 1] and kidx[0, 0, 0, :2].tolist() == [0, 1]
    assert kidx[0, 0, 1, :2].tolist() == [1, 2]


def test_masked_grads_query_tiles_torch_autograd():
    """As test_masked_grads_torch_autograd with 32-row query tiles against
    64-key tiles: the element mask is keep[i // 32, j // 64]."""
    n, d, t, q = 192, 8, 64, 32
    qq, kk, vv, do = _rand((1, n, 1, d), 44, 1.5), _rand((1, n, 1, d), 45, 1.5), _rand((1, n, 1, d), 46), _rand((1, n, 1, d), 47)
    sc = 0.5
    for causal in (False, True):
        keep = orc.candidates(n, causal, t, q_tile=q).copy()
        keep[5, 0] = False
        keep[2, 1] = False
        keep[3, 1] = True
        g = orc.backward(qq, kk, vv, do, keep=keep[None, None], scale=sc, causal=causal, tile=t, q_tile=q)
        tq, tk, tv = (torch.from_numpy(x[0, :, 0]).requires_grad_() for x in (qq, kk, vv))
        tdo = torch.from_numpy(do[0, :, 0])
        S = sc * tq @ tk.T
        if causal:
            S = S.masked_fill(~torch.ones(n, n, dtype=torch.bool).tril(), float("-inf"))
        P = torch.softmax(S, -1)
        O = P @ tv
        dS_dense, = torch.autograd.grad(O, S, tdo, retain_graph=True)
        M = torch.from_numpy(np.kron(keep, np.ones((q, t), bool))[:n, :n])
        dQ, dK = torch.autograd.grad(S, (tq, tk), torch.where(M, dS_dense, 0.0))
        dV, = torch.autograd.grad(torch.where(M, P, 0.0).detach() @ tv, tv, tdo)
        np.testing.assert_allclose(g["dQ"][0, :, 0], dQ.numpy(), atol=1e-11)
        np.testing.assert_allclose(g["dK"][0, :, 0], dK.numpy(), atol=1e-11)
        np.testing.assert_allclose(g["dV"][0, :, 0], dV.numpy(), atol=1e-11)


def test_query_tile_selection_invariants():
    """With half-height query tiles each half keeps its own rows' skipped mass
    below negl_prob (I3 per tile), keeps at least one key tile (I5), and is
    never less sparse than the full-height mask: a full tile's weight is the
    larger of its halves', so every weight-sorted prefix the full tile skips,
    each half can skip too."""
    x = make_inputs(small(1000, H=2, d=64, causal=True, kind="blocks", seed=3))
    f = orc.forward(x["q"], x["k"], x["v"], causal=True)
    p = np.exp(f["tile_lse"] - f["lse"][..., None])
    for pi in (0.01, 0.05, 0.2):
        k128 = orc.mask_from_stats(f["tile_lse"], f["lse"], 1000, True, pi)
        k64 = orc.mask_from_stats(f["tile_lse"], f["lse"], 1000, True, pi, q_tile=64)
        assert k64.shape == (1, 2, 16, 8) and k64.sum(axis=3).min() >= 1
        for qt in range(16):
            rows = p[0, :, qt * 64:min(1000, (qt + 1) * 64), :]
            assert ((rows * ~k64[0, :, qt, None, :]).sum(-1) < pi).all()
        assert k64.sum() <= 2 * k128.sum()


def test_sampled_head_group_query_tiles_match_full_oracle():
    """The sampled evaluation with 32-row query tiles against 64-key tiles
    reproduces the full oracle's mask, G_Q rows and G_K/G_V key tiles."""
    n, d, t, q = 300, 16, 64, 32
    for causal, win in ((False, 0), (True, 0), (True, 90)):
        qq, kk, vv, do = (_rand((1, n, 2, d), 70, 1.5), _rand((1, n, 1, d), 71, 1.5), _rand((1, n, 1, d), 72),
                          _rand((1, n, 2, d), 73))
        f = orc.forward(qq, kk, vv, causal=causal, tile=t, window=win)
        keep = orc.mask_from_stats(f["tile_lse"], f["lse"], n, causal, 0.2, tile=t, window=win, q_tile=q)
        g = orc.backward(qq, kk, vv, do, keep=keep, causal=causal, tile=t, window=win, q_tile=q)
        sp = orc.sampled_head_group(qq, kk, vv, do, [0, 1], 0.2, causal, q_tiles=[0, 2, 4], k_tiles=[0, 3, 4],
                                    tile=t, block=t, window=win, q_tile=q)
        for h in range(2):
            assert (sp["keep"][h] == keep[0, h]).all()
        for (h, qt, dq) in sp["dQ"]:
            r = slice(qt * t, min(n, qt * t + t))
            np.testing.assert_allclose(dq, g["dQ"][0, r, h], atol=1e-11)
        for kt in (0, 3, 4):
            r = slice(kt * t, min(n, kt * t + t))
            np.testing.assert_allclose(sp["dK"][kt], g["dK"][0, r, 0], atol=1e-11)
            np.testing.assert_allclose(sp["dV"][kt], g["dV"][0, r, 0], atol=1e-11)
