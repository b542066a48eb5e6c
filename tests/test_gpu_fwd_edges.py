"""Forward parity at the boundaries of its key-tile processing: sequence
lengths around the 64-key halves and 128-key tiles the kernel consumes
(a ragged last tile is copied with a byte range that zero-fills its padding
rows, and each half masks its padded keys on its own), for both head sizes,
causal and not, and with sliding windows whose edge cuts inside a half.
Checks O, the row LSE, the tile LSE and the compact statistics against the
fp64 oracle.  GPU only."""
import numpy as np
import pytest
import torch

from helpers import assert_close_out, flush_print, gpu_available, packed_to_rows
from oracle import backlite_oracle as orc
from workloads import make_inputs, small

pytestmark = pytest.mark.gpu

LENGTHS = [63, 64, 65, 127, 191, 193, 255, 257]
CASES = [(n, d, causal, 0) for n in LENGTHS for d in (64, 128) for causal in (False, True)]
CASES += [(193, 128, True, 70), (257, 64, True, 100)]
IDS = [f"n{n}-d{d}-{'causal' if c else 'full'}" + (f"-w{w}" if w else "") for n, d, c, w in CASES]


@pytest.mark.parametrize("n,d,causal,window", CASES, ids=IDS)
def test_forward_edges(n, d, causal, window):
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    from block_sparse_attention_fa_amd import _lib
    w = small(n, H=2, Hk=1, d=d, causal=causal, kind="gaussian", seed=n + d)
    flush_print(f"[case] {w.name} window={window}")
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (x[nm].to(dev) for nm in ("q", "k", "v"))
    tw = torch.empty(_lib.tile_w_elems(w.B, w.H, n, causal), dtype=torch.float64, device=dev)
    o, lse, tl = bl.fwd(q, k, v, causal=causal, window=window, tile_w=tw)
    torch.cuda.synchronize()
    ref = orc.forward(x["q"], x["k"], x["v"], causal=causal, window=window)
    assert_close_out("O", o.cpu(), ref["O"])
    assert_close_out("lse", lse.cpu(), ref["lse"])
    got = packed_to_rows(tl.cpu().numpy(), w.B, w.H, n, causal)
    rt = ref["tile_lse"]
    assert not np.isnan(got).any()
    sel = np.isfinite(rt) & (rt - ref["lse"][..., None] > -60.0)
    assert_close_out("tile_lse", got[sel], rt[sel])
    # tiles the oracle finds empty (outside the window) are -inf on the GPU too
    cand = orc.candidates(n, causal, window=window)
    rows = np.arange(n)
    empty = ~np.isfinite(rt) & cand[rows // 128][None, None]
    assert np.isneginf(got[empty]).all()
    # compact statistics: the oracle's log-weights per 64-row half on the
    # forward's own fp32 outputs, bit for bit
    want = orc.tile_log_weights(got, lse.cpu().numpy().astype(np.float64), n, causal, window=window, q_tile=64)
    T, Tq = (n + 127) // 128, (n + 63) // 64
    pairs = T * (T + 1) // 2 if causal else T * T
    tw2 = tw.cpu().numpy().reshape(w.B, w.H, pairs, 2)
    for qt in range(Tq):
        for kt in range(T):
            if not cand[qt // 2, kt]:
                continue
            p = (qt // 2) * ((qt // 2) + 1) // 2 + kt if causal else (qt // 2) * T + kt
            np.testing.assert_array_equal(tw2[:, :, p, qt % 2], want[:, :, qt, kt])
