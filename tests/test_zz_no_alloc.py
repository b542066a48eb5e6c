"""The allocation-free backward entry point (backlite_bwd_noalloc) through the
C ABI: two calls in a row on one GPU, the second with a smaller input, each
checked against backlite_bwd with a base workspace (the same recompute path)
bit for bit, and against the oracle to the gradient bound.  GPU only."""
import pytest
import torch

from helpers import assert_close_grad, flush_print, gpu_available
from oracle import backlite_oracle as orc
from workloads import make_inputs, small

pytestmark = pytest.mark.gpu

NEGL = 0.05
# first call: a causal GQA problem whose sink-like key tiles split their lists;
# second: a smaller non-causal one with a ragged tail
CASES = [small(1536, H=4, Hk=1, d=64, causal=True, kind="positional", seed=9, period=512.0),
         small(383, H=3, Hk=1, d=128, causal=False, kind="gaussian", seed=6)]


def _run(bl, w):
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    xg = {k: v.to(dev) for k, v in x.items()}
    o, lse, tl, olo = bl.fwd(xg["q"], xg["k"], xg["v"], causal=w.causal, with_residual=True)
    m = bl.mask(tl, lse, w.n, w.causal, NEGL)
    ref_ws = bl._lib.bwd_workspace(xg["q"], xg["k"], m, stored_tiles=0)
    want = bl.bwd(xg["q"], xg["k"], xg["v"], o, xg["do"], lse, m, causal=w.causal, o_lo=olo, workspace=ref_ws)
    out = tuple(torch.full_like(t, float("nan")) for t in want)
    torch.cuda.synchronize()
    got = bl._lib.bwd_noalloc(xg["q"], xg["k"], xg["v"], o, xg["do"], lse, m, out, causal=w.causal, o_lo=olo)
    torch.cuda.synchronize()
    return x, m, want, got


def test_noalloc_matches_backward_twice_second_smaller():
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    for w in CASES:
        flush_print(f"[case] noalloc {w.name}")
        x, m, want, got = _run(bl, w)
        for name, a, b in zip(("dQ", "dK", "dV"), got, want):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name} differs from backlite_bwd"
        keep = m["keep"].cpu().numpy().astype(bool)
        g = orc.backward(x["q"], x["k"], x["v"], x["do"], keep=keep, causal=w.causal)
        for name, a, r in (("dQ", got[0], g["dQ"]), ("dK", got[1], g["dK"]), ("dV", got[2], g["dV"])):
            rl, cs = assert_close_grad(name, a.cpu(), r)
            flush_print(f"  {name}: rel-L2 {rl:.2e} cos {cs:.6f}")
