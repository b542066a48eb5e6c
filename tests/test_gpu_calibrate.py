"""negl_prob calibration on the GPU path against the oracle's calibration
(the same bisection over the oracle's fp64 forward, mask and backward).  GPU only."""
import pytest
import torch

from helpers import flush_print, gpu_available
from oracle import backlite_oracle as orc
from workloads import TINY, make_inputs, small

pytestmark = pytest.mark.gpu


def _gpu(w):
    if not gpu_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fa_amd as bl
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    return bl, x, {k: v.to(dev) for k, v in x.items()}


@pytest.mark.parametrize("w,win", [(small(640, H=2, Hk=1, d=64, causal=True, kind="gaussian", seed=22), 0),
                                   (small(768, H=4, Hk=2, d=128, causal=False, kind="gaussian", seed=23), 0),
                                   (small(900, H=2, Hk=1, d=64, causal=True, kind="gaussian", seed=24), 256)],
                         ids=["causal-gqa", "noncausal-gqa", "causal-window256"])
def test_calibration_matches_oracle(w, win):
    bl, x, xg = _gpu(w)
    iters = 6
    got = bl.calibrate_negl_prob(xg["q"], xg["k"], xg["v"], xg["do"], causal=w.causal, iters=iters, window=win)
    ref = orc.calibrate(x["q"], x["k"], x["v"], x["do"], causal=w.causal, iters=iters, window=win)
    flush_print(f"  gpu {got['negl_prob']} (sparsity {got['sparsity']:.3f}) oracle {ref['negl_prob']} "
                f"(sparsity {ref['sparsity']:.3f}); probes {got['probes']} / {ref['probes']}")
    # the probes decide identically unless an oracle metric sits within the GPU's
    # gradient error (<= 1e-2 rel-L2, far less in cosine) of a target
    margin = min(min(abs(c - 0.99), abs(r - 0.1)) for c, r in ref["agreement"].values())
    if got["probes"] != ref["probes"]:
        assert margin < 1e-2, f"probe decisions differ with margin {margin}"
    else:
        assert got["negl_prob"] == ref["negl_prob"] and abs(got["sparsity"] - ref["sparsity"]) < 1e-12
    for nm in ("dQ", "dK", "dV"):
        cg, rg = got["agreement"][nm]
        co, ro = ref["agreement"][nm]
        assert abs(cg - co) < 2e-3 and abs(rg - ro) < 1e-2, (nm, cg, co, rg, ro)


def test_calibration_block_diagonal_takes_pi_max():
    bl, x, xg = _gpu(TINY)
    got = bl.calibrate_negl_prob(xg["q"], xg["k"], xg["v"], xg["do"], causal=False, pi_max=0.9, iters=4)
    assert got["negl_prob"] == 0.9 and got["probes"] == [(0.9, True)]
    assert abs(got["sparsity"] - (1.0 - 1.0 / 8)) < 1e-12
