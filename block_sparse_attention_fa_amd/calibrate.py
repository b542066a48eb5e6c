"""negl_prob calibration on the GPU path.

The pages describe a tool that sets the weight BackLite neglects so that the
gradients stay within a minimum cosine similarity and a maximum relative L2
difference of exact attention's ("Introducing BackLite", "Experiments" and
"Preliminary results with Wan 2.1 1.3b", Fig. 4: cosine > 0.99, relative L2
< 0.1; README "Overview", Tunable).  They do not give its search.  This one
bisects negl_prob, which relies on the keep sets shrinking as negl_prob
grows: pi_max is tried first, then `iters` halvings of [lo, hi] with lo always
within the targets (lo = 0 is the dense backward).

Every forward, mask and backward runs in the library's kernels; the dense
reference is the same library at negl_prob = 0.  The similarity numbers come
from the library's reduction kernel (backlite_similarity_sums: fp64 sums of
a*b, a*a, b*b and (a-b)^2); only the final square roots and divisions of those
four scalars are taken on the host.
"""
from __future__ import annotations

import math

import torch

from . import _lib

GRADS = ("dQ", "dK", "dV")


def _agreement(g, ref) -> dict:
    """{name: (cosine, rel-L2)} of each gradient against the reference."""
    sums = [_lib.similarity_sums(a, r) for a, r in zip(g, ref)]
    out = {}
    for nm, s in zip(GRADS, sums):
        ab, aa, bb, dd = s[:4].tolist()
        cos = 1.0 if aa == 0.0 and bb == 0.0 else ab / math.sqrt(aa * bb) if aa > 0 and bb > 0 else 0.0
        rel = math.sqrt(dd / bb) if bb > 0 else math.sqrt(dd)
        out[nm] = (cos, rel)
    return out


def _within(agree, cos_min, rel_max) -> bool:
    return all(c > cos_min and r < rel_max for c, r in agree.values())


def calibrate_negl_prob(q, k, v, do, causal=False, scale=None, cos_min=0.99, rel_max=0.1, pi_max=0.5,
                        iters=8, window=0) -> dict:
    """The largest negl_prob in [0, pi_max] (to pi_max / 2^iters) whose sparse
    gradients G_Q, G_K, G_V all have cosine > cos_min and rel-L2 < rel_max
    against the dense ones, for this batch (q, k, v [B, n, H(_k), d] bf16 and
    the output gradient do, on the GPU).

    Returns negl_prob, upper (the smallest value tried outside the targets, or
    pi_max), agreement {name: (cosine, rel-L2)} at negl_prob, sparsity at
    negl_prob, and the probes [(negl_prob, within targets)] in order.
    window > 0 (causal only): a sliding-window layer; the dense reference has
    the same window.
    """
    if not (0.0 < pi_max < 1.0) or iters < 0:
        raise ValueError("pi_max must be in (0, 1) and iters >= 0")
    B, n, H, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o, lse, tl, olo = _lib.fwd(q, k, v, scale=scale, causal=causal, with_residual=True, window=window)
    dense_lists = _lib.mask(None, lse, n, causal, 0.0, window=window)
    ws = _lib.bwd_workspace(q, k, dense_lists, causal=causal, window=window)
    ref = tuple(t.clone() for t in _lib.bwd(q, k, v, o, do, lse, dense_lists, scale=scale, causal=causal,
                                            workspace=ws, o_lo=olo, window=window))
    stats = torch.zeros(2, dtype=torch.int64, device=q.device)

    def probe(pi):
        stats.zero_()
        m = _lib.mask(tl, lse, n, causal, pi, stats=stats, window=window)
        g = _lib.bwd(q, k, v, o, do, lse, m, scale=scale, causal=causal, workspace=ws, o_lo=olo, window=window)
        agree = _agreement(g, ref)
        s = stats.tolist()
        return _within(agree, cos_min, rel_max), agree, 1.0 - s[1] / s[0]

    probes = []
    ok, agree, sp = probe(pi_max)
    probes.append((pi_max, ok))
    if ok:
        return dict(negl_prob=pi_max, upper=pi_max, agreement=agree, sparsity=sp, probes=probes)
    lo, hi = 0.0, pi_max
    best_agree, best_sp = _agreement(ref, ref), 0.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        ok, agree, sp = probe(mid)
        probes.append((mid, ok))
        if ok:
            lo, best_agree, best_sp = mid, agree, sp
        else:
            hi = mid
    return dict(negl_prob=lo, upper=hi, agreement=best_agree, sparsity=best_sp, probes=probes)
