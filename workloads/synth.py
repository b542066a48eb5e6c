"""Seeded synthetic inputs for the BackLite attention workloads.

The pages measure BackLite on Wan 2.1 video latents (32k tokens for a 5 s
480p clip, 75k for 720p) and on Nanochat / LLM context extension (8k -> 128k);
none of those weights or datasets exist here, so these generators stand in for
them with the same shapes and a comparable attention structure
("Introducing BackLite", Introduction).

This module holds no attention arithmetic: it only draws Q, K, V and G_O.
Both the oracle tests and the GPU path consume its tensors.

Randomness: numpy PCG64 streams derived from ``SeedSequence([seed, stream])``;
each large tensor is filled in fixed 4 Mi-element chunks, chunk c drawing from
``SeedSequence([seed, stream]).spawn(nchunks)[c]``, so the values do not depend
on the number of threads used.  Streams: 0 = per-head structure, 1 = Q noise,
2 = K noise, 3 = V, 4 = G_O.  Values are drawn in fp32 and rounded to bf16
(round-to-nearest-even) by torch.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np
import torch

CHUNK = 1 << 22


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hk: int
    n: int
    d: int
    causal: bool
    kind: str                      # "blocks" | "positional" | "fourier3d" | "gaussian"
    negl_probs: tuple = (0.05,)
    grid: tuple = ()               # (t, y, x) for fourier3d
    period: float = 512.0          # longest positional period
    seed: int = 0
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads.  Shapes follow the pages: the tiny block-structured case,
# an 8k causal GQA LLM, the Wan 2.1 480p / 720p latent grids (21 frames x 30x52
# and 21 x 45x80 tokens) and a 128k causal LLM.
TINY = Workload("tiny-blocks-1k", 1, 2, 2, 1024, 64, False, "blocks", (0.05, 0.0))
LLM8K = Workload("llm-8k-causal-gqa", 1, 32, 8, 8192, 128, True, "positional",
                 (0.0, 0.01, 0.05, 0.1), period=512.0)
DIT480 = Workload("dit-480p-32k", 1, 40, 40, 32760, 128, False, "fourier3d",
                  (0.05, 0.0), grid=(21, 30, 52))
DIT720 = Workload("dit-720p-75k", 1, 40, 40, 75600, 128, False, "fourier3d",
                  (0.01, 0.05, 0.1, 0.0), grid=(21, 45, 80))
LLM128K = Workload("llm-128k-causal", 1, 8, 8, 131072, 128, True, "positional",
                   (0.1, 0.0), period=2048.0)

ALL = {w.name: w for w in (TINY, LLM8K, DIT480, DIT720, LLM128K)}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(seed: int, stream: int, count: int) -> np.ndarray:
    out = np.empty(count, np.float32)
    nch = max(1, (count + CHUNK - 1) // CHUNK)
    seeds = np.random.SeedSequence([seed, stream]).spawn(nch)

    def fill(c):
        g = np.random.Generator(np.random.PCG64(seeds[c]))
        s = c * CHUNK
        e = min(count, s + CHUNK)
        g.standard_normal(e - s, dtype=np.float32, out=out[s:e])

    if nch == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nch)))
    return out


def _positional(n: int, d: int, period: float) -> np.ndarray:
    """Sinusoidal position code: pairs (cos, sin) of 2*pi*t/P_f with a geometric
    ladder of periods from `period` down to 4 tokens."""
    nf = d // 2
    f = np.arange(nf, dtype=np.float64)
    P = period * (4.0 / period) ** (f / max(1, nf - 1))
    t = np.arange(n, dtype=np.float64)[:, None]
    ang = 2.0 * math.pi * t / P[None, :]
    pos = np.empty((n, d), np.float64)
    pos[:, 0::2] = np.cos(ang)
    pos[:, 1::2] = np.sin(ang)
    return pos.astype(np.float32)


def _structure(w: Workload) -> np.ndarray | None:
    """Shared Q/K structure term, shape [n, Hk, d] fp32 (or [n, 1, d])."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 0])))
    n, d, Hk = w.n, w.d, w.Hk
    if w.kind == "blocks":
        # 128-token clusters, one centre per cluster and kv head, scaled by 3.
        ncl = (n + 127) // 128
        c = rng.standard_normal((Hk, ncl, d)).astype(np.float32)
        cl = np.arange(n) // 128
        return 3.0 * np.transpose(c[:, cl, :], (1, 0, 2))
    if w.kind == "positional":
        return 2.5 * _positional(n, d, w.period)[:, None, :]
    if w.kind == "fourier3d":
        T_, Y_, X_ = w.grid
        assert T_ * Y_ * X_ == n, "grid must tile the sequence"
        tt, yy, xx = np.meshgrid(np.arange(T_), np.arange(Y_), np.arange(X_), indexing="ij")
        coords = np.stack([tt.ravel(), yy.ravel(), xx.ravel()], 1).astype(np.float64)  # t-major raster
        R = 16
        out = np.empty((n, Hk, d), np.float32)
        for g in range(Hk):
            a = rng.standard_normal((R, d))
            u = rng.standard_normal((R, 3))
            u /= np.linalg.norm(u, axis=1, keepdims=True)
            lam = np.exp(rng.uniform(math.log(4.0), math.log(32.0), R))
            phi = rng.uniform(0.0, 2.0 * math.pi, R)
            feat = np.cos(2.0 * math.pi * (coords @ u.T) / lam[None, :] + phi[None, :])  # [n, R]
            out[:, g, :] = (3.0 * math.sqrt(2.0 / R) * (feat @ a)).astype(np.float32)
        return out
    if w.kind == "gaussian":
        return None
    raise ValueError(f"unknown workload kind {w.kind}")


def make_inputs(w: Workload, device: str | torch.device = "cpu") -> dict:
    """Q, K, V, G_O as bf16 tensors, Q/G_O [B,n,H,d], K/V [B,n,Hk,d]."""
    B, n, H, Hk, d = w.B, w.n, w.H, w.Hk, w.d
    G = H // Hk
    st = _structure(w)
    q = _normal(w.seed, 1, B * n * H * d).reshape(B, n, H, d)
    k = _normal(w.seed, 2, B * n * Hk * d).reshape(B, n, Hk, d)
    if st is not None:
        if st.shape[1] == 1:
            q += st[None]
            k += st[None]
        else:
            q += np.repeat(st, G, axis=1)[None]
            k += st[None]
    if w.kind == "positional":
        k[:, :4] *= 4.0                       # four attention-sink keys with norm x4
    v = _normal(w.seed, 3, B * n * Hk * d).reshape(B, n, Hk, d)
    do = _normal(w.seed, 4, B * n * H * d).reshape(B, n, H, d)
    out = {}
    for name, arr in (("q", q), ("k", k), ("v", v), ("do", do)):
        out[name] = torch.from_numpy(arr).to(torch.bfloat16).to(device)
    return out


def small(n: int, H: int = 2, Hk: int | None = None, d: int = 64, causal: bool = False,
          kind: str = "gaussian", B: int = 1, seed: int = 0, **kw) -> Workload:
    """A small ad-hoc workload for parity cases (ragged n, GQA, causal)."""
    return Workload(f"small-{kind}-b{B}h{H}k{Hk or H}n{n}d{d}{'c' if causal else ''}",
                    B, H, Hk or H, n, d, causal, kind, seed=seed, **kw)
