#!/usr/bin/env python3
"""Benchmark of the BackLite hot path on one MI355X.

One step = the whole path over one batch of synthetic input resident in HBM:
forward with tile statistics -> mask from statistics -> block-sparse backward.
Default workload: the 32k-token video-DiT shape (B=1, H=40, n=32760 = 21x30x52
latent grid, d=128, bf16, non-causal, negl_prob=0.05).

Printed JSON line (rank 0): value = dense-equivalent backward throughput,
10*d*B*H*n^2 FLOP / sparse-backward time, in TFLOP/s; plus forward, mask and
backward ms, sparsity, the executed-tile MFMA fraction of the bf16 dense peak,
the backward speedup over the same library's dense (negl_prob = 0) backward,
the roofline of the dominant kernel from per-launch HIP events, and the fp64
oracle timed on the host on a bounded sample.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload dit-480p-32k]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse attn bwd ms + dense-equiv TFLOP/s & MFMA % peak, 32k DiT, negl_prob=0.05"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TILE = 128


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dit-480p-32k")
    ap.add_argument("--negl", type=float, default=None, help="negl_prob (default: the workload's first)")
    ap.add_argument("--stats", choices=["rows", "compact"], default="rows",
                    help="statistics the mask reads: per-row tile LSEs, or the forward's compact per-pair log-weights")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window of a causal workload (key j visible to query i iff i - window < j <= i)")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--cpu-rows", type=int, default=20480,
                    help="query rows per sampled head in the oracle's timed sample")
    ap.add_argument("--cpu-heads", default=None,
                    help="comma-separated query heads the oracle is timed on (default: every head up to 8k "
                         "tokens, else the first, middle and last head, or first and last with H < 16)")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-backward comparison")
    ap.add_argument("--grad-check", action="store_true",
                    help="report cosine and rel-L2 of the sparse gradients against the dense (negl_prob = 0) ones")
    ap.add_argument("--gq-path", choices=["stored", "recompute", "atomic"], default="stored",
                    help="G_Q from stored bf16 G_S tiles (workspace slots), by recomputation, or by fp32 atomics "
                         "inside the G_K/G_V pass (fused single pass)")
    ap.add_argument("--gs-budget-gb", type=float, default=None,
                    help="device memory for G_S slots (default: a slot for every kept tile when they fit); "
                         "query tiles past the budget recompute G_Q")
    ap.add_argument("--q-tile", type=int, choices=[64, 128], default=128,
                    help="rows of the backward's query tiles (the headline uses the workload's 128x128 tiles)")
    ap.add_argument("--no-q64", action="store_true",
                    help="skip the extra measurement of the sparse backward with 64-row query tiles")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (scale for memory counters)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("bwd.hip", "bwd_dkdv.h", "bwd_dkdv_d128_gs.hip", "bwd_gs.hip", "bwd_common.h", "bl_device.h"):
        with open(os.path.join(ROOT, "block_sparse_attention_fa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """Bytes per launch of the dK/dV kernel from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated: L2-miss traffic, Infinity Cache
    hits included), if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"dkdv_{workload}_traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("l2_miss_bytes_per_launch")


def visible_pairs(rows, window):
    """(i, j) pairs with j <= i < rows that a sliding window of `window` keys
    allows (window 0: all of them)."""
    if window <= 0 or window >= rows:
        return rows * (rows + 1) / 2
    return window * (window + 1) / 2 + (rows - window) * float(window)


def default_cpu_heads(w):
    if w.n <= 8192:
        return list(range(w.H))
    return [0, w.H // 2, w.H - 1] if w.H >= 16 else [0, w.H - 1]


def cpu_baseline(w, x_cpu, heads, negl, rows, window=0):
    """fp64 oracle on the sampled query heads, query rows [0, rows) of each:
    forward, mask and backward of those rows against all keys.  Rate = the
    sample's dense-equivalent backward FLOP / the oracle's backward seconds;
    the full job's oracle backward time is extrapolated from that rate (x H
    heads and the full row count)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import backlite_oracle as orc
    n, d = w.n, w.d
    rows = min(rows, n)
    rr = np.arange(rows)
    nt = (rows + TILE - 1) // TILE
    per_head = []
    fl_total = 0.0
    for j, h in enumerate(heads):
        q, k, v, do = (orc.to_f64(x_cpu[nm][:, :, j:j + 1]) for nm in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        f = orc.forward(q, k, v, causal=w.causal, rows=rr, window=window)
        t1 = time.perf_counter()
        # tile weights / selection on the sampled query tiles only
        tl = np.full((1, 1, n, f["tile_lse"].shape[-1]), -np.inf)
        ls = np.zeros((1, 1, n))
        tl[:, :, :rows] = f["tile_lse"]
        ls[:, :, :rows] = f["lse"]
        a = orc.tile_log_weights(tl, ls, n, w.causal, window=window)
        cand = orc.candidates(n, w.causal, window=window).copy()
        cand[nt:] = False                       # only the sampled query tiles
        keep = orc.select_keep(a, cand, negl)
        t2 = time.perf_counter()
        orc.backward(q, k, v, do, keep=keep, causal=w.causal, q_rows=rr, window=window)
        t3 = time.perf_counter()
        per_head.append((h, t1 - t0, t2 - t1, t3 - t2))
        # dense-equivalent: every (row, key) pair the causal rule (and window) allows
        fl_total += 10.0 * d * (visible_pairs(rows, window) if w.causal else rows * n)
        log(f"[bench] oracle head {h}: forward {t1 - t0:.2f} s, mask {t2 - t1:.2f} s, backward {t3 - t2:.2f} s")
    bwd_s = sum(p[3] for p in per_head)
    rate = fl_total / bwd_s / 1e12
    full_fl = 10.0 * d * w.B * w.H * (visible_pairs(n, window) if w.causal else float(n) * n)
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return {
        "value": rate,
        "unit": "TFLOP/s (dense-equivalent backward)",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"query heads {','.join(str(h) for h in heads)}, rows 0-{rows - 1} of each, of the {w.name} "
                   f"problem against all {n} keys, fp64 numpy; per head (forward / mask / backward s): "
                   + "; ".join(f"h{h} {a:.2f}/{b:.2f}/{c:.2f}" for h, a, b, c in per_head)),
        "heads": list(heads),
        "rows_per_head": rows,
        "bwd_s": bwd_s,
        "fwd_s": sum(p[1] for p in per_head),
        "full_job_bwd_s_extrapolated": full_fl / (rate * 1e12),
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the hot path would shard by (batch, kv-head group) with no exchange; multi-GPU runs are "
              "not implemented", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_attention_fa_amd as bl
    from block_sparse_attention_fa_amd import _lib
    from workloads import ALL, make_inputs

    w = ALL[args.workload]
    negl = w.negl_probs[0] if args.negl is None else args.negl
    B, H, Hk, n, d, causal = w.B, w.H, w.Hk, w.n, w.d, w.causal
    win = args.window
    if win < 0 or (win and not causal):
        sys.exit(f"--window {win}: a sliding window needs a causal workload and window >= 0")
    dev = torch.device("cuda:0")
    log(f"[bench] workload {w.name}: B={B} H={H} H_k={Hk} n={n} d={d} causal={causal} window={win} "
        f"negl_prob={negl}")
    t = time.time()
    x = make_inputs(w)
    log(f"[bench] inputs generated in {time.time() - t:.1f} s")
    cpu_heads = ([int(h) for h in args.cpu_heads.split(",")] if args.cpu_heads else default_cpu_heads(w))
    if any(h < 0 or h >= H for h in cpu_heads):
        sys.exit(f"--cpu-heads {args.cpu_heads}: heads must lie in [0, {H})")
    # the oracle's sample: the chosen query heads and their key/value heads
    x_cpu = {nm: x[nm][:, :, cpu_heads].contiguous() for nm in ("q", "do")}
    x_cpu.update({nm: x[nm][:, :, [h // (H // Hk) for h in cpu_heads]].contiguous() for nm in ("k", "v")})
    q, k, v, do = (x[nm].to(dev) for nm in ("q", "k", "v", "do"))
    del x
    T = (n + TILE - 1) // TILE

    if args.copy_calibration_mib:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give the
        # scale between those counters and bytes moved
        nb = args.copy_calibration_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # every buffer allocated once, outside the timed region
    tl = torch.empty(_lib.tile_lse_elems(B, H, n, causal), dtype=torch.float32, device=dev)
    compact = args.stats == "compact"
    tw = torch.empty(_lib.tile_w_elems(B, H, n, causal), dtype=torch.float64, device=dev) if compact else None
    stats = torch.zeros(2, dtype=torch.int64, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stored = args.gq_path == "stored"
    atomic = args.gq_path == "atomic"
    if atomic and args.q_tile != TILE:
        sys.exit("--gq-path atomic takes 128-row query tiles")

    def backward(lists, ws, o, lse, olo):
        if atomic:
            return _lib.bwd_atomic(q, k, v, o, do, lse, lists, causal=causal, window=win, workspace=ws,
                                   out=(dq, dk, dv), o_lo=olo)
        return bl.bwd(q, k, v, o, do, lse, lists, causal=causal, window=win, workspace=ws, out=(dq, dk, dv),
                      o_lo=olo)

    def workspace(lists):
        # G_S slots: a budget, or one slot per kept tile when they fit in free
        # device memory (counted once here, outside the timed region)
        if atomic:
            return _lib.bwd_atomic_workspace(q, k)
        if not stored:
            return _lib.bwd_workspace(q, k, lists, stored_tiles=0)
        if args.gs_budget_gb is not None:
            return _lib.bwd_workspace(q, k, lists, stored_tiles="auto", causal=causal, window=win,
                                      gs_budget_bytes=int(args.gs_budget_gb * 1e9))
        tiles = int(lists["qcnt"].sum().item())
        free, _ = torch.cuda.mem_get_info(dev)
        tiles = min(tiles, max(0, (free - (4 << 30)) // _lib.slot_bytes(lists.get("q_tile", TILE))))
        return _lib.bwd_workspace(q, k, lists, stored_tiles=tiles)

    QT = args.q_tile
    o0, lse0, _, _ = bl.fwd(q, k, v, causal=causal, window=win, tile_lse=tl, with_residual=True)
    ws = workspace(bl.mask(tl, lse0, n, causal, negl, window=win, q_tile=QT))
    del o0, lse0

    def step(rec=None):
        o, lse, _, olo = bl.fwd(q, k, v, causal=causal, window=win, tile_lse=tl, with_residual=True, tile_w=tw)
        if rec is not None:
            rec[0].record()
        if compact:
            m = _lib.mask_compact(tw, B, H, n, causal, negl, stats=stats, window=win, q_tile=QT)
        else:
            m = bl.mask(tl, lse, n, causal, negl, window=win, stats=stats, q_tile=QT)
        if rec is not None:
            rec[1].record()
        backward(m, ws, o, lse, olo)
        return o, lse, olo

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stats.zero_()

    # the timed steps run without the library's per-kernel event timer (its
    # two event records per launch are visible at small sizes); the per-kernel
    # times come from a separate pass of the same number of steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        ev[i][0].record()
        step(rec=(ev[i][1], ev[i][2]))
        ev[i][3].record()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    st = stats.cpu().tolist()
    _lib.profile_reset()
    _lib.profile_enable(True)
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    _lib.profile_enable(False)
    prof = _lib.profile_read()
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    mask_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    bwd_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / args.steps
    cand, kept = st[0] / args.steps, st[1] / args.steps
    sparsity = 1.0 - kept / cand if cand else 0.0
    has_slots = not atomic and ws.numel() > _lib.bwd_workspace_bytes(B, H, Hk, n, d)
    gq_state = _lib.bwd_state(ws, B, H, Hk, n, d) if has_slots else (False, int(kept), 0)
    gq_stored = gq_state[0]
    ws_bytes = ws.numel()
    peak_mem = torch.cuda.max_memory_allocated(dev)

    # the same library's dense backward (negl_prob = 0: every candidate tile)
    dense_ms = None
    dense_stored = None
    sparse_grads = (dq.clone(), dk.clone(), dv.clone()) if (args.grad_check and not args.no_dense) else None
    if not args.no_dense:
        o, lse, olo = step()
        md = bl.mask(None, lse, n, causal, 0.0, window=win)  # dense: the query-tile height does not matter
        del ws
        ws = workspace(md)
        for _ in range(max(1, args.warmup)):
            backward(md, ws, o, lse, olo)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            backward(md, ws, o, lse, olo)
        e1.record()
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / args.steps
        dense_stored = _lib.bwd_stored_taken(ws, B, H, Hk, n, d)[0] if (
            not atomic and ws.numel() > _lib.bwd_workspace_bytes(B, H, Hk, n, d)) else False

    # dense-vs-sparse gradients (after the dense timing dq, dk, dv hold the dense ones)
    grad_cmp = None
    if sparse_grads is not None:
        grad_cmp = {}
        for nm, sp, de in (("dQ", sparse_grads[0], dq), ("dK", sparse_grads[1], dk), ("dV", sparse_grads[2], dv)):
            a_, r_ = sp.float().flatten(), de.float().flatten()
            grad_cmp[nm] = {"cos": float(torch.dot(a_, r_) / (a_.norm() * r_.norm())),
                            "rel_l2": float((a_ - r_).norm() / r_.norm())}
        del sparse_grads

    pairs_dense = visible_pairs(n, win) if causal else float(n) * n
    f_dense_bwd = 10.0 * d * B * H * pairs_dense
    f_fwd = 4.0 * d * B * H * pairs_dense
    tile_bwd_flop = 10.0 * QT * TILE * d  # per executed (query tile, key tile) pair
    dense_equiv_tflops = f_dense_bwd / (bwd_ms * 1e-3) / 1e12
    mfma_frac = kept * tile_bwd_flop / (bwd_ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)

    # per-step kernel time: with the stored-G_S path each backward pass launches
    # two variants of the G_K/G_V and G_Q kernels, one of which returns at once,
    # so the library's per-name totals are divided by the step count
    kms = {k_: (v_[0] / args.steps if v_[1] else None) for k_, v_ in prof.items()}
    # dominant kernel: dK/dV pass; algorithmic work = 4 of the 5 backward GEMMs
    # (S, G_P, G_V, G_K) per executed tile = 8*128*128*d FLOP
    dkdv_ms = kms.get("dkdv")
    dkdv_flop = kept * 8.0 * QT * TILE * d
    achieved = dkdv_flop / (dkdv_ms * 1e-3) / 1e12 if dkdv_ms else None
    roofline = {"kernel": "dkdv", "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS if achieved else None,
                "traffic": measured_traffic(w.name)}

    # the stored-G_S G_Q pass streams each kept tile's bf16 G_S (32 KB) and its
    # row sums (2 KB) from HBM and writes G_Q once: an HBM-bound pass
    roofline_gq = None
    if gq_stored and kms.get("dq"):
        gq_bytes = kept * _lib.slot_bytes(QT) + B * n * H * d * 2
        gbs = gq_bytes / (kms["dq"] * 1e-3) / 1e9
        roofline_gq = {"kernel": "dqs", "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                       "frac": gbs / PEAK_HBM_GBS}

    # The same sparse backward with 64-row query tiles (the finer mask the
    # per-row statistics allow): mask + backward timed over the same steps, on
    # the forward's outputs of the last step.
    q64 = None
    if QT == TILE and not args.no_q64 and not atomic and dense_ms is not None:
        o, lse, olo = step()
        st64 = torch.zeros(2, dtype=torch.int64, device=dev)
        m64 = bl.mask(tl, lse, n, causal, negl, window=win, q_tile=64)
        ws64 = workspace(m64)
        for _ in range(max(1, args.warmup)):
            m64 = bl.mask(tl, lse, n, causal, negl, window=win, q_tile=64)
            bl.bwd(q, k, v, o, do, lse, m64, causal=causal, window=win, workspace=ws64, out=(dq, dk, dv), o_lo=olo)
        torch.cuda.synchronize()
        ev64 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            ev64[i][0].record()
            m64 = bl.mask(tl, lse, n, causal, negl, window=win, q_tile=64, stats=st64)
            ev64[i][1].record()
            bl.bwd(q, k, v, o, do, lse, m64, causal=causal, window=win, workspace=ws64, out=(dq, dk, dv), o_lo=olo)
            ev64[i][2].record()
        torch.cuda.synchronize()
        m64_ms = sum(e[0].elapsed_time(e[1]) for e in ev64) / args.steps
        b64_ms = sum(e[1].elapsed_time(e[2]) for e in ev64) / args.steps
        s64 = st64.cpu().tolist()
        kept64 = s64[1] / args.steps
        q64 = {"q_tile": 64, "bwd_ms": b64_ms, "mask_ms": m64_ms, "sparsity": 1.0 - s64[1] / s64[0],
               "executed_64x128_tiles_per_step": kept64,
               "dense_equiv_tflops": f_dense_bwd / (b64_ms * 1e-3) / 1e12,
               "bwd_speedup_vs_dense": dense_ms / b64_ms,
               "executed_tile_mfma_frac": kept64 * 10.0 * 64 * TILE * d / (b64_ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
               "gq_path": ("stored" if _lib.bwd_state(ws64, B, H, Hk, n, d)[0] else "partly stored or recompute")
               if ws64.numel() > _lib.bwd_workspace_bytes(B, H, Hk, n, d) else "recompute",
               "bwd_workspace_gb": ws64.numel() / 1e9}
        del ws64, m64

    # mask algorithmic bytes: tile-LSE of every candidate pair (512 B), the row LSE
    # and D-like row data of each query tile, bitmap + list entries written
    Tq = (n + QT - 1) // QT
    mask_bytes = cand * 512 + B * H * n * 4 + B * H * Tq * T * 1 + kept * 2 * 2 + 2 * B * H * (Tq + T) * 4
    delta_bytes = B * H * n * (4 * d + 4 + 2 * d)  # O, G_O, O_lo read; D written

    out = {
        "metric": METRIC,
        "value": dense_equiv_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "H_k": Hk, "n": n, "d": d, "causal": causal,
                   "window": win, "negl_prob": negl, "tile": TILE, "q_tile": QT, "stats": args.stats},
        "bwd_ms": bwd_ms,
        "fwd_ms": fwd_ms,
        "mask_ms": mask_ms,
        "dense_bwd_ms": dense_ms,
        "bwd_speedup_vs_dense": (dense_ms / bwd_ms) if dense_ms else None,
        "dense_vs_sparse_grads": grad_cmp,
        "gq_path": "atomic" if atomic else (
            "stored" if gq_stored else ("partly stored" if gq_state[2] else "recompute")),
        "gq_stored_tiles": gq_state[2],
        "peak_mem_gb": peak_mem / 1e9,
        "dense_gq_path": None if dense_stored is None else ("stored" if dense_stored else "recompute"),
        "bwd_workspace_gb": ws_bytes / 1e9,
        "sparsity": sparsity,
        "executed_tiles_per_step": kept,
        "candidate_tiles_per_step": cand,
        "executed_tile_mfma_frac": mfma_frac,
        "fwd_tflops": f_fwd / (fwd_ms * 1e-3) / 1e12,
        "fwd_mfma_frac": f_fwd / (fwd_ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "kernel_ms_per_step": kms,
        "mask_gbs": (mask_bytes / ((kms["mask_select"] + kms["mask_transpose"]) * 1e-3) / 1e9)
        if kms.get("mask_select") and kms.get("mask_transpose") else None,
        "delta_gbs": delta_bytes / (kms["delta"] * 1e-3) / 1e9 if kms.get("delta") else None,
        "wall_s_timed": wall,
        "roofline": roofline,
        "roofline_gq": roofline_gq,
        "q_tile_64": q64,
        "cpu_baseline": None,
    }
    log(f"[bench] fwd {fwd_ms:.3f} ms  mask {mask_ms:.3f} ms  bwd {bwd_ms:.3f} ms  dense bwd "
        f"{dense_ms if dense_ms is None else round(dense_ms, 3)} ms  sparsity {sparsity:.3f}  "
        f"dense-equiv {dense_equiv_tflops:.1f} TFLOP/s  exec-tile MFMA {100 * mfma_frac:.1f}%")
    if q64:
        log(f"[bench] 64-row query tiles: mask {q64['mask_ms']:.3f} ms  bwd {q64['bwd_ms']:.3f} ms  sparsity "
            f"{q64['sparsity']:.3f}  speedup vs dense {q64['bwd_speedup_vs_dense']:.2f}x")
    if args.cpu_baseline == "on":
        del q, k, v, do, tl, ws, dq, dk, dv
        log(f"[bench] oracle CPU baseline on {min(args.cpu_rows, n)} rows of heads {cpu_heads} ...")
        out["cpu_baseline"] = cpu_baseline(w, x_cpu, cpu_heads, negl, args.cpu_rows, win)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
