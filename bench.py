#!/usr/bin/env python3
"""Throughput of the drafter hot path on one MI355X.

One bench step = one draft_block(4) call over the E4B-shaped batch-16 workload (backbone 2560, hidden 256, 4 Q-only
layers over a shared K=V cache of 8192 keys per sequence, 3 sliding layers with window 512 and one full layer,
2048-centroid top-32 masked head over a 262144 vocabulary, the -1e30 logits row written every step). Inputs are
synthetic (seeded counter-based generator) and resident in HBM before the timed region.

Prints one JSON line: draft tokens/s (value), µs per drafter step, the roofline of the timed launch (algorithmic
bytes / HIP-event duration against 8 TB/s), and the CPU oracle timed on a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def algorithmic_bytes(shape, batch, lens, distinct_clusters, with_logits=True):
    """Bytes one drafter step must move: weights once, each cache's K (= V) once over the keys it reads (the
    sliding window counted once for the three sliding layers), the selected clusters' head rows, their ordering
    ids, the logits row, and target hidden / embedding rows / hidden_out."""
    H, Bb, F, Q, hd = shape.hidden, shape.backbone, shape.ffn, shape.q_dim, shape.head_dim
    per_layer = (Q * H + H * Q + 3 * F * H) * 2 + (hd + 4 * H) * 2
    weights = (2 * Bb * H + Bb * H + shape.n_centroids * H + H) * 2 + shape.n_layer * per_layer
    kv = sum(shape.n_kv_head * hd * 2 * (L + min(shape.swa_window, L)) for L in lens)
    head = distinct_clusters * shape.vsc * H * 2
    ids = 4 * shape.top_k * shape.vsc * batch
    logits = 4 * shape.vocab * batch if with_logits else 0
    io = 2 * Bb * batch * 3
    return weights + kv + head + ids + logits + io, dict(weights=weights, kv=kv, head=head, ids=ids, logits=logits,
                                                         io=io)


def cpu_baseline(wl, seconds):
    """The oracle as it stands, on single-row drafter steps of the same workload, for about `seconds`."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle as O
    from fixtures import synth
    shape = wl.shape
    w = synth.make_weights(shape, seed=wl.seed)
    inp = synth.make_inputs(wl, with_target_embd=False)
    m = O.Model(O.config_from(shape), w)
    ks = [inp["k_sliding"].numpy().view(np.uint16), inp["k_full"].numpy().view(np.uint16)]
    kv = O.SharedKV(k=ks, v=ks, lens=[inp["len_sliding"], inp["len_full"]], rope=inp["rope"].numpy())
    th = inp["target_hidden"].numpy().view(np.uint16)
    tok = inp["last_token"].numpy()
    rows_emb = synth.LazyRows(wl.seed, shape)
    for b in range(wl.batch):
        rows_emb[int(tok[b])]  # generate the embedding rows outside the timed loop
    done = 0
    t0 = time.perf_counter()
    while True:
        O.drafter_step(m, th, tok, rows_emb, kv, rows=[done % wl.batch])
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": done / dt, "unit": "draft tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} single-row drafter steps of the {wl.name} workload (rows 0..{min(done, wl.batch) - 1},"
                      f" first step of the block), fp64 NumPy oracle, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="e4b_b16_ctx8192_block4")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus above 1 is not supported"}))
        sys.exit(2)

    import numpy as np
    import torch

    from fixtures import synth
    from mtp_drafter_step_amd import Drafter, SharedKV

    wl = synth.WORKLOADS[args.workload]
    shape, B, n = wl.shape, wl.batch, wl.n_steps
    dev = "cuda"
    w = synth.make_weights(shape, seed=wl.seed, device=dev)
    inp = synth.make_inputs(wl, device=dev, with_target_embd=True)
    kv = SharedKV(inp["k_sliding"], inp["k_full"], inp["len_sliding"], inp["len_full"], inp["rope"])
    d = Drafter(shape, w, max_batch=B)
    out = {}
    ws = d.workspace(B)
    th, tok, temb = inp["target_hidden"], inp["last_token"], inp["target_embd"]

    def run():
        return d.draft_block(n, th, tok, temb, kv, want_logits=True, out=out, workspace=ws)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()

    # distinct clusters selected per step (for the head-row bytes), from this run's own logits rows
    ordering = w["token_ordering"].cpu().numpy()
    inv = np.empty_like(ordering)
    inv[ordering] = np.arange(ordering.size, dtype=ordering.dtype)
    lg = out["logits"].view(torch.int32).cpu().numpy()
    U = []
    for i in range(n):
        fin = lg[i] != np.int32(np.uint32(0xF149F2CA).view(np.int32))
        clusters = set()
        for b in range(B):
            clusters |= set((inv[np.nonzero(fin[b])[0]] // shape.vsc).tolist())
        U.append(len(clusters))
    u_mean = float(np.mean(U))
    step_bytes, parts = algorithmic_bytes(shape, B, inp["len_full"], u_mean)
    step_bytes_rows, _ = algorithmic_bytes(shape, B, inp["len_full"], B * shape.top_k)

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        run()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = wall * 1e3 / args.steps
    tokens = B * n * args.steps
    value = tokens / wall
    avg_launch_s = float(np.mean(launch_ms)) * 1e-3
    achieved = n * step_bytes / avg_launch_s / 1e9

    res = {
        "metric": "draft tokens/sec and µs per drafter step; achieved HBM GB/s vs roofline",
        "value": value, "unit": "draft tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "context": wl.context, "draft_block": n,
                   "backbone": shape.backbone, "hidden": shape.hidden, "vocab": shape.vocab,
                   "n_centroids": shape.n_centroids, "top_k": shape.top_k, "swa_window": shape.swa_window,
                   "logits_row_written": True},
        "us_per_drafter_step": float(np.mean(launch_ms)) * 1e3 / n,
        "us_per_drafter_step_p10_p90": [float(np.percentile(launch_ms, 10)) * 1e3 / n,
                                        float(np.percentile(launch_ms, 90)) * 1e3 / n],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "draft_block launch (all kernels of 4 drafter steps)",
                     "bytes_per_launch": n * step_bytes, "bytes_per_step_parts": parts,
                     "distinct_clusters_per_step": U, "bytes_per_launch_per_row_clusters": n * step_bytes_rows,
                     "avg_launch_us": avg_launch_s * 1e6},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
