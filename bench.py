#!/usr/bin/env python3
"""Throughput of the drafter hot path on one MI355X.

One bench step = one draft_block(4) call over the E4B-shaped batch-16 workload (backbone 2560, hidden 256, 4 Q-only
layers over a shared K=V cache of 8192 keys per sequence, 3 sliding layers with window 512 and one full layer,
2048-centroid top-32 masked head over a 262144 vocabulary, the -1e30 logits row written every step). Inputs are
synthetic (seeded counter-based generator) and resident in HBM before the timed region.
--workload e26b_b32_ctx32768_block4 times the 26B-A4B-shaped drafter instead (backbone 2816, hidden 1024, 8 query
heads over one kv head, batch 32, context 32768, window 1024) with the dense tied head over the full table.

Prints one JSON line: draft tokens/s (value), µs per drafter step, the roofline of the dominant kernel (its
algorithmic bytes per launch over its HIP-event launch duration, against 8 TB/s; at batch <= 16 that kernel is the
persistent one, whose launch is the whole draft block), warm (back to back) and cold (after a 1 GiB streaming read
that evicts L2 and the memory-side cache), per launch site of the per-stage kernels as well, and the CPU oracle
timed on a bounded sample on this host with all BLAS threads and with one.
--cold-only runs only calls that each follow a sweep (for counter collection; prints no JSON line).

Host-only helper modes (no GPU) turn rocprofv3 output of this script into the text summaries kept in profiles/:
  --summarize-stats DIR   kernel-trace statistics of a bench run
  --summarize-pmc FETCH_DIR WRITE_DIR   FETCH_SIZE / WRITE_SIZE per dispatch of the dominant kernel, scaled by what
                          the same counters read for the calibration copy (--copy-probe) of known size
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak
CSRC = os.path.join(ROOT, "mtp_drafter_step_amd", "csrc")
# the source file of each kernel; a kernel's digest covers that file and the shared headers
KERNEL_FILE = {"k_stream_read": "k_stream.hip", "k_attn_mfma": "k_attention.hip", "k_attn": "k_attention.hip", "k_attn_mq": "k_attention_shared.hip", "k_head": "k_head.hip",
               "k_head_dense": "k_head.hip", "k_final": "k_head.hip", "k_fill": "k_head.hip",
               "k_zero_u64": "k_head.hip", "k_gather_rows": "k_head.hip",
               "k_sample_tiles": "k_head.hip", "k_sample_pick": "k_head.hip", "k_gemm": "k_gemm.hip",
               "k_group": "k_head.hip", "k_head_grouped": "k_head.hip", "k_topk_rows": "k_head.hip",
               "k_rownorm": "k_gemm.hip", "k_merge": "k_gemm.hip", "k_team": "k_team.hip"}
PROFILES = os.path.join(ROOT, "profiles")
COPY_PROBE_BYTES = 512 << 20

# launch-site label (as recorded by the library's timing records) -> kernel symbol stem
SITE_KERNEL = {"pre": "k_pre", "qproj": "k_qproj", "attn_sliding": "k_attn_mfma", "attn_full": "k_attn_mfma",
               "o_proj": "k_oproj",
               "down": "k_dense", "ffn": "k_ffn", "post": "k_post", "head": "k_head", "final": "k_final",
               "scores": "k_dense", "fill": "k_fill", "head_dense": "k_head_dense", "zero_keys": "k_zero_u64",
               "sample_tiles": "k_sample_tiles", "sample_pick": "k_sample_pick",
               # the large-batch path
               "rownorm": "k_rownorm", "post_norm": "k_rownorm", "attn_merge": "k_merge",
               "pre_gemm": "k_gemm", "qproj_gemm": "k_gemm", "o_proj_gemm": "k_gemm", "ffn_gemm": "k_gemm",
               "down_gemm": "k_gemm", "post_gemm": "k_gemm", "scores_gemm": "k_gemm",
               "head_select": "k_topk_rows", "head_group": "k_group", "head_grouped": "k_head_grouped",
               # the persistent kernel: every step of a call in one launch
               "team": "k_team"}


def site_kernel(site, shape, shared=False):
    """Kernel behind a launch site for this shape (the matrix-core attention covers head_dim 256 with up to eight
    query heads per kv head; other shapes run the vector-ALU attention; caches shared by the rows run the
    multi-query attention)."""
    if site.startswith("attn_") and shared and shape.head_dim == 256:
        return "k_attn_mq"
    if site.startswith("attn_") and not (shape.head_dim == 256 and shape.n_head // shape.n_kv_head <= 8):
        return "k_attn"
    return SITE_KERNEL[site]


def source_digest(kernel: str) -> str:
    """sha256[:16] of the sources that define `kernel` (its file plus device.h and kernels.h)."""
    h = hashlib.sha256()
    extra = ("attn_mfma.h",) if kernel in ("k_team", "k_attn_mfma") else ()
    for name in ("device.h", "kernels.h", *extra, KERNEL_FILE.get(kernel, "k_layers.hip")):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def step_bytes(shape, batch, lens, distinct_clusters, with_logits=True, shared=False):
    """Bytes one drafter step must move: weights once, each cache's K (= V) once over the keys it reads (the
    sliding window counted once for the three sliding layers), the selected clusters' head rows and their ordering
    ids (the dense head: the whole table), the logits row, and target hidden / embedding rows / hidden_out."""
    H, Bb, F, Q, hd = shape.hidden, shape.backbone, shape.ffn, shape.q_dim, shape.head_dim
    per_layer = (Q * H + H * Q + 3 * F * H) * 2 + (hd + 4 * H) * 2
    weights = (2 * Bb * H + Bb * H + shape.n_centroids * H + H) * 2 + shape.n_layer * per_layer
    # a shared cache (rows of one sequence) is needed once: its longest row's keys
    kv_lens = [max(lens)] if shared else lens
    kv = sum(shape.n_kv_head * hd * 2 * (L + min(shape.swa_window, L)) for L in kv_lens)
    dense = shape.n_centroids == 0
    head = shape.vocab * H * 2 if dense else distinct_clusters * shape.vsc * H * 2
    ids = 0 if dense else 4 * shape.top_k * shape.vsc * batch
    logits = 4 * shape.vocab * batch if with_logits else 0
    io = 2 * Bb * batch * 3
    return weights + kv + head + ids + logits + io, dict(weights=weights, kv=kv, head=head, ids=ids, logits=logits,
                                                         io=io)


def site_bytes(site, shape, batch, lens, distinct_clusters, shared=False):
    """Algorithmic bytes of one launch of a launch site: the weights and cache rows the step needs from it, its
    activation inputs and outputs (fp32), and its share of the logits row. Intermediates that exist only because
    the path is split into kernels (attention partials) count for the merge only."""
    B, H, Bb, F, QD, hd = batch, shape.hidden, shape.backbone, shape.ffn, shape.q_dim, shape.head_dim
    act = lambda n: 4 * B * n  # noqa: E731  fp32 activation rows
    if site.endswith("_gemm"):  # the large-batch path: the same weights and activations as the fused stages
        base = {"pre_gemm": "pre", "qproj_gemm": "qproj", "o_proj_gemm": "o_proj", "ffn_gemm": "ffn",
                "down_gemm": "down"}.get(site)
        if site == "post_gemm":
            return 2 * Bb * H + act(H) + 2 * B * Bb
        if site == "scores_gemm":
            return 2 * shape.n_centroids * H + act(H) + act(shape.n_centroids)
        if site == "ffn_gemm":
            return 2 * 2 * F * H + act(H) + act(F)
        return site_bytes(base, shape, batch, lens, distinct_clusters, shared)
    if site in ("rownorm", "post_norm"):  # residual stream, partials, norm weights, normed output
        return 4 * act(H) + 4 * H
    if site == "attn_merge":
        return act(QD) * 2
    if site == "fill":  # the -1e30 logits rows
        return 4 * shape.vocab * B
    W = shape.swa_window
    if site == "pre":
        return 2 * H * 2 * Bb + 2 * 2 * B * Bb + act(H)
    if site == "qproj":
        return 2 * QD * H + 2 * H + 3 * act(H) + act(QD)
    if site in ("attn_sliding", "attn_full"):
        keys = sum(L if site == "attn_full" else min(W, L) for L in ([max(lens)] if shared else lens))
        return shape.n_kv_head * hd * 2 * keys + 2 * hd + 2 * act(QD)
    if site == "o_proj":
        return 2 * H * QD + act(QD) + act(H) * (QD // 256)
    if site == "ffn":  # with the masked head, a quarter of the -1e30 logits fill
        fill = 0 if shape.n_centroids == 0 else 4 * shape.vocab * B // shape.n_layer
        return 2 * 2 * F * H + 2 * H + 3 * act(H) + act(F) + fill
    if site == "down":
        return 2 * H * F + act(F) + act(H)
    if site == "post":
        return 2 * (Bb + shape.n_centroids) * H + 2 * H + 2 * act(H) + 2 * B * Bb + act(shape.n_centroids)
    if site == "head":
        n = shape.top_k * shape.vsc
        return distinct_clusters * shape.vsc * H * 2 + 4 * n * B + act(shape.n_centroids) + act(H) + 4 * n * B
    if site == "head_select":  # centroid scores in, selections out
        return act(shape.n_centroids) + 4 * shape.top_k * B
    if site == "head_group":
        return 4 * shape.top_k * B * 2 + 8 * shape.n_centroids
    if site == "head_grouped":  # each selected cluster once (at most the whole table), ids, scatter
        n = shape.top_k * shape.vsc
        return min(distinct_clusters, shape.n_centroids) * shape.vsc * H * 2 + act(H) + 3 * 4 * n * B
    if site == "head_dense":  # the whole table once, h in, the full logits rows out
        return shape.vocab * H * 2 + act(H) + 4 * shape.vocab * B + 8 * B
    if site == "final":
        return 8 * max(shape.top_k, 1) * B + 4 * B
    if site == "zero_keys":
        return 8 * B
    if site == "sample_tiles":  # every scored logit once
        return 4 * (shape.vocab if shape.n_centroids == 0 else shape.top_k * shape.vsc) * B
    if site == "sample_pick":  # one 4096-wide tile per row, its ids, the tile sums, the drawn token and probability
        return 4 * 4096 * B * (1 if shape.n_centroids == 0 else 2) + 4 * 256 * B + 8 * B
    raise KeyError(site)


def site_flops(site, shape, lens, shared):
    """Algorithmic flops of one attention launch over a cache shared by the rows (a dense contraction): for every
    query (row, head), 2 * keys * head_dim for the scores and as many for P.V; None for the other sites."""
    if not (shared and site.startswith("attn_")):
        return None
    keys = sum(L if site == "attn_full" else min(shape.swa_window, L) for L in lens)
    return 4.0 * shape.n_head * keys * shape.head_dim


def host_cpu():
    """(model name, usable cores) of this host, from /proc/cpuinfo and the process's CPU affinity."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return model, cores


def cpu_baseline(wl, seconds, w_dev=None, inp_dev=None):
    """The oracle as it stands, on single-row drafter steps of the same workload, for about `seconds` twice: with the
    BLAS thread pools at their default size, then limited to one thread. The weights and inputs are the
    GPU-generated ones copied to the host when given (the generator is bit-identical on both devices), else
    generated on the host."""
    from threadpoolctl import threadpool_info, threadpool_limits

    import torch

    import oracle as O
    from fixtures import synth

    def host(x):
        if isinstance(x, torch.Tensor):
            return x.cpu()
        if isinstance(x, dict):
            return {k: host(v) for k, v in x.items()}
        if isinstance(x, list):
            return [host(v) for v in x]
        return x

    shape = wl.shape
    w = host(w_dev) if w_dev is not None else synth.make_weights(shape, seed=wl.seed)
    if inp_dev is not None:
        inp = {k: host(v) for k, v in inp_dev.items() if k != "target_embd"}
    else:
        inp = synth.make_inputs(wl, with_target_embd=False)
    m = O.Model(O.config_from(shape), w)
    import numpy as np
    ks = [inp["k_sliding"].numpy().view(np.uint16), inp["k_full"].numpy().view(np.uint16)]
    kv = O.SharedKV(k=ks, v=ks, lens=[inp["len_sliding"], inp["len_full"]], rope=inp["rope"].numpy(),
                    shared=[wl.shared_kv, wl.shared_kv])
    th = inp["target_hidden"].numpy().view(np.uint16)
    tok = inp["last_token"].numpy()
    rows_emb = synth.LazyRows(wl.seed, shape)
    for b in range(wl.batch):
        rows_emb[int(tok[b])]  # generate the embedding rows outside the timed loop

    def timed():
        done = 0
        t0 = time.perf_counter()
        while True:
            O.drafter_step(m, th, tok, rows_emb, kv, rows=[done % wl.batch])
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        return done, time.perf_counter() - t0

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    done, dt = timed()
    with threadpool_limits(limits=1):
        done1, dt1 = timed()
    model, cores = host_cpu()
    return {"value": done / dt, "unit": "draft tokens/s", "cores": int(threads), "kind": "oracle",
            "us_per_drafter_step_per_row": dt / done * 1e6,
            "host": {"cpu_model": model, "nproc": cores},
            "one_thread": {"value": done1 / dt1, "unit": "draft tokens/s", "cores": 1,
                           "us_per_drafter_step_per_row": dt1 / done1 * 1e6,
                           "sample": f"{done1} single-row drafter steps, {dt1:.1f} s"},
            "sample": f"{done} single-row drafter steps of the {wl.name} workload (rows 0..{min(done, wl.batch) - 1},"
                      f" first step of the block), fp64 NumPy oracle with {threads} BLAS threads, {dt:.1f} s; then "
                      f"the same with one thread"}


def traffic_file(kernel, workload):
    return os.path.join(PROFILES, f"{kernel}__{workload}.traffic.md")


def load_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None when absent or taken on another source."""
    p = traffic_file(kernel, workload)
    if not os.path.exists(p):
        return None
    m = re.search(r"<!-- traffic-json: (\{.*\}) -->", open(p).read())
    if not m:
        return None
    t = json.loads(m.group(1))
    if t.get("source_sha256_16") != source_digest(kernel):
        return None
    return t


# ----------------------------------------------------------------------------------------------------------------
# GPU run

def run_bench(args):
    import numpy as np
    import torch

    from fixtures import synth
    from mtp_drafter_step_amd import Drafter, SharedKV

    wl = synth.WORKLOADS[args.workload]
    shape, B, n = wl.shape, wl.batch, wl.n_steps
    dev = "cuda"
    w = synth.make_weights(shape, seed=wl.seed, device=dev)
    inp = synth.make_inputs(wl, device=dev, with_target_embd=True)
    kv = SharedKV(inp["k_sliding"], inp["k_full"], inp["len_sliding"], inp["len_full"], inp["rope"],
                  shared=wl.shared_kv)
    from mtp_drafter_step_amd import abi as _abi
    d = Drafter(shape, w, max_batch=B, options={_abi.MTPD_OPT_PERSISTENT: args.persistent})
    out = {}
    ws = d.workspace(B)
    th, tok, temb = inp["target_hidden"], inp["last_token"], inp["target_embd"]

    uni = None
    if args.temperature:
        g = torch.Generator(device=dev).manual_seed(wl.seed + 17)
        uni = torch.rand(n, B, generator=g, device=dev, dtype=torch.float32)

    def run():
        if args.temperature:
            return d.draft_block_sampled(n, th, tok, temb, kv, args.temperature, uni, want_logits=True, out=out,
                                         workspace=ws)
        return d.draft_block(n, th, tok, temb, kv, want_logits=True, out=out, workspace=ws)

    def copy_probe():
        # calibration copy of known size for the HBM byte counters (a plain device-to-device copy)
        src = torch.empty(COPY_PROBE_BYTES // 4, dtype=torch.int32, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.cold_only:  # profiling mode: every call after a sweep that evicts L2 and the memory-side cache
        from mtp_drafter_step_amd import stream_read
        sweep = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        sink = torch.zeros(4, dtype=torch.int32, device=dev)
        for i in range(args.cold_steps):
            stream_read(sweep, sink)
            run()
            torch.cuda.synchronize()
            print(f"cold call {i + 1} of {args.cold_steps} done", flush=True)
        del sweep
        if args.copy_probe:
            copy_probe()
        return

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()

    # distinct clusters selected per step (for the head-row bytes), from this run's own logits rows
    U = []
    if shape.n_centroids > 0:
        ordering = w["token_ordering"].cpu().numpy()
        inv = np.empty_like(ordering)
        inv[ordering] = np.arange(ordering.size, dtype=ordering.dtype)
        lg = out["logits"].view(torch.int32).cpu().numpy()
        for i in range(n):
            fin = lg[i] != np.int32(np.uint32(0xF149F2CA).view(np.int32))
            clusters = set()
            for b in range(B):
                clusters |= set((inv[np.nonzero(fin[b])[0]] // shape.vsc).tolist())
            U.append(len(clusters))
    u_mean = float(np.mean(U)) if U else 0.0
    lens = [int(x) for x in inp["len_full"]]
    sbytes, parts = step_bytes(shape, B, lens, u_mean, shared=wl.shared_kv)

    # timed region: the K draft_block calls back to back on torch's current stream, nothing else in between
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = B * n * args.steps / wall
    # then the same number of calls, each between two events, for the per-call distribution (outside the timed
    # region: event records between the calls add a few microseconds per call)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in ev:  # create the events before the loop
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev[i][0].record(stream)
        run()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    launch_ms = np.array([a.elapsed_time(b) for a, b in ev])
    us_drafter_step = float(np.median(launch_ms)) * 1e3 / n

    # the library's streaming read (one pass over 1 GiB) gives the measured read rate of this device and, run
    # before a call, evicts L2 and the 256 MB memory-side cache with clean lines
    from mtp_drafter_step_amd import stream_read
    sweep = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    read_ms = []
    for _ in range(8):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        stream_read(sweep, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        read_ms.append(e0.elapsed_time(e1))
    read_gbs = sweep.numel() * 4 / (min(read_ms) * 1e-3) / 1e9

    def flush():
        stream_read(sweep, sink)

    def timed_records(drafter, call, calls, cold):
        """Per-launch (site, ms) records of `calls` calls in timing mode; with cold, a sweep before each call (the
        sweep is not a recorded launch)."""
        drafter.timing(True)
        for _ in range(calls):
            if cold:
                flush()
            call()
        torch.cuda.synchronize()
        drafter.timing(False)
        return drafter.timing_records()

    def tally(recs, calls, drafter_shape):
        per_site = {}
        for name, ms in recs:
            per_site.setdefault(name, []).append(ms)
        per_kernel = {}
        for site, v in per_site.items():
            k = site_kernel(site, drafter_shape, wl.shared_kv)
            e = per_kernel.setdefault(k, {"launches": 0, "total_ms": 0.0, "bytes": 0.0, "sites": []})
            e["launches"] += len(v)
            e["total_ms"] += float(np.sum(v))
            e["bytes"] += len(v) * site_launch_bytes(site)
            fl = site_flops(site, shape, lens, wl.shared_kv)
            if fl is not None:
                e["flops"] = e.get("flops", 0.0) + len(v) * fl
            e["sites"].append(site)
        return per_site, per_kernel

    def site_launch_bytes(site):
        return sbytes * n if site == "team" else site_bytes(site, shape, B, lens, u_mean, shared=wl.shared_kv)

    # per-kernel durations: the same calls with every launch bracketed by HIP events that the runtime records at
    # the kernel's start and end (on the library's launch stream, which is torch's current stream), warm (back to
    # back) and cold (a sweep before each call)
    calls = args.timing_steps
    per_site, per_kernel = tally(timed_records(d, run, calls, False), calls, shape)
    cold_site, cold_kernel = tally(timed_records(d, run, args.cold_steps, True), args.cold_steps, shape)
    dom = max(per_kernel, key=lambda k: per_kernel[k]["total_ms"])
    dk = per_kernel[dom]
    avg_launch_s = dk["total_ms"] / dk["launches"] * 1e-3
    bytes_per_launch = dk["bytes"] / dk["launches"]
    achieved = bytes_per_launch / avg_launch_s / 1e9
    tr = load_traffic(dom, wl.name)
    traffic = None if tr is None else tr["hbm_bytes_per_launch"]
    ck = cold_kernel.get(dom)
    cold_launch_s = ck["total_ms"] / ck["launches"] * 1e-3 if ck else None
    if "flops" in dk:  # a dense contraction (attention over a cache shared by the rows): priced on the matrix cores
        tfl = dk["flops"] / dk["launches"] / avg_launch_s / 1e12
        roof = {"bound": "mfma", "achieved": tfl, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": tfl / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic,
                "algorithmic_flops_per_launch": dk["flops"] / dk["launches"], "algorithmic_GBs": achieved}
        if cold_launch_s:
            ctf = dk["flops"] / dk["launches"] / cold_launch_s / 1e12
            roof["cold"] = {"avg_launch_us": cold_launch_s * 1e6, "achieved": ctf,
                            "frac": ctf / MFMA_BF16_PEAK_TFLOPS}
    else:
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic}
        if cold_launch_s:
            cga = bytes_per_launch / cold_launch_s / 1e9
            roof["cold"] = {"avg_launch_us": cold_launch_s * 1e6, "achieved": cga, "frac": cga / HBM_PEAK_GBS,
                            "frac_of_measured_read_peak": cga / read_gbs}
        roof["frac_of_measured_read_peak"] = achieved / read_gbs
    roof.update({"kernel": dom, "launch_sites": sorted(set(dk["sites"])),
                 "scope": ("the whole drafter step: one launch runs every step of a draft block" if dom == "k_team"
                           else "the dominant kernel (step_roofline has the whole step)"),
                 "launches_per_drafter_step": dk["launches"] / (calls * n),
                 "avg_launch_us": avg_launch_s * 1e6, "algorithmic_bytes_per_launch": bytes_per_launch,
                 "traffic_source": None if tr is None else os.path.relpath(traffic_file(dom, wl.name), ROOT)})

    def kernels_of(pk, ncalls):
        return {k: {"launches_per_drafter_step": v["launches"] / (ncalls * n),
                    "avg_launch_us": v["total_ms"] / v["launches"] * 1e3,
                    "us_per_drafter_step": v["total_ms"] * 1e3 / (ncalls * n),
                    "algorithmic_GBs": v["bytes"] / (v["total_ms"] * 1e-3) / 1e9,
                    "algorithmic_TFLOPs": (v["flops"] / (v["total_ms"] * 1e-3) / 1e12) if "flops" in v else None,
                    "sites": sorted(set(v["sites"]))}
                for k, v in sorted(pk.items(), key=lambda kv_: -kv_[1]["total_ms"])}

    def sites_of(warm, cold, ncalls):
        out_ = {}
        for site, v in sorted(warm.items(), key=lambda kv_: -sum(kv_[1])):
            b = site_launch_bytes(site)
            wu = float(np.mean(v)) * 1e3
            e = {"launches_per_drafter_step": len(v) / (ncalls * n), "avg_launch_us": wu,
                 "algorithmic_bytes_per_launch": b, "GBs": b / (wu * 1e-6) / 1e9,
                 "frac": b / (wu * 1e-6) / 1e9 / HBM_PEAK_GBS}
            if site in cold:
                cu = float(np.mean(cold[site])) * 1e3
                e.update({"cold_avg_launch_us": cu, "cold_GBs": b / (cu * 1e-6) / 1e9,
                          "cold_frac": b / (cu * 1e-6) / 1e9 / HBM_PEAK_GBS})
            out_[site] = e
        return out_

    kernels_table = kernels_of(per_kernel, calls)
    sites_table = sites_of(per_site, cold_site, calls)

    # the per-stage kernels on the same inputs (the path taken when the persistent kernel does not apply): warm and
    # cold per launch site, e.g. the full and the sliding attention separately
    per_stage = None
    if dom == "k_team" and not args.no_per_stage:
        d2 = Drafter(shape, w, max_batch=B, options={_abi.MTPD_OPT_PERSISTENT: 0})
        out2 = {}
        ws2 = d2.workspace(B)

        def run2():
            return d2.draft_block(n, th, tok, temb, kv, want_logits=True, out=out2, workspace=ws2)

        for _ in range(3):
            run2()
        torch.cuda.synchronize()
        ps_warm, _ = tally(timed_records(d2, run2, calls, False), calls, shape)
        ps_cold, _ = tally(timed_records(d2, run2, args.cold_steps, True), args.cold_steps, shape)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(calls):
            run2()
        e1.record(stream)
        torch.cuda.synchronize()
        per_stage = {"us_per_drafter_step": e0.elapsed_time(e1) * 1e3 / (calls * n),
                     "sites": sites_of(ps_warm, ps_cold, calls)}
        d2.close()
        del d2, ws2, out2

    # cold regime for the whole call: a sweep before each timed call (the first drafter step of the block starts
    # cold; the next ones run on what it brought in), and single drafter steps after a sweep each
    cold_ms, cold_step_ms = [], []
    for _ in range(args.cold_steps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        cold_ms.append(e0.elapsed_time(e1))
    out1 = {}
    for _ in range(args.cold_steps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        d.drafter_step(th, tok, temb, kv, want_logits=True, out=out1, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        cold_step_ms.append(e0.elapsed_time(e1))
    del sweep
    us_cold = float(np.median(cold_ms)) * 1e3 / n if cold_ms else None
    us_cold_step = float(np.median(cold_step_ms)) * 1e3 if cold_step_ms else None

    if args.copy_probe:
        copy_probe()

    res = {
        "metric": "draft tokens/sec and µs per drafter step; achieved HBM GB/s vs roofline",
        "value": value, "unit": "draft tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "context": wl.context, "draft_block": n,
                   "backbone": shape.backbone, "hidden": shape.hidden, "vocab": shape.vocab,
                   "n_centroids": shape.n_centroids, "top_k": shape.top_k, "swa_window": shape.swa_window,
                   "head": "dense" if shape.n_centroids == 0 else "masked",
                   "logits_row_written": True, "graph_replay": True,
                   "token_choice": f"sampled, temperature {args.temperature}" if args.temperature else "argmax"},
        "us_per_drafter_step": us_drafter_step,
        "us_per_drafter_step_p10_p90": [float(np.percentile(launch_ms, 10)) * 1e3 / n,
                                        float(np.percentile(launch_ms, 90)) * 1e3 / n],
        "roofline": roof,
        "step_roofline": {"algorithmic_bytes_per_drafter_step": sbytes, "parts": parts,
                          "distinct_clusters_per_step": U,
                          "achieved_GBs": sbytes / (us_drafter_step * 1e-6) / 1e9,
                          "frac": sbytes / (us_drafter_step * 1e-6) / 1e9 / HBM_PEAK_GBS,
                          "frac_of_measured_read_peak": sbytes / (us_drafter_step * 1e-6) / 1e9 / read_gbs,
                          "cold_block_us_per_drafter_step": us_cold,
                          "cold_block_frac": sbytes / (us_cold * 1e-6) / 1e9 / HBM_PEAK_GBS if us_cold else None,
                          "cold_single_step_us": us_cold_step,
                          "cold_single_step_frac": (sbytes / (us_cold_step * 1e-6) / 1e9 / HBM_PEAK_GBS
                                                    if us_cold_step else None),
                          "us_per_drafter_step_for_60pct": sbytes / (0.6 * HBM_PEAK_GBS * 1e9) * 1e6},
        "measured_read_peak": {"GBs": read_gbs, "how": "best of 8 passes of the library's streaming read "
                                                       "(mtpd_stream_read) over a resident 1 GiB buffer, timed "
                                                       "with HIP events"},
        "kernels": kernels_table,
        "sites": sites_table,
        "per_stage_kernels": per_stage,
        "kernel_source_sha256_16": source_digest(dom),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, w, inp)
    print(json.dumps(res), flush=True)


# ----------------------------------------------------------------------------------------------------------------
# host-only summaries of rocprofv3 output

def _find(dirname, suffix):
    hits = sorted(glob.glob(os.path.join(dirname, "**", f"*{suffix}"), recursive=True))
    if not hits:
        sys.exit(f"no *{suffix} under {dirname}")
    return hits[0]


def _stem(name):
    n = name[5:] if name.startswith("void ") else name
    n = n.replace("(anonymous namespace)::", "").replace("mtpd::", "")
    return n.split("(")[0]


def summarize_stats(args):
    path = _find(args.summarize_stats, "kernel_stats.csv")
    rows = list(csv.DictReader(open(path)))
    mine = [r for r in rows if "mtpd::" in r["Name"]]
    lines = [f"# Kernel-trace statistics: drafter kernels, {args.workload}", "",
             f"Command: `{args.cmd}`", "",
             "Kernel source sha256[:16]: " + ", ".join(
                 f"{f} `{source_digest(k)}`" for f, k in (("k_layers.hip", "k_ffn"), ("k_attention.hip", "k_attn_mfma"),
                                                          ("k_attention_shared.hip", "k_attn_mq"),
                                                          ("k_head.hip", "k_head"), ("k_gemm.hip", "k_gemm"),
                                                          ("k_team.hip", "k_team"),
                                                          ("k_stream.hip", "k_stream_read"))), "",
             "Only the library's kernels are listed (the run also holds the input generator's and torch's own "
             "kernels, which are outside the timed calls).", "",
             "| kernel | calls | avg µs | min µs | max µs | total µs | share of library time |", "|---|---|---|---|---|---|---|"]
    tot = sum(float(r["TotalDurationNs"]) for r in mine)
    for r in sorted(mine, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{_stem(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['TotalDurationNs']) / 1e3:.1f} | {100 * float(r['TotalDurationNs']) / tot:.1f}% |")
    # the persistent kernel runs whole draft blocks and single drafter steps: its dispatches split by duration
    trace = glob.glob(os.path.join(args.summarize_stats, "**", "*kernel_trace.csv"), recursive=True)
    if trace:
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in csv.DictReader(open(trace[0]))
                if _stem(r["Kernel_Name"]).startswith("k_team")]
        if durs:
            cut = 0.6 * max(durs)
            lines += ["", "Persistent kernel dispatches by kind (from the kernel trace; a draft_block(4) launch runs four "
                          "steps, so the two kinds separate by duration):", "",
                      "| kind | calls | avg µs | min µs | max µs |", "|---|---|---|---|---|"]
            for kind, v in (("draft_block(4)", [x for x in durs if x >= cut]),
                            ("drafter_step", [x for x in durs if x < cut])):
                if v:
                    lines.append(f"| {kind} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"drafter_kernels__{args.workload}.stats.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print(out)


def summarize_pmc(args):
    fetch_dir, write_dir = args.summarize_pmc

    def per_dispatch(dirname, counter):
        path = _find(dirname, "counter_collection.csv")
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    out = {}
    for counter, dirname in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = per_dispatch(dirname, counter)
        ker = [v for k, v in vals.items() if _stem(k).startswith(args.kernel)]
        if not ker:
            sys.exit(f"no dispatch of {args.kernel} with {counter} in {dirname}")
        kv = [x for v in ker for x in v]
        copies = sorted(x for k, v in vals.items() if "copyBuffer" in k or "copy" in _stem(k).lower() for x in v)
        big = copies[-3:]
        if not big:
            sys.exit(f"no copy dispatch with {counter} in {dirname}")
        copy_kib = sorted(big)[len(big) // 2]
        factor = (COPY_PROBE_BYTES / 1024.0) / copy_kib  # known bytes over counted KiB of the copy
        out[counter] = {"kernel_kib_per_dispatch": sum(kv) / len(kv), "dispatches": len(kv),
                        "copy_kib": copy_kib, "copy_known_kib": COPY_PROBE_BYTES / 1024.0, "factor": factor,
                        "bytes_per_launch": sum(kv) / len(kv) * 1024.0 * factor}
        if counter == "FETCH_SIZE" and max(kv) > 4 * max(min(kv), 1e-9):
            # launches of very different size (the full layer's attention against the sliding layers'): the two
            # groups separately, split at a quarter of the largest
            big_ = [x for x in kv if x >= max(kv) / 4]
            small_ = [x for x in kv if x < max(kv) / 4]
            out[counter]["groups"] = {"large": {"dispatches": len(big_),
                                                "bytes_per_launch": sum(big_) / len(big_) * 1024.0 * factor},
                                      "small": {"dispatches": len(small_),
                                                "bytes_per_launch": sum(small_) / len(small_) * 1024.0 * factor}}
    total = out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]
    t = {"kernel": args.kernel, "workload": args.workload, "hbm_bytes_per_launch": total,
         "fetch_bytes_per_launch": out["FETCH_SIZE"]["bytes_per_launch"],
         "write_bytes_per_launch": out["WRITE_SIZE"]["bytes_per_launch"], "source_sha256_16": source_digest(args.kernel)}
    lines = [f"# HBM traffic per launch: {args.kernel}, {args.workload}", "",
             f"Commands: `{args.cmd}`", "",
             f"Kernel source sha256[:16] ({KERNEL_FILE.get(args.kernel, 'k_layers.hip')} with the shared headers): "
             f"`{source_digest(args.kernel)}`", "",
             "Each counter is read per dispatch in KiB, averaged over the kernel's dispatches, and scaled by the "
             f"ratio of known bytes to counted KiB for the calibration copy ({COPY_PROBE_BYTES >> 20} MiB "
             "device-to-device copy run by the same command).", "",
             "| counter | kernel KiB / dispatch | dispatches | copy KiB counted | copy KiB known | factor | bytes / launch |",
             "|---|---|---|---|---|---|---|"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        o = out[c]
        lines.append(f"| {c} | {o['kernel_kib_per_dispatch']:.1f} | {o['dispatches']} | {o['copy_kib']:.1f} | "
                     f"{o['copy_known_kib']:.1f} | {o['factor']:.4f} | {o['bytes_per_launch']:.0f} |")
    g = out["FETCH_SIZE"].get("groups")
    if g:
        t["fetch_groups"] = g
        lines += ["", "FETCH_SIZE by launch size (split at a quarter of the largest dispatch):", "",
                  "| group | dispatches | fetch bytes / launch |", "|---|---|---|"]
        for k in ("large", "small"):
            lines.append(f"| {k} | {g[k]['dispatches']} | {g[k]['bytes_per_launch']:.0f} |")
    lines += ["", f"HBM bytes per launch (fetch + write): {total:.0f}", "", f"<!-- traffic-json: {json.dumps(t)} -->"]
    os.makedirs(PROFILES, exist_ok=True)
    p = traffic_file(args.kernel, args.workload)
    open(p, "w").write("\n".join(lines) + "\n")
    print(p)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--timing-steps", type=int, default=10, help="calls timed per kernel after the timed region")
    ap.add_argument("--cold-steps", type=int, default=10, help="calls timed after a cache-evicting sweep each")
    ap.add_argument("--workload", default="e4b_b16_ctx8192_block4")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="time draft_block_sampled at this temperature instead of the argmax draft_block")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle seconds per thread setting")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-stage", action="store_true", help="skip timing the per-stage kernels beside the "
                                                                 "persistent kernel")
    ap.add_argument("--persistent", type=int, choices=(0, 1), default=1,
                    help="0: time the per-stage kernels only (the persistent kernel switched off)")
    ap.add_argument("--cold-only", action="store_true",
                    help="profiling mode: only calls after a cache-evicting sweep each (no JSON line)")
    ap.add_argument("--copy-probe", action="store_true", help="run the counter calibration copy after timing")
    ap.add_argument("--summarize-stats", metavar="DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--kernel", default="k_attn_mfma")
    ap.add_argument("--cmd", default="", help="the command that produced the rocprofv3 output (recorded)")
    args = ap.parse_args()
    if args.summarize_stats:
        return summarize_stats(args)
    if args.summarize_pmc:
        return summarize_pmc(args)
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus above 1 is not supported"}))
        sys.exit(2)
    run_bench(args)


if __name__ == "__main__":
    main()
