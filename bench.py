#!/usr/bin/env python3
"""Benchmark of the sparse FP8 MLA decode hot path on one MI355X.

One step = one pass of the whole path over one batch, two launches:
  1. the partial kernel, which resolves the req-local top-k indices through
     the block table and also writes their req-local -> global conversion
     (fill -1) from the same index and table loads;
  2. the split combine kernel (when the selector picks S > 1).
That is dsv4_sparse_decode_with_slots.  The sequential form of the same work
(a conversion launch, then the partial kernel over the global slots, then the
combine: three launches) is timed beside it.
The workload is the long-context low-batch decode: B=1 query token, H=64
heads, top-k 2048 of 131072 cache slots (block size 64, shuffled pages, 1 %
invalid), fp8_ds_mla rows, sink logits, softmax scale 512^-0.5.

Cache residency: the timed steps rotate over R replicas of the cache (the
same bytes at R different addresses, each with its own block table), with R
chosen so that the rows touched between two uses of one replica exceed twice
the 256 MB Infinity Cache.  Every step therefore reads its rows from HBM, as
a decode layer does in a model whose other layers and weights stream through
the caches in between.  A single-replica (cache-warm) figure is reported
beside it for context.

The steps are captured once into a HIP graph (through torch.cuda.graph) and
replayed: a decode step is launch-bound, and serving engines replay decode
steps from graphs.  Per-kernel average durations come from HIP events around
graphs of K back-to-back launches of each kernel alone, on the stream the
kernels run on.

Prints ONE JSON line.  Options: --steps K --warmup W --gpus 1 (more GPUs are
not supported: the path runs on one GPU) --replicas R --no-cpu-baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("attended KV tokens/sec + achieved HBM GB/s, sparse FP8 MLA decode B=1 "
          "topk=2048 H=64")
WORKLOAD_CONFIG = 2
HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0         # MI355X dense bf16 MFMA
INFINITY_CACHE_BYTES = 256 << 20
ROW_BYTES = 584                   # 576 data + 8 scale bytes per valid entry
INDEX_BYTES = 4


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough to defeat the caches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-workload", type=int, default=None, metavar="CI",
                    help="instead of the benchmark: run the selector's decode of workload CI "
                         "(0-4) --steps times, for counter passes, and print its algorithmic "
                         "work as JSON")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the batch and split-count sweeps (profiler runs: their launches "
                         "share the headline kernel's name)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the per-workload decode table (all five seeded workloads)")
    ap.add_argument("--no-context-parallel", action="store_true",
                    help="skip the one-GPU share of a context-parallel decode")
    ap.add_argument("--no-two-kernel", action="store_true",
                    help="skip the fused vs two-kernel comparison on the large-batch workload")
    ap.add_argument("--scrub", action="store_true",
                    help="decode with the scrub flag (non-finite cache elements read as 0)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed steps one by one instead of replaying a graph "
                         "(for hardware-counter runs, which count per dispatch)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="before the steps, copy this many MB device-to-device once: a kernel "
                         "of known traffic that calibrates the HBM byte counters")
    return ap.parse_args()


def _source_digest() -> str:
    """Digest of the decode kernels' sources with comments and whitespace
    removed, so that an edit to a comment does not orphan the counters taken
    on the same code."""
    h = hashlib.sha256()
    for name in ("decode.hip", "decode_short.hip", "decode_common.hpp",
                 "device_util.hpp", "fastdiv.hpp", "internal.hpp"):
        with open(os.path.join(ROOT, "sparse_mla_attention_block_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _one_super_tile(plan, kt: int) -> bool:
    """The short-split kernel's variant for splits of at most one 64-row
    super-tile (chunks are whole 32-entry tiles)."""
    chunk = -(-kt // plan.num_splits)
    return -(-chunk // 32) * 32 <= 64


def _partial_kernel_name(plan, kt: int, scrub: bool) -> str:
    """The partial kernel one slot-writing decode launches, as rocprofv3 names it."""
    import sparse_mla_attention_block_amd as dsv4
    sc = "true" if scrub else "false"
    if plan.partial_kernel == dsv4.DSV4_KERNEL_SHORT:
        one = "true" if _one_super_tile(plan, kt) else "false"
        return f"decode_short_kernel<{plan.heads_per_group}, {sc}, true, false, true, {one}>"
    emit = "true" if not plan.balanced_splits and -(-kt // plan.num_splits) <= 1024 else "false"
    return f"decode_partial_kernel<{plan.heads_per_group}, {sc}, {emit}>"


def _traffic_from_profile(digest: str, kernel: str):
    """HBM bytes per launch of the partial kernel from the committed counter
    summary, if it was taken on the current kernel source and kernel variant."""
    path = os.path.join(ROOT, "profiles", "decode_partial_long_lowbatch_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_digest") != digest or rec.get("kernel") != kernel:
        return None
    return rec.get("hbm_bytes_per_launch")


def main() -> int:
    args = _parse()
    if args.profile_workload is not None:
        return profile_workload(args.profile_workload, args.steps)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the decode path "
              "is single-GPU, and this benchmark times one GPU.", file=sys.stderr)
        return 2
    import torch
    import sparse_mla_attention_block_amd as dsv4
    from synth import make_workload

    K, W = args.steps, args.warmup
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = make_workload(WORKLOAD_CONFIG)
    B, H, Kt = w.B, w.H, w.Kt
    nb, stride = w.num_blocks, w.page_stride
    n_valid_slots = int((w.topk_idx >= 0).sum())   # req-local entries that resolve (all do here)

    # Replicas: the same cache bytes at R addresses.
    touched = n_valid_slots * (ROW_BYTES + 64)      # data sectors + one scale sector per row
    R = args.replicas or max(1, math.ceil(2 * INFINITY_CACHE_BYTES / touched))
    base = torch.from_numpy(w.kv).to(dev)
    pool = torch.empty((R, nb, stride), dtype=torch.uint8, device=dev)
    pool.copy_(base.unsqueeze(0).expand(R, nb, stride))
    del base
    bt0 = torch.from_numpy(w.block_table.astype(np.int64)).to(dev)
    offs = (torch.arange(R, device=dev, dtype=torch.int64) * nb).view(R, 1, 1)
    bt_all = torch.where(bt0.unsqueeze(0) >= 0, bt0.unsqueeze(0) + offs, -1).to(torch.int32)
    bt_all = bt_all.reshape(R * B, -1).contiguous()
    maxb = bt_all.shape[1]
    idx = torch.from_numpy(w.topk_idx).to(dev)
    q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
    sink = torch.from_numpy(w.sink).to(dev)
    gslots = torch.empty((B, Kt), dtype=torch.int32, device=dev)
    gslots_all = torch.empty((R, B, Kt), dtype=torch.int32, device=dev)
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)

    flags = dsv4.DSV4_DECODE_SCRUB if args.scrub else 0
    desc = dsv4.make_desc(batch=B, num_heads=H, topk=w.topk, swa=w.swa, block_size=w.block_size,
                          num_blocks=R * nb, page_stride=stride, sm_scale=w.sm_scale, flags=flags)
    plan = dsv4.dsv4_sparse_decode_plan(desc, 0)
    S = plan.num_splits
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
    desc = dsv4.make_desc(batch=B, num_heads=H, topk=w.topk, swa=w.swa, block_size=w.block_size,
                          num_blocks=R * nb, page_stride=stride, sm_scale=w.sm_scale, workspace=ws,
                          flags=flags)
    part_o, part_l = dsv4.workspace_split_views(ws, B, H, S) if S > 1 else (None, None)
    kv = pool.view(-1)
    # The block-table form of the same decode (req-local indices).
    desc_tbl = dsv4.make_desc(batch=B, num_heads=H, topk=w.topk, swa=w.swa,
                              block_size=w.block_size, num_blocks=R * nb, page_stride=stride,
                              sm_scale=w.sm_scale, max_blocks_per_seq=maxb,
                              block_table_stride=maxb, workspace=ws, flags=flags)
    plan_tbl = dsv4.dsv4_sparse_decode_plan(desc_tbl, S)

    def convert(r, dst):
        dsv4.dsv4_convert_req_index_to_global(None, B, bt_all[r * B:(r + 1) * B], maxb, maxb, idx,
                                              Kt, B, Kt, w.block_size, None, -1, dst)

    def partial(slots):
        dsv4.dsv4_sparse_decode_partial(desc, q, kv, None, slots, None, sink, out, lse, S)

    def partial_tbl(r):
        dsv4.dsv4_sparse_decode_partial_with_slots(desc_tbl, q, kv, bt_all[r * B:(r + 1) * B],
                                                   idx, None, sink, out, lse, S, gslots)

    def combine():
        if S > 1:
            dsv4.dsv4_combine_splits(B, H, S, part_o, part_l, sink, out, lse)

    def step(r):
        dsv4.dsv4_sparse_decode_with_slots(desc_tbl, q, kv, bt_all[r * B:(r + 1) * B], idx, None,
                                           sink, out, lse, S, gslots)

    def step_seq(r):
        convert(r, gslots)
        partial(gslots)
        combine()

    for r in range(R):
        convert(r, gslots_all[r])
    torch.cuda.synchronize()

    def capture(fn, n, offset=0):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(offset % R)            # warm the stream outside the graph
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(n):
                fn((offset + i) % R)
        return g

    if args.calib_copy_mb:
        src = torch.empty(args.calib_copy_mb << 20, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.eager:
        for i in range(W):
            step(i % R)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record()
        for i in range(K):
            step((W + i) % R)
        ev1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    else:
        g_warm = capture(step, W) if W > 0 else None
        g_main = capture(step, K, offset=W)
        # Warmup, then the timed region: exactly K steps.
        if g_warm is not None:
            g_warm.replay()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record()
        g_main.replay()
        ev1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3
    ms_per_step = wall_ms / K
    ev_ms_per_step = ev0.elapsed_time(ev1) / K

    # Correctness of the timed launches: every replica holds the same rows, so
    # the last step's output must equal a fresh single call (same bytes).
    out_timed = out.clone()
    lse_timed = lse.clone()

    # Per-kernel average durations: K back-to-back launches of one kernel.
    def time_graph(g, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g.replay()                    # untimed pass
        torch.cuda.synchronize()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    # The conversion's output of the timed steps, checked against a fresh
    # conversion of the same replica's table.
    conv_timed = gslots.clone()
    last_r = (W + K - 1) % R
    conv_ok = bool(torch.equal(conv_timed, gslots_all[last_r]))

    kt_conv = time_graph(capture(lambda r: convert(r, gslots), K), K)
    kt_part = time_graph(capture(partial_tbl, K), K)
    kt_part_slots = time_graph(capture(lambda r: partial(gslots_all[r]), K), K)
    kt_comb = time_graph(capture(lambda r: combine(), K), K) if S > 1 else 0.0
    seq_ms_per_step = time_graph(capture(step_seq, K), K)

    # Floors: the partial kernel's own gather (same grid, same row loads over
    # the same rotating replicas, no arithmetic), and an empty launch (a
    # 4-byte fill kernel) for the launch cost of a graph node.
    words = torch.empty(plan.grid_partial * plan.block_partial, dtype=torch.int32, device=dev)
    kt_gather = time_graph(capture(lambda r: dsv4.dsv4_gather_floor(
        desc_tbl, kv, bt_all[r * B:(r + 1) * B], idx, None, S, words), K), K)
    tiny = torch.empty(1, dtype=torch.int32, device=dev)
    kt_empty = time_graph(capture(lambda r: tiny.fill_(r), K), K)

    # Cache writer (not part of the decode step): quantise-and-store of a
    # 65536-row bulk, rotating over replicas of rows and pages so that each
    # launch reads and writes HBM.
    wn, wbs = 65536, 64
    wpages = wn // wbs
    wrep = max(2, math.ceil(2 * INFINITY_CACHE_BYTES / (wn * (1024 + 584))))
    wrows = torch.randn((wrep * wn, 512), device=dev).to(torch.bfloat16)
    wpool = torch.empty((wrep * wpages, wbs * ROW_BYTES), dtype=torch.uint8, device=dev)
    # A prefill-like chunk: consecutive rows fill whole pages in order, the
    # pages themselves drawn in shuffled order from the pool.
    pos = torch.arange(wn, device=dev)
    wslots = torch.stack([torch.randperm(wpages, device=dev)[pos // wbs] * wbs + pos % wbs
                          + r * wn for r in range(wrep)]).to(torch.int64)

    def writer(r):
        dsv4.dsv4_quantize_store(wrows[r * wn:(r + 1) * wn], 512, wslots[r], wn, wpool, wbs,
                                 wrep * wpages, wbs * ROW_BYTES, dsv4.DSV4_STORE_SANITIZE)

    kt_writer = time_graph(capture(lambda r: writer(r % wrep), K), K)
    writer_bytes = wn * (512 * 2 + 8 + ROW_BYTES)
    del wrows, wpool, wslots

    # Cache-warm reference: one replica, same step.
    g_hot = capture(lambda r: step(0), K)
    hot_ms_per_step = time_graph(g_hot, K)
    kt_part_hot = time_graph(capture(lambda r: partial_tbl(0), K), K)

    partial_tbl(0)
    combine()
    torch.cuda.synchronize()
    same = bool(torch.equal(out_timed, out) and torch.equal(lse_timed, lse))
    step_seq(0)
    torch.cuda.synchronize()
    same_seq = bool(torch.equal(out_timed, out) and torch.equal(lse_timed, lse))

    # B-sweep of the headline shape: B tokens per step with the same index
    # list, token b of a step reading its own cache replica (same rows,
    # different addresses), the replicas rotated across steps.
    sweep = []
    K2 = min(K, 400)
    for Bs in () if args.no_sweep else (2, 4, 8, 16, 32, 64):
        if 2 * Bs > R:
            break
        dk = dict(batch=Bs, num_heads=H, topk=w.topk, swa=w.swa, block_size=w.block_size,
                  num_blocks=R * nb, page_stride=stride, sm_scale=w.sm_scale,
                  max_blocks_per_seq=maxb, block_table_stride=maxb)
        plan_s = dsv4.dsv4_sparse_decode_plan(dsv4.make_desc(**dk), 0)
        Ss = plan_s.num_splits
        ws_s = torch.empty(max(plan_s.workspace_bytes, 16), dtype=torch.uint8, device=dev)
        desc_s = dsv4.make_desc(workspace=ws_s, **dk)
        q_s = q.expand(Bs, H, 512).contiguous()
        idx_s = idx.expand(Bs, Kt).contiguous()
        gs = torch.empty((Bs, Kt), dtype=torch.int32, device=dev)
        out_s = torch.empty((Bs, H, 512), dtype=torch.bfloat16, device=dev)
        lse_s = torch.empty((Bs, H), dtype=torch.float32, device=dev)
        nrot = R // Bs

        def step_s(r, Bs=Bs, Ss=Ss, desc_s=desc_s, q_s=q_s, idx_s=idx_s, gs=gs, out_s=out_s,
                   lse_s=lse_s, nrot=nrot):
            start = (r % nrot) * Bs
            dsv4.dsv4_sparse_decode_with_slots(desc_s, q_s, kv, bt_all[start:start + Bs], idx_s,
                                               None, sink, out_s, lse_s, Ss, gs)

        ms_s = time_graph(capture(step_s, K2), K2)
        bytes_s = Bs * (n_valid_slots * (ROW_BYTES + INDEX_BYTES) + H * 512 * 2 * 2)
        sweep.append({"B": Bs, "num_splits": Ss, "heads_per_group": plan_s.heads_per_group,
                      "ms_per_step": ms_s, "tokens_per_s": Bs * n_valid_slots / (ms_s * 1e-3),
                      "GBps": bytes_s / (ms_s * 1e-3) / 1e9,
                      "frac": bytes_s / (ms_s * 1e-3) / 1e9 / HBM_PEAK_GBPS})
        del ws_s, q_s, idx_s, gs, out_s, lse_s

    # The headline step at forced split counts (the selector picks 32).
    split_sweep = []
    for Sf in () if args.no_sweep else (8, 16, 32, 64):
        dk = dict(batch=B, num_heads=H, topk=w.topk, swa=w.swa, block_size=w.block_size,
                  num_blocks=R * nb, page_stride=stride, sm_scale=w.sm_scale,
                  max_blocks_per_seq=maxb, block_table_stride=maxb, flags=flags)
        plan_f = dsv4.dsv4_sparse_decode_plan(dsv4.make_desc(**dk), Sf)
        ws_f = torch.empty(max(plan_f.workspace_bytes, 16), dtype=torch.uint8, device=dev)
        desc_f = dsv4.make_desc(workspace=ws_f, **dk)

        def step_f(r, Sf=Sf, desc_f=desc_f):
            dsv4.dsv4_sparse_decode_with_slots(desc_f, q, kv, bt_all[r * B:(r + 1) * B], idx, None,
                                               sink, out, lse, Sf, gslots)

        ms_f = time_graph(capture(step_f, K2), K2)
        split_sweep.append({"num_splits": Sf, "heads_per_group": plan_f.heads_per_group,
                            "partial_kernel": ("short" if plan_f.partial_kernel ==
                                               dsv4.DSV4_KERNEL_SHORT else "pipelined"),
                            "ms_per_step": ms_f, "tokens_per_s": n_valid_slots / (ms_f * 1e-3)})
        del ws_f

    # Phase timeline of the headline partial kernel (short-split plans only):
    # the stamped variant on a cold replica, per-phase medians over the
    # workgroups in shader-clock cycles.
    timeline = short_timeline(dsv4, desc_tbl, plan_tbl, q, kv, bt_all, B, idx, sink, out, lse, S,
                              R)

    # A measured bandwidth reference: a 1 GiB device-to-device copy.
    csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    csrc.fill_(1)
    kt_copy = time_graph(capture(lambda r: cdst.copy_(csrc), 20), 20)
    copy_GBps = 2 * (1 << 30) / (kt_copy * 1e-3) / 1e9
    del csrc, cdst

    # Algorithmic work: valid entries (rows + index) and q per launch of the
    # partial kernel; flops 2*512*H per entry for QK and again for PV.
    n_valid = n_valid_slots
    part_bytes = n_valid * (ROW_BYTES + INDEX_BYTES) + B * H * 512 * 2
    step_bytes = part_bytes + B * H * (512 * 2 + 4)
    flops = n_valid * 2048 * H
    # A plain device copy of the partial kernel's algorithmic bytes, its
    # sources rotated so that every launch reads HBM: what one launch that
    # moves this little data takes without any dependent loads.
    crep = max(2, math.ceil(2 * INFINITY_CACHE_BYTES / part_bytes))
    csrc = torch.empty(crep * part_bytes, dtype=torch.uint8, device=dev)
    csrc.fill_(1)
    cdst = torch.empty(part_bytes, dtype=torch.uint8, device=dev)
    kt_copy_small = time_graph(capture(
        lambda r: cdst.copy_(csrc[(r % crep) * part_bytes:(r % crep + 1) * part_bytes]), K), K)
    del csrc, cdst
    tokens_per_s = n_valid / (ms_per_step * 1e-3)
    achieved = part_bytes / (kt_part * 1e-3) / 1e9
    digest = _source_digest()
    kname = _partial_kernel_name(plan_tbl, w.topk + w.swa, args.scrub)
    traffic = None if args.scrub else _traffic_from_profile(digest, kname)

    rec = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "attended KV tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "long_lowbatch: B=1 H=64 topk=2048 swa=0, 131072 slots/seq, block 64, "
                        "shuffled pages, 1% invalid, fp8_ds_mla rows, sink, sm_scale 512^-0.5",
            "B": B, "H": H, "topk": w.topk, "swa": w.swa, "block_size": w.block_size,
            "valid_entries": n_valid, "num_splits": S, "grid_partial": plan.grid_partial,
            "heads_per_group": plan.heads_per_group, "scrub": bool(args.scrub),
            "replicas": R, "cache_pool_GB": round(R * nb * stride / 1e9, 2),
            "graph_replay": not args.eager, "parallelism": "single GPU",
            "step": "partial kernel resolving the indices through the block table and "
                    "writing their global slots, then the combine",
        },
        "achieved_hbm_GBps_step": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "roofline": {
            "bound": "hbm",
            "kernel": kname,
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "frac_of_measured_copy": achieved / copy_GBps,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": part_bytes,
            "mfma_frac": flops / (kt_part * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
        },
        "kernels_ms": {"convert": kt_conv, "decode_partial": kt_part, "combine": kt_comb,
                       "decode_partial_global_slots": kt_part_slots},
        "floors_ms": {"gather_only": kt_gather, "empty_launch": kt_empty,
                      "partial_over_gather": kt_part / kt_gather,
                      "copy_of_partial_bytes": kt_copy_small,
                      "copy_of_partial_bytes_frac": part_bytes / (kt_copy_small * 1e-3) / 1e9
                      / HBM_PEAK_GBPS},
        "measured_copy_GBps": copy_GBps,
        "b_sweep": sweep,
        "split_sweep": split_sweep,
        "event_ms_per_step": ev_ms_per_step,
        "partial_timeline": timeline,
        "writer": {"rows": wn, "block_size": wbs, "sanitize": True, "replicas": wrep,
                   "ms": kt_writer, "algorithmic_bytes": writer_bytes,
                   "GBps": writer_bytes / (kt_writer * 1e-3) / 1e9,
                   "frac": writer_bytes / (kt_writer * 1e-3) / 1e9 / HBM_PEAK_GBPS},
        "cache_warm": {"ms_per_step": hot_ms_per_step, "decode_partial_ms": kt_part_hot,
                       "tokens_per_s": n_valid / (hot_ms_per_step * 1e-3)},
        "timed_output_matches_single_call": same,
        "launches_per_step": 2 if S > 1 else 1,
        "conversion_output_matches": conv_ok,
        "sequential_step": {
            "steps": "conversion, then the partial kernel over the global slots, then the "
                     "combine, in one stream",
            "launches_per_step": 3 if S > 1 else 2,
            "ms_per_step": seq_ms_per_step,
            "tokens_per_s": n_valid / (seq_ms_per_step * 1e-3),
            "output_matches_step": same_seq,
        },
        "kernel_source_digest": digest,
    }

    if not args.no_workloads:
        rec["workloads"] = workloads_leg(dev)
    if not args.no_context_parallel:
        rec["context_parallel_share"] = context_parallel_leg(dev, out, lse)
    if not args.no_two_kernel:
        rec["two_kernel_large_batch"] = two_kernel_leg(dev, capture_fn=None)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, out, lse, args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


def short_timeline(dsv4, desc, plan, q, kv, bt_all, B, idx, sink, out, lse, S, R):
    """Per-phase breakdown of the short-split kernel (include/dsv4_diag.h,
    dsv4_short_timeline) on the benchmark's inputs (block-table form): ten
    launches over cold replicas, stamps of the last; medians over its
    workgroups."""
    import torch
    if plan.partial_kernel != dsv4.DSV4_KERNEL_SHORT:
        return None
    stamps = torch.zeros(plan.grid_partial * 10, dtype=torch.int64, device=q.device)
    for i in range(10):
        r = (R - 1 - i) % R
        dsv4.dsv4_short_timeline(desc, q, kv, bt_all[r * B:(r + 1) * B], idx, None, sink, out,
                                 lse, S, stamps)
    torch.cuda.synchronize()
    t = stamps.view(-1, 10).cpu().numpy().astype(np.int64)
    t = t[t[:, 1] > 0]
    cyc = t[:, 8] - t[:, 1]
    real = np.maximum(1, t[:, 9] - t[:, 0])
    mhz = float(np.median(cyc / real * 100.0))
    names = ["resolve_and_issue", "dequant_st0", "barrier_wait", "qk", "softmax", "pv_and_rest",
             "epilogue"]
    phases = {n: int(np.median(t[:, k + 2] - t[:, k + 1])) for k, n in enumerate(names)}
    one = "true" if _one_super_tile(plan, idx.shape[1]) else "false"
    return {"kernel": f"decode_short_kernel<{plan.heads_per_group}, false, true, true, false, "
                      f"{one}> (stamped variant)",
            "workgroups": int(t.shape[0]), "clock_MHz": mhz,
            "wg_span_us_median": float(np.median(real)) / 100.0,
            "wg_start_spread_us": float(t[:, 0].max() - t[:, 0].min()) / 100.0,
            "phase_cycles_median": phases}


def profile_workload(ci: int, steps: int) -> int:
    """Runs the fused decode of one of the five workloads `steps` times,
    launch after launch, so that a profiler's counters can be averaged per
    dispatch; prints the valid entries and algorithmic flops of one call."""
    import torch
    import sparse_mla_attention_block_amd as dsv4
    from synth import make_workload
    w = make_workload(ci)
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev) if a is not None else None
    q = t(w.q.view(np.int16)).view(torch.bfloat16)
    kv, bt, idx, vl, sink = t(w.kv), t(w.block_table), t(w.topk_idx), t(w.valid_len), t(w.sink)
    out = torch.empty((w.B, w.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
    dk = dict(batch=w.B, num_heads=w.H, topk=w.topk, swa=w.swa, block_size=w.block_size,
              num_blocks=w.num_blocks, page_stride=w.page_stride, sm_scale=w.sm_scale,
              max_blocks_per_seq=w.max_blocks_per_seq, block_table_stride=w.block_table.shape[1])
    if w.per_row_splits:                       # the configuration's per-row split count
        dk["flags"] = dsv4.DSV4_DECODE_BALANCE
    plan = dsv4.dsv4_sparse_decode_plan(dsv4.make_desc(**dk), w.num_splits)
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
    desc = dsv4.make_desc(workspace=ws, **dk)
    for _ in range(steps):
        dsv4.dsv4_sparse_decode(desc, q, kv, bt, idx, vl, sink, out, lse, w.num_splits)
    torch.cuda.synchronize()
    n_valid = 0
    for b in range(w.B):
        v = w.topk if w.valid_len is None else min(max(int(w.valid_len[b]), 0), w.topk)
        n_valid += int((w.topk_idx[b, :v] >= 0).sum() + (w.topk_idx[b, w.topk:] >= 0).sum())
    print(json.dumps({"workload": w.name, "valid_entries": n_valid,
                      "algorithmic_flops": n_valid * 2048 * w.H,
                      "heads_per_group": plan.heads_per_group, "num_splits": plan.num_splits,
                      "balanced_splits": plan.balanced_splits, "launches": steps}), flush=True)
    return 0


def _valid_entries(w) -> int:
    """Entries that take part: index >= 0, inside valid_len for the main
    part, and on a page the sequence's block table names."""
    seq = np.arange(w.B) // w.s_q
    k = np.arange(w.Kt)[None, :]
    vl = (np.clip(w.valid_len[seq], 0, w.topk) if w.valid_len is not None
          else np.full(w.B, w.topk))[:, None]
    ti = w.topk_idx
    blk = np.where(ti >= 0, ti // w.block_size, 0)
    inb = blk < w.max_blocks_per_seq
    page = w.block_table[seq[:, None], np.where(inb, blk, 0)]
    live = (ti >= 0) & ((k >= w.topk) | (k < vl)) & inb & (page >= 0) & (page < w.num_blocks)
    return int(live.sum())


def workloads_leg(dev, K=100, pool_cap_bytes=8 << 30):
    """The library's decode (partial kernel, then the combine when the plan
    splits) on each of the five seeded workloads, at the plan the selector
    picks (the tiny workload forces one split).  Average launch durations
    from HIP graphs of K decodes: warm (one copy of the cache) and cold (the
    cache rotated over R replicas, R sized so that the rows read between two
    uses of a replica exceed twice the Infinity Cache, within
    pool_cap_bytes; `MB_between_reuse` says how far that got).  Throughput
    and the roofline fractions use the cold time and the algorithmic work:
    584 + 4 bytes and 2048*H flops per valid entry, q read, output and lse
    written."""
    import torch
    import sparse_mla_attention_block_amd as dsv4
    from synth import CONFIGS, make_workload
    res = []
    for ci in range(len(CONFIGS)):
        w = make_workload(ci)
        B, H, Kt = w.B, w.H, w.Kt
        nb, stride = w.num_blocks, w.page_stride
        n_valid = _valid_entries(w)
        touched = n_valid * (ROW_BYTES + 64)
        R = max(1, min(math.ceil(2 * INFINITY_CACHE_BYTES / touched),
                       pool_cap_bytes // (nb * stride), K))
        base = torch.from_numpy(w.kv).to(dev)
        pool = torch.empty((R, nb, stride), dtype=torch.uint8, device=dev)
        pool.copy_(base.unsqueeze(0).expand(R, nb, stride))
        del base
        bt0 = torch.from_numpy(w.block_table.astype(np.int64)).to(dev)
        bts = [torch.where(bt0 >= 0, bt0 + r * nb, -1).to(torch.int32).contiguous()
               for r in range(R)]
        idx = torch.from_numpy(w.topk_idx).to(dev)
        vl = None if w.valid_len is None else torch.from_numpy(w.valid_len).to(dev)
        q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
        sink = torch.from_numpy(w.sink).to(dev)
        out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        kw = dict(batch=B, num_heads=H, topk=w.topk, swa=w.swa, block_size=w.block_size,
                  num_blocks=R * nb, page_stride=stride, sm_scale=w.sm_scale,
                  max_blocks_per_seq=w.max_blocks_per_seq,
                  block_table_stride=w.block_table.shape[1], tokens_per_seq=w.s_q)
        # The ragged batch's configuration chooses the split count per row:
        # balanced splits (the uniform selector plan is timed beside it).
        flags = dsv4.DSV4_DECODE_BALANCE if w.per_row_splits else 0
        plan = dsv4.dsv4_sparse_decode_plan(dsv4.make_desc(flags=flags, **kw), w.num_splits)
        ws = (torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
              if plan.workspace_bytes else None)
        desc = dsv4.make_desc(workspace=ws, flags=flags, **kw)
        desc_pipe = dsv4.make_desc(workspace=ws, flags=flags | dsv4.DSV4_DECODE_PIPELINED, **kw)
        kv = pool.view(-1)

        def timed(rot, d=desc, S=w.num_splits):
            def decode(r):
                dsv4.dsv4_sparse_decode(d, q, kv, bts[r], idx, vl, sink, out, lse, S)

            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                decode(0)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(K):
                    decode(i % R if rot else 0)
            g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / K * 1e3

        warm_us = timed(False)
        cold_us = timed(True)
        kname = "short" if plan.partial_kernel == dsv4.DSV4_KERNEL_SHORT else "pipelined"
        pipe = {"pipelined_warm_us": timed(False, desc_pipe),
                "pipelined_cold_us": timed(True, desc_pipe)} if kname != "pipelined" else {}
        # The short-context batch's configured plan (split-K capped at 4, the
        # pages' short-list cap) beside the selector's.
        cap4 = {}
        if w.name == "short_batch":
            plan4 = dsv4.dsv4_sparse_decode_plan(dsv4.make_desc(**kw), 4)
            cap4 = {"cap4_plan": {
                "num_splits": plan4.num_splits, "heads_per_group": plan4.heads_per_group,
                "partial_kernel": ("short" if plan4.partial_kernel == dsv4.DSV4_KERNEL_SHORT
                                   else "pipelined"),
                "warm_us": timed(False, desc, 4), "cold_us": timed(True, desc, 4)}}
        nbytes = n_valid * (ROW_BYTES + INDEX_BYTES) + B * H * (512 * 2 * 2 + 4)
        flops = n_valid * 2048 * H
        # Per-row split counts: the uniform selector plan of the same decode.
        uni = {}
        if w.per_row_splits:
            planu = dsv4.dsv4_sparse_decode_plan(dsv4.make_desc(**kw), w.num_splits)
            wsu = (torch.empty(planu.workspace_bytes, dtype=torch.uint8, device=dev)
                   if planu.workspace_bytes else None)
            descu = dsv4.make_desc(workspace=wsu, **kw)
            uw, uc = timed(False, descu), timed(True, descu)
            uni = {"uniform_plan": {
                "num_splits": planu.num_splits, "warm_us": uw, "cold_us": uc,
                "GBps": nbytes / (uc * 1e-6) / 1e9,
                "frac_hbm": nbytes / (uc * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                "TFLOPs": flops / (uc * 1e-6) / 1e12,
                "frac_mfma": flops / (uc * 1e-6) / 1e12 / BF16_PEAK_TFLOPS}}
            del wsu
        gbps = nbytes / (cold_us * 1e-6) / 1e9
        tflops = flops / (cold_us * 1e-6) / 1e12
        res.append({
            "workload": w.name, "B": B, "H": H, "topk": w.topk, "swa": w.swa,
            "valid_entries": n_valid, "heads_per_group": plan.heads_per_group,
            "num_splits": plan.num_splits, "grid_partial": plan.grid_partial,
            "partial_kernel": kname, "balanced_splits": plan.balanced_splits,
            **pipe, **cap4, **uni,
            "replicas": R, "MB_between_reuse": round(R * touched / 1e6, 1),
            "warm_us": warm_us, "cold_us": cold_us,
            "tokens_per_s": n_valid / (cold_us * 1e-6),
            "algorithmic_bytes": nbytes, "GBps": gbps, "frac_hbm": gbps / HBM_PEAK_GBPS,
            "TFLOPs": tflops, "frac_mfma": tflops / BF16_PEAK_TFLOPS,
        })
        del pool, bts, ws, kv
        torch.cuda.empty_cache()
    return res


def context_parallel_leg(dev, full_out, full_lse, K=100, pool_cap_bytes=8 << 30):
    """One GPU's part of a context-parallel decode of the benchmark workload
    over n = 2, 4, 8 GPUs: each GPU decodes its share of the index list
    (topk / n entries, no sink) into a normalised output and lse, the n
    results are all-gathered (not run: one GPU) and merged with the sink by
    the combine.  Times: the share's decode, cold over rotating cache
    replicas and warm; the final combine of n partials.  All n shares are
    also decoded and merged here, and the merge is compared with the
    benchmark's own full decode (`max_abs_out_diff_vs_full`)."""
    import torch
    import sparse_mla_attention_block_amd as dsv4
    from synth import make_workload
    w = make_workload(WORKLOAD_CONFIG)
    B, H, Kt = w.B, w.H, w.Kt
    nb, stride = w.num_blocks, w.page_stride
    n_valid = _valid_entries(w)
    R = max(1, min(K, pool_cap_bytes // (nb * stride)))
    base = torch.from_numpy(w.kv).to(dev)
    pool = torch.empty((R, nb, stride), dtype=torch.uint8, device=dev)
    pool.copy_(base.unsqueeze(0).expand(R, nb, stride))
    del base
    bt0 = torch.from_numpy(w.block_table.astype(np.int64)).to(dev)
    bts = [torch.where(bt0 >= 0, bt0 + r * nb, -1).to(torch.int32).contiguous() for r in range(R)]
    idx = torch.from_numpy(w.topk_idx).to(dev)
    q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
    sink = torch.from_numpy(w.sink).to(dev)
    kv = pool.view(-1)

    def graph_us(fn, rot):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(0)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(K):
                fn(i % R if rot else 0)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K * 1e3

    res = []
    for n in (2, 4, 8):
        m = w.topk // n
        kw = dict(batch=B, num_heads=H, topk=m, swa=0, block_size=w.block_size,
                  num_blocks=R * nb, page_stride=stride, sm_scale=w.sm_scale,
                  max_blocks_per_seq=w.max_blocks_per_seq,
                  block_table_stride=w.block_table.shape[1], topk_idx_stride=Kt)
        plan = dsv4.dsv4_sparse_decode_plan(dsv4.make_desc(**kw), 0)
        ws = (torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
              if plan.workspace_bytes else None)
        desc = dsv4.make_desc(workspace=ws, **kw)
        part_out = torch.empty((B, H, n, 512), dtype=torch.bfloat16, device=dev)
        part_lse = torch.empty((B, H, n), dtype=torch.float32, device=dev)
        so = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
        sl = torch.empty((B, H), dtype=torch.float32, device=dev)
        for i in range(n):                        # every share, for the merge check
            dsv4.dsv4_sparse_decode(desc, q, kv, bts[0], idx[:, i * m:], None, None, so, sl, 0)
            part_out[:, :, i] = so
            part_lse[:, :, i] = sl
        mo = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
        ml = torch.empty((B, H), dtype=torch.float32, device=dev)

        def share(r):
            dsv4.dsv4_sparse_decode(desc, q, kv, bts[r], idx, None, None, so, sl, 0)

        def merge(r):
            dsv4.dsv4_combine_splits(B, H, n, part_out, part_lse, sink, mo, ml)

        merge(0)
        torch.cuda.synchronize()
        diff = (mo.float() - full_out.float()).abs().max().item()
        dlse = (ml - full_lse).abs().max().item()
        cold = graph_us(share, True)
        warm = graph_us(share, False)
        comb = graph_us(merge, False)
        res.append({
            "gpus": n, "share_entries": m, "heads_per_group": plan.heads_per_group,
            "num_splits": plan.num_splits, "share_decode_us_cold": cold,
            "share_decode_us_warm": warm, "final_combine_us": comb,
            "per_gpu_us_without_exchange": cold + comb,
            "all_gather_bytes_in_per_gpu": (n - 1) * B * H * (512 * 2 + 4),
            "max_abs_out_diff_vs_full": diff, "max_abs_lse_diff_vs_full": dlse,
        })
        del ws
    del pool, bts, kv
    torch.cuda.empty_cache()
    return {"workload": "long_lowbatch shares: B=1 H=64, topk 2048 cut into n contiguous shares",
            "replicas": R, "valid_entries_full": n_valid, "shares": res}


def two_kernel_leg(dev, capture_fn=None, K=50):
    """Fused decode against the two-kernel path (gather + dequantise into
    dense bf16 rows, then attention over them) on the large-batch workload
    (B=256, H=64, top-k 512 + SWA 128, 8192 slots per sequence): average
    launch durations from HIP graphs of K launches each, the cache rotated
    over replicas so that every launch reads its rows from HBM."""
    import torch
    import sparse_mla_attention_block_amd as dsv4
    from synth import make_workload
    w = make_workload(3)
    B, H, Kt = w.B, w.H, w.Kt
    nb, stride = w.num_blocks, w.page_stride
    n_valid = int((w.topk_idx >= 0).sum())
    R = max(1, math.ceil(2 * INFINITY_CACHE_BYTES / (n_valid * (ROW_BYTES + 64))))
    base = torch.from_numpy(w.kv).to(dev)
    pool = torch.empty((R, nb, stride), dtype=torch.uint8, device=dev)
    pool.copy_(base.unsqueeze(0).expand(R, nb, stride))
    del base
    bt0 = torch.from_numpy(w.block_table.astype(np.int64)).to(dev)
    bts = [torch.where(bt0 >= 0, bt0 + r * nb, -1).to(torch.int32).contiguous() for r in range(R)]
    idx = torch.from_numpy(w.topk_idx).to(dev)
    q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
    sink = torch.from_numpy(w.sink).to(dev)
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    dense = torch.empty((B, Kt, 512), dtype=torch.bfloat16, device=dev)
    mask = torch.empty((B, Kt), dtype=torch.uint8, device=dev)
    desc = dsv4.make_desc(batch=B, num_heads=H, topk=w.topk, swa=w.swa, block_size=w.block_size,
                          num_blocks=R * nb, page_stride=stride, sm_scale=w.sm_scale,
                          max_blocks_per_seq=w.max_blocks_per_seq,
                          block_table_stride=w.block_table.shape[1])
    plan = dsv4.dsv4_sparse_decode_plan(desc, 0)
    assert plan.num_splits == 1            # no split-K at >= 256 tokens: no workspace
    kv = pool.view(-1)

    def fused(r):
        dsv4.dsv4_sparse_decode(desc, q, kv, bts[r], idx, None, sink, out, lse, 0)

    def gather(r):
        dsv4.dsv4_gather_dequant(desc, kv, bts[r], idx, None, dense, mask)

    def attend(r):
        dsv4.dsv4_dense_decode(desc, q, dense, mask, sink, out, lse, 0)

    def timed(fn):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(0)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(K):
                fn(i % R)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K * 1e3

    t_fused = timed(fused)
    fused_out = out.clone()
    t_gather = timed(gather)
    t_attend = timed(attend)
    gather(0)
    attend(0)
    torch.cuda.synchronize()
    diff = (out.float() - fused_out.float()).abs().max().item()
    kv_bytes = n_valid * (ROW_BYTES + INDEX_BYTES)
    dense_bytes = B * Kt * (1024 + 1)
    return {
        "workload": "large_batch: B=256 H=64 topk=512 swa=128, 8192 slots/seq, block 64",
        "replicas": R, "launches": K,
        "fused_us": t_fused, "gather_us": t_gather, "dense_attention_us": t_attend,
        "two_kernel_us": t_gather + t_attend,
        "fused_speedup": (t_gather + t_attend) / t_fused,
        "fused_GBps": kv_bytes / (t_fused * 1e-6) / 1e9,
        "gather_GBps": (kv_bytes + dense_bytes) / (t_gather * 1e-6) / 1e9,
        "dense_attention_GBps": dense_bytes / (t_attend * 1e-6) / 1e9,
        "max_abs_out_diff_vs_fused": diff,
    }


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, out_gpu, lse_gpu, seconds):
    """The fp64 CPU oracle, as it stands, timed on this host over repeated
    full decodes of the same workload (about `seconds` of CPU work)."""
    import oracle
    threads = oracle.default_threads()
    reps, n_valid = 0, 0
    t0 = time.perf_counter()
    ref = None
    while True:
        ref_out, ref_lse, n_valid = oracle.decode_workload(w, nthreads=threads)
        reps += 1
        if ref is None:
            ref = (ref_out, ref_lse)
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    # The same oracle on one thread, over a third of the time budget.
    reps1 = 0
    t1 = time.perf_counter()
    while True:
        oracle.decode_workload(w, nthreads=1)
        reps1 += 1
        if time.perf_counter() - t1 >= seconds / 3:
            break
    dt1 = time.perf_counter() - t1
    got = out_gpu.float().double().cpu().numpy()
    err = np.abs(got - ref[0])
    bound = 2e-2 + 1e-2 * np.abs(ref[0])
    lse_err = float(np.max(np.abs(lse_gpu.double().cpu().numpy() - ref[1])))
    return {
        "value": reps * n_valid / dt,
        "unit": "attended KV tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{reps} full decodes of the benchmark workload ({n_valid} valid entries x "
                  f"64 heads each), fp64 C oracle, {threads} threads, {dt:.1f} s",
        "host_cpus": os.cpu_count(),
        "cpu_model": _cpu_model(),
        "single_thread": {"value": reps1 * n_valid / dt1, "cores": 1,
                          "sample": f"{reps1} full decodes, 1 thread, {dt1:.1f} s"},
        "parity_vs_gpu": {"max_abs_out_err": float(err.max()),
                          "within_tolerance": bool((err <= bound).all()) and lse_err <= 1e-3,
                          "max_abs_lse_err": lse_err},
    }


if __name__ == "__main__":
    sys.exit(main())
