#!/usr/bin/env python3
"""Benchmark of the rx hot path on one MI355X.

One step = one pass of every hot-path operation over one batch of synthetic
rank buffers (N = 8 separate HBM allocations):
  1. DDA flat local reduce              rx_reduce_flat
  2. DDA tree per-rank step             rx_reduce_scatter_chunk_bcast (rank = step % N)
  3. FP8 block quantizer                rx_quant_fp8
  4. fused dequant-reduce-requant, with the dequantized high-precision
     output                             rx_dequant_reduce_requant (REQUANT + hp)

The default workload is the decode-size message: 8 x 32x8192 BF16 (512 KiB
per rank), low-precision leg in E5M2 with 256-element blocks. Inputs are
resident in HBM before timing starts; the batches rotate over enough copies
(>= 2 GiB in total) that every step reads its inputs from HBM rather than
from the 256 MB Infinity Cache. The low-precision tree step (one rank's
share of a low-precision reduce-scatter + all-gather), the separate
dequantization pass, the flat low-precision sum without requantization and
the in-place one-device allreduces (rx_allreduce_local, flat / tree / low
precision) are timed beside the step, as is the tree step for each rank on
its own (`tree_step_by_rank_us`), and the flat reduce over the first k rank
buffers for k = 1..N (`reduce_flat_us_by_nsrc`).

Output: one JSON line (see the fields below). Per-kernel times come from HIP
events around back-to-back launches of that kernel alone, on the stream the
kernel runs on; `rocprofv3 --kernel-trace --stats` of the same command
reports the per-dispatch durations.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD published peak
METRIC = "effective HBM GB/s (% of MI355X peak) per reduce kernel; µs at 512 KB msg"

KERNEL_SOURCES = {
    "reduce_flat": ["reduce.hip", "rx_device.hpp"],
    "tree_step": ["reduce.hip", "rx_device.hpp"],
    "quant_fp8": ["quant.hip", "rx_device.hpp"],
    "dequant_reduce_requant": ["drr.hpp", "drr.hip", "rx_device.hpp"],
    "lp_tree_step": ["drr.hpp", "drr.hip", "rx_device.hpp"],
    "dequant_separate": ["drr.hpp", "drr.hip", "rx_device.hpp"],
    "lp_flat_sum": ["drr.hpp", "drr.hip", "rx_device.hpp"],
    "allreduce_local_flat": ["reduce.hip", "rx_device.hpp"],
    "allreduce_local_tree": ["reduce.hip", "rx_device.hpp"],
    "allreduce_local_lowprec": ["quant.hip", "drr.hpp", "drr.hip", "rx_device.hpp"],
}
# rocprofv3 kernel names (substrings of the mangled names)
KERNEL_SYMBOLS = {
    "reduce_flat": "k_reduce_flat",
    "tree_step": "k_tree",
    "quant_fp8": "k_quant",
    "dequant_reduce_requant": "k_drr",
    "lp_tree_step": "k_drr",
    "dequant_separate": "k_drr",
    "lp_flat_sum": "k_drr",
    "allreduce_local_flat": "k_tree",
    "allreduce_local_tree": "k_tree (N launches)",
    "allreduce_local_lowprec": "k_quant, k_drr",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode",
                   help="decode | tree | lp_fp32 | lp_bf16 | flat_uniform")
    p.add_argument("--kernel-reps", type=int, default=0,
                   help="launches per kernel-only timing (0 = auto)")
    p.add_argument("--warm", action="store_true",
                   help="reuse one batch every step (cache-warm; labelled)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true",
                   help="launch from a Python loop instead of replaying HIP graphs")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    return p.parse_args()


def sha_of(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "allreduce_reduction_rx_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary
    (profiles/traffic_<workload>.md), or None when absent or when the
    kernel's source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    want = sha_of(KERNEL_SOURCES[kernel])
    for line in open(path):
        m = re.match(r"- (\w+): source_sha256=(\w+) hbm_bytes_per_launch=(\d+)", line.strip())
        if m and m.group(1) == kernel:
            return float(m.group(3)) if m.group(2) == want else None
    return None


class Batch:
    """One set of device buffers for a step."""

    def __init__(self, w, srcs_dev, lp_fmt, lp_block, torch):
        dev = srcs_dev[0].device
        n, count = w.nsrc, w.count
        dt = srcs_dev[0].dtype
        nb = -(-count // lp_block)
        self.srcs = srcs_dev
        self.flat_out = torch.empty(count, dtype=dt, device=dev)
        self.tree_dsts = [torch.empty(count, dtype=dt, device=dev) for _ in range(n)]
        self.codes = [torch.empty(count, dtype=torch.uint8, device=dev) for _ in range(n)]
        self.scales = [torch.empty(nb, dtype=torch.float32, device=dev) for _ in range(n)]
        self.out_codes = torch.empty(count, dtype=torch.uint8, device=dev)
        self.out_scales = torch.empty(nb, dtype=torch.float32, device=dev)
        self.out_hp = torch.empty(count, dtype=dt, device=dev)
        self.lp_dst_codes = [torch.empty(count, dtype=torch.uint8, device=dev) for _ in range(n)]
        self.lp_dst_scales = [torch.empty(nb, dtype=torch.float32, device=dev) for _ in range(n)]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only (got --gpus {args.gpus}); "
              "the multi-GPU collective is out of scope here", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import allreduce_reduction_rx_amd as rx
    import rxgen as G

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    rx.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    w = G.WORKLOADS[args.workload]
    n, count = w.nsrc, w.count
    e = w.elem_bytes
    if w.fp8:
        lp_fmt, lp_block = w.fp8, w.block
    else:
        lp_fmt, lp_block = ("e5m2", 256) if w.dtype == G.BF16 else ("e4m3", 128)
    nb = -(-count // lp_block)
    tdt = torch.bfloat16 if w.dtype == G.BF16 else torch.float32

    # ---- inputs: generate once on the host, upload, replicate on device ----
    host = w.sources()
    base = []
    for h in host:
        t = torch.from_numpy(h.view(np.int16) if h.dtype == np.uint16 else h).to(dev)
        base.append(t.view(tdt) if h.dtype == np.uint16 else t)
    chunk_lo, chunk_hi = rx.rx_tree_chunk(count, n, w.dtype, 0)
    chunk = chunk_hi - chunk_lo

    lp_lo, lp_hi = rx.rx_lp_tree_chunk(count, n, lp_block, 0)
    lp_chunk = lp_hi - lp_lo
    bytes_k = {
        "reduce_flat": n * count * e + count * e,
        "tree_step": 2 * n * chunk * e,
        "quant_fp8": n * (count * e + count + 4 * nb),
        "dequant_reduce_requant": n * (count + 4 * nb) + (count + 4 * nb) + count * e,
    }
    step_bytes = sum(bytes_k.values())
    # measured beside the step, not part of it: the low-precision tree step
    # and the whole local allreduce (every buffer read once and written once;
    # low precision: quantize every buffer, then one pass that reduces,
    # requantizes, dequantizes and writes every buffer)
    bytes_k["lp_tree_step"] = 2 * n * (lp_chunk + 4 * (lp_chunk // lp_block))
    # the separate dequantization of the requantized message (SUM, one
    # source) and the flat low-precision reduce without requantization (SUM
    # over the N quantized sources), both into the message's dtype
    bytes_k["dequant_separate"] = (count + 4 * nb) + count * e
    bytes_k["lp_flat_sum"] = n * (count + 4 * nb) + count * e
    bytes_k["allreduce_local_flat"] = 2 * n * count * e
    bytes_k["allreduce_local_tree"] = 2 * n * count * e
    bytes_k["allreduce_local_lowprec"] = (n * (count * e + count + 4 * nb)   # quantize
                                          + n * (count + 4 * nb) + n * count * e)  # reduce + write all
    per_batch_bytes = (n * count * e            # sources
                       + count * e              # flat out
                       + n * count * e          # tree destinations
                       + n * (count + 4 * nb)   # codes + scales
                       + count + 4 * nb + count * e
                       + n * (count + 4 * nb))    # low-precision tree destinations
    if args.warm:
        nsets = 1
    else:
        nsets = max(1, min(256, -(-(2 << 30) // per_batch_bytes)))
    free, _ = torch.cuda.mem_get_info()
    nsets = max(1, min(nsets, int(0.6 * free // per_batch_bytes)))
    batches = [Batch(w, base, lp_fmt, lp_block, torch)]
    for _ in range(nsets - 1):
        batches.append(Batch(w, [b.clone() for b in base], lp_fmt, lp_block, torch))
    torch.cuda.synchronize()

    def k_flat(b, i):
        rx.rx_reduce_flat(b.srcs, b.flat_out)

    def k_tree(b, i):
        rx.rx_reduce_scatter_chunk_bcast(b.srcs, i % n, b.tree_dsts)

    def k_quant(b, i):
        rx.rx_quant_fp8(b.srcs, lp_fmt, lp_block, b.codes, b.scales)

    def k_drr(b, i):
        rx.rx_dequant_reduce_requant(b.codes, b.scales, lp_fmt, lp_block, rx.RX_DRR_REQUANT,
                                     b.out_codes, b.out_scales, b.out_hp)

    def k_lp_tree(b, i):
        rx.rx_lp_reduce_scatter_chunk_bcast(b.codes, b.scales, lp_fmt, lp_block, i % n,
                                            b.lp_dst_codes, b.lp_dst_scales)

    def k_dequant(b, i):
        rx.rx_dequant_reduce_requant([b.out_codes], [b.out_scales], lp_fmt, lp_block,
                                     rx.RX_DRR_SUM, out_hp=b.out_hp)

    def k_lp_flat(b, i):
        rx.rx_dequant_reduce_requant(b.codes, b.scales, lp_fmt, lp_block, rx.RX_DRR_SUM,
                                     out_hp=b.out_hp)

    kernels = [("reduce_flat", k_flat), ("tree_step", k_tree),
               ("quant_fp8", k_quant), ("dequant_reduce_requant", k_drr)]

    def step(i):
        b = batches[i % nsets]
        for _, fn in kernels:
            fn(b, i)

    # whole in-place local allreduce (rx_allreduce_local), on buffers of
    # zeros so that repeated in-place sums stay finite (kernel time does not
    # depend on the values)
    ar_bufs = [[torch.zeros(count, dtype=tdt, device=dev) for _ in range(n)]
               for _ in range(max(1, min(nsets, 32)))]
    ws_bytes = rx.rx_allreduce_local_workspace(n, count, lp_block)
    ar_ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def k_ar_flat(b, i):
        rx.rx_allreduce_local(ar_bufs[i % len(ar_bufs)], rx.RX_ALGO_FLAT, lp_fmt, lp_block)

    def k_ar_tree(b, i):
        rx.rx_allreduce_local(ar_bufs[i % len(ar_bufs)], rx.RX_ALGO_TREE, lp_fmt, lp_block)

    def k_ar_lp(b, i):
        rx.rx_allreduce_local(ar_bufs[i % len(ar_bufs)], rx.RX_ALGO_LOWPREC, lp_fmt, lp_block, ar_ws)

    kernels_timed = kernels + [("lp_tree_step", k_lp_tree), ("dequant_separate", k_dequant),
                               ("lp_flat_sum", k_lp_flat), ("allreduce_local_flat", k_ar_flat),
                               ("allreduce_local_tree", k_ar_tree),
                               ("allreduce_local_lowprec", k_ar_lp)]

    def capture(calls):
        """HIP graph of the given launches (captured on torch's capture
        stream, which is the stream the binding launches on)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in calls:
                c()
        return g

    def timed(run, reps_inner):
        """ms per inner repetition of run(), HIP events on the launch stream."""
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        run()
        z.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(z) / reps_inner

    # ---- whole-step timing: W untimed steps, then exactly K timed steps ----
    if args.no_graph:
        for i in range(args.warmup):
            step(i)
        t_wall = time.perf_counter()
        step_ms = timed(lambda: [step(i) for i in range(args.steps)], args.steps)
        wall_s = time.perf_counter() - t_wall
    else:
        g_warm = capture([lambda i=i: step(i) for i in range(max(1, args.warmup))])
        g_steps = capture([lambda i=i: step(i) for i in range(args.steps)])
        if args.warmup:
            g_warm.replay()
        t_wall = time.perf_counter()
        step_ms = timed(g_steps.replay, args.steps)
        wall_s = time.perf_counter() - t_wall
        del g_warm, g_steps

    # ---- per-kernel timing: back-to-back launches of one kernel ----
    per_kernel = {}
    for name, fn in kernels_timed:
        reps = args.kernel_reps or max(50, min(2000, int(0.05 / max(1e-7, bytes_k[name] / 4e12))))
        calls = [lambda i=i: fn(batches[i % nsets], i) for i in range(reps)]
        if args.no_graph:
            for c in calls[:10]:
                c()
            us = timed(lambda: [c() for c in calls], reps) * 1000.0
        else:
            g = capture(calls)
            g.replay()
            us = timed(g.replay, reps) * 1000.0
            del g
        gbs = bytes_k[name] / (us * 1e-6) / 1e9
        per_kernel[name] = {"us": round(us, 3), "GB/s": round(gbs, 1),
                            "frac": round(gbs / PEAK_HBM_GBS, 4),
                            "bytes": bytes_k[name], "launches": reps}

    # ---- the tree step for each rank on its own (median over ranks) ----
    by_rank = []
    for k in range(n):
        reps = per_kernel["tree_step"]["launches"]
        calls = [lambda i=i, k=k: rx.rx_reduce_scatter_chunk_bcast(batches[i % nsets].srcs, k,
                                                                   batches[i % nsets].tree_dsts)
                 for i in range(reps)]
        if args.no_graph:
            us = timed(lambda: [c() for c in calls], reps) * 1000.0
        else:
            g = capture(calls)
            g.replay()
            us = timed(g.replay, reps) * 1000.0
            del g
        by_rank.append(round(us, 3))

    # ---- the flat reduce over the first k rank buffers, k = 1..N (DDA
    # flat's latency against the number of ranks, one GPU's share) ----
    flat_by_nsrc = []
    for k in range(1, n + 1):
        reps = per_kernel["reduce_flat"]["launches"]
        calls = [lambda i=i, k=k: rx.rx_reduce_flat(batches[i % nsets].srcs[:k],
                                                    batches[i % nsets].flat_out)
                 for i in range(reps)]
        if args.no_graph:
            us = timed(lambda: [c() for c in calls], reps) * 1000.0
        else:
            g = capture(calls)
            g.replay()
            us = timed(g.replay, reps) * 1000.0
            del g
        flat_by_nsrc.append(round(us, 3))

    # ---- parity spot check of batch 0 against the oracle-free invariants:
    # the tree chunk must equal the flat result on that chunk ----
    b0 = batches[0]
    rx.rx_reduce_flat(b0.srcs, b0.flat_out)
    rx.rx_reduce_scatter_chunk_bcast(b0.srcs, 0, b0.tree_dsts)
    torch.cuda.synchronize()
    lo, hi = rx.rx_tree_chunk(count, n, w.dtype, 0)
    tree_ok = all(torch.equal(d[lo:hi].view(torch.int16 if tdt == torch.bfloat16 else torch.int32),
                              b0.flat_out[lo:hi].view(torch.int16 if tdt == torch.bfloat16 else torch.int32))
                  for d in b0.tree_dsts)

    dominant = max((k for k, _ in kernels), key=lambda k: per_kernel[k]["us"])
    dk = per_kernel[dominant]
    traffic = read_traffic(dominant, args.workload)
    value = step_bytes / (step_ms * 1e-3) / 1e9

    us_single, us_events = single_launch_us(torch, rx, k_flat, batches, stream)
    floors = launch_floors(torch, rx, n * count * e) if n * count * e <= (64 << 20) else None
    copy = copy_ceiling(torch, stream)
    ceil = stream_ceilings(torch, rx, stream)
    for k in per_kernel.values():
        k["frac_of_copy_ceiling"] = round(k["GB/s"] / ceil["copy"]["GB/s"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, host, lp_fmt, lp_block, args.cpu_seconds, step_bytes)

    e_name = "BF16" if w.dtype == G.BF16 else "FP32"
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {n} x {count} {e_name} rank buffers "
                        f"({count * e / 1024:.0f} KiB each), step = flat reduce + tree step "
                        f"(chunk {chunk}) + FP8 quant ({lp_fmt}, block {lp_block}) + "
                        f"dequant-reduce-requant with {e_name} output",
            "nsrc": n, "count": count, "io_dtype": e_name.lower(),
            "fp8": lp_fmt, "block": lp_block,
            "cache": "warm (one batch reused)" if args.warm else f"cold (rotating {nsets} batches, "
                     f"{nsets * per_batch_bytes / 2**30:.2f} GiB)",
            "step_bytes": step_bytes,
        },
        "roofline": {
            "bound": "hbm", "kernel": dominant,
            "achieved": dk["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(dk["GB/s"] / PEAK_HBM_GBS, 4),
            "traffic": traffic,
        },
        "kernels": per_kernel,
        "us_reduce_flat": per_kernel["reduce_flat"]["us"],
        "reduce_flat_us_by_nsrc": flat_by_nsrc,
        "tree_step_by_rank_us": by_rank,
        "tree_step_median_over_ranks_us": sorted(by_rank)[len(by_rank) // 2],
        "us_reduce_flat_single_launch": us_single,
        "us_event_pair_alone": us_events,
        "launch_floors": floors,
        "tree_matches_flat": bool(tree_ok),
        "copy_ceiling": copy,
        "stream_ceilings": ceil,
        "wall_s": round(wall_s, 4),
        "launch": "python loop" if args.no_graph else "HIP graph replay",
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def copy_ceiling(torch, stream):
    """A plain device-to-device copy of 1 GiB (4x the Infinity Cache), the
    practical streaming ceiling on this GPU: (read + write bytes) / time."""
    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    reps = 20
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    z.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(z) * 1000.0 / reps
    gbs = 2 * nbytes / (us * 1e-6) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"GB/s": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
            "bytes": 2 * nbytes, "us": round(us, 1)}


def stream_ceilings(torch, rx, stream):
    """Read, write and copy rates of the library's plain 16-byte-per-lane
    streaming kernels over 1 GiB (4x the Infinity Cache), best over 1, 2, 4
    and 8 workgroups per CU with and without nontemporal hints: the HBM
    ceilings a streaming kernel reaches on this GPU. Bytes counted: read +
    written."""
    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    sink = torch.empty(rx.rxtest_stream_sink_bytes(8) // 4, dtype=torch.float32, device="cuda:0")
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for kind, name, moved in ((rx.RXTEST_READ, "read", nbytes), (rx.RXTEST_WRITE, "write", nbytes),
                              (rx.RXTEST_COPY, "copy", 2 * nbytes)):
        best = None
        for wgs in (1, 2, 4, 8):
            for nt in (False, True):
                d = sink if kind == rx.RXTEST_READ else dst
                run = lambda: rx.rxtest_stream(kind, src, d, nbytes, wgs, nt, stream)
                run(); run()
                reps = 10
                torch.cuda.synchronize()
                a.record(stream)
                for _ in range(reps):
                    run()
                z.record(stream)
                torch.cuda.synchronize()
                us = a.elapsed_time(z) * 1000.0 / reps
                gbs = moved / (us * 1e-6) / 1e9
                if best is None or gbs > best["GB/s"]:
                    best = {"GB/s": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
                            "wgs_per_cu": wgs, "nontemporal": nt}
        out[name] = best
    del src, dst, sink
    torch.cuda.empty_cache()
    return out


def launch_floors(torch, rx, in_bytes, reps=256):
    """What a plain streaming kernel costs per back-to-back launch at this
    message size, cold (graph replay, each launch on its own slice of a
    1 GiB rotation): a launch with no memory access, a read of in_bytes, and
    a copy of in_bytes (best of 1/2/4 workgroups per CU, with and without
    nontemporal hints)."""
    total = 1 << 30
    slices = total // in_bytes
    src = torch.zeros(total // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.zeros_like(src)
    sink = torch.empty(rx.rxtest_stream_sink_bytes(8) // 4, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = in_bytes // 4

    def timed(calls):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in calls:
                c()
        g.replay()
        torch.cuda.synchronize()
        a.record(stream)
        g.replay()
        z.record(stream)
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(z) * 1000.0 / len(calls)

    out = {"bytes": in_bytes}
    out["empty_us"] = round(timed([lambda: rx.rxtest_stream(rx.RXTEST_EMPTY, None, None, 0, 1)
                                   for _ in range(reps)]), 3)
    for kind, name in ((rx.RXTEST_READ, "read_us"), (rx.RXTEST_COPY, "copy_us")):
        best = None
        for wgs in (1, 2, 4):
            for nt in (False, True):
                calls = []
                for i in range(reps):
                    k = i % slices
                    s_ = src[k * per:(k + 1) * per]
                    d_ = sink if kind == rx.RXTEST_READ else dst[k * per:(k + 1) * per]
                    calls.append(lambda s_=s_, d_=d_, wgs=wgs, nt=nt:
                                 rx.rxtest_stream(kind, s_, d_, in_bytes, wgs, nt))
                us = timed(calls)
                best = us if best is None else min(best, us)
        out[name] = round(best, 3)
    del src, dst, sink
    torch.cuda.empty_cache()
    return out


def single_launch_us(torch, rx, fn, batches, stream, reps=200):
    """Median µs of one launch on its own (the GPU-side dispatch included),
    bracketed by its own HIP events. Each launch is queued behind a 512 MiB
    streaming read, so the host has enqueued the events and the launch before
    the GPU reaches them and no host-side call overhead is timed; the read
    also leaves the caches cold. Rotates over the cold batches."""
    nbytes = 512 << 20
    busy = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(0.0)
    sink = torch.empty(rx.rxtest_stream_sink_bytes(2) // 4, dtype=torch.float32, device="cuda:0")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps + 10)]
    torch.cuda.synchronize()
    for i, (a, z) in enumerate(evs):
        rx.rxtest_stream(rx.RXTEST_READ, busy, sink, nbytes, 2, True, stream)
        a.record(stream)
        fn(batches[i % len(batches)], i)
        z.record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(z) * 1000.0 for a, z in evs[10:])
    # the same pair of events with nothing between them
    for a, z in evs:
        rx.rxtest_stream(rx.RXTEST_READ, busy, sink, nbytes, 2, True, stream)
        a.record(stream)
        z.record(stream)
    torch.cuda.synchronize()
    t0 = sorted(a.elapsed_time(z) * 1000.0 for a, z in evs[10:])
    del busy, sink
    torch.cuda.empty_cache()
    return round(ts[len(ts) // 2], 3), round(t0[len(t0) // 2], 3)


def cpu_baseline(w, host, lp_fmt, lp_block, seconds, step_bytes):
    """The oracle (single-threaded plain C) running the same step on a
    bounded sample: whole steps while they fit in `seconds`, else a prefix of
    every rank buffer, scaled to GB/s with the same algorithmic bytes."""
    import numpy as np

    import oracle as O

    n = w.nsrc
    fmt = O.FMT[lp_fmt]
    dt = O.BF16 if w.dtype == 1 else O.FP32
    cnt = w.count
    sample = "full message"
    # bound the sample: at most 2^22 elements per rank buffer
    if cnt > (1 << 22):
        cnt = 1 << 22
        sample = f"first {cnt} elements of each rank buffer"
    srcs = [h[:cnt] for h in host]
    e = w.elem_bytes
    nb = -(-cnt // lp_block)
    lo, hi = O.tree_chunk(cnt, n, dt, 0)
    sbytes = (n * cnt * e + cnt * e) + 2 * n * (hi - lo) * e + n * (cnt * e + cnt + 4 * nb) + \
        n * (cnt + 4 * nb) + (cnt + 4 * nb) + cnt * e
    dsts = [np.empty(cnt, dtype=srcs[0].dtype) for _ in range(n)]
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.reduce_flat(srcs, dt)
        O.reduce_scatter_chunk_bcast(srcs, dt, reps % n, dsts)
        codes, scales = O.quant_fp8(srcs, dt, fmt, lp_block)
        O.dequant_reduce_requant(codes, scales, fmt, lp_block, O.DRR_REQUANT, dt, True)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    gbs = sbytes * reps / el / 1e9
    cpu = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} oracle step(s) over the {sample} ({sbytes} algorithmic bytes "
                      f"per step), {el:.1f} s on one host core ({cpu}, "
                      f"{os.cpu_count()} logical CPUs visible)"}


if __name__ == "__main__":
    main()
