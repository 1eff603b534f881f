#!/usr/bin/env python3
"""Benchmark of the rx hot path on one MI355X.

One step = one pass of every hot-path operation over one batch of synthetic
rank buffers (N = 8 separate HBM allocations):
  1. DDA flat local reduce              rx_reduce_flat
  2. DDA tree per-rank step             rx_reduce_scatter_chunk_bcast (rank = step % N)
  3. FP8 block quantizer                rx_quant_fp8
  4. fused dequant-reduce-requant, with the dequantized high-precision
     output                             rx_dequant_reduce_requant (REQUANT + hp)

The step workload (`value`, `ms_per_step`, `roofline`, `kernels`) is the
decode-size message the headline "µs at 512 KB" names: 8 x 32x8192 BF16
(512 KiB per rank); its low-precision leg uses E5M2 with 256-element blocks
(the BF16 message format of the large low-precision workload). Inputs are
resident in HBM before timing starts and the batches rotate over >= 2 GiB,
so every step reads its inputs from HBM rather than from the 256 MB Infinity
Cache.

`configs` then times, in the same run, the kernels each of the five message
shapes is quoted on, each with its own rotation (>= 2 GiB of inputs and
outputs, or one launch when a launch alone moves that much):
  cfg1  8 x 200 FP32 (10x20), rank-id fill (-> 28.0) and U[-1,1): flat reduce
  cfg2  8 x 262,144 BF16 (512 KiB), N(0,1): flat reduce
  cfg3  8 x 2,097,152 BF16 (4 MiB), N(0,1): tree step for every rank
  cfg4  8 x 16,777,216 FP32 (64 MiB), N(0,1) + 1% x100: quant E4M3/128,
        DRR-REQUANT with and without the FP32 output
  cfg5  8 x 268,435,456 BF16 (512 MiB), Laplace(0,1): quant E5M2/256,
        DRR-REQUANT with the fused BF16 output and without it, the separate
        dequantization
Every generated input buffer's SHA-256 is recorded beside its config.

Times: HIP events on the launch stream around back-to-back launches of one
kernel (captured in a HIP graph), divided by the launch count (`us`,
`frac`). Where the committed rocprofv3 kernel trace of the same command
(profiles/kernels_<workload>.md) holds the kernel at the current source
hash, its average per-dispatch duration is reported beside it (`us_trace`,
`frac_trace`): under the profiler each dispatch starts on an idle GPU, so at
decode size the trace durations run longer than the back-to-back interval.

Floors, timed the same way in the same run: `launch_floors` (an empty
launch, a read and a copy of the decode message's 4 MiB, on one 1 GiB
rotation) and the tree step's own memory pattern without its arithmetic
(`tree_step_pattern_floor`, and cfg3's `pattern_floor`: each rank buffer's
chunk copied into its own destination, the same 2N streams in the same
allocations and rotation). cfg3's `offset_layout` times the step and that
floor again on rank buffers spaced buffer size + 2 KiB apart in one
allocation, so the 2N chunks do not share their offset modulo 4 MiB.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD published peak
METRIC = "effective HBM GB/s (% of MI355X peak) per reduce kernel; µs at 512 KB msg"
ROTATE_BYTES = 2 << 30  # >= 8x the 256 MB Infinity Cache

# the sources each measured kernel is built and launched from (a committed
# profile's figures are used only while their hash is unchanged)
_COMMON = ["rx_device.hpp", "rx_internal.hpp", "api.hip"]
_FLAT = ["reduce.hip", "reduce_common.hpp"] + _COMMON
_TREE = ["tree.hip", "reduce_common.hpp"] + _COMMON
_QUANT = ["quant.hip"] + _COMMON
_DRR = ["drr.hpp", "drr.hip", "drr_16x1.hip", "drr_16x1s.hip", "drr_16x1w.hip", "drr_pf.hip", "drr_8x2.hip",
        "drr_4x4.hip", "drr_4x1.hip", "drr_4x1t.hip"] + _COMMON
_LP = ["allreduce_lp.hip", "quant.hip", "drr.hpp", "drr.hip"] + _COMMON
KERNEL_SOURCES = {
    "reduce_flat": _FLAT, "tree_step": _TREE, "quant_fp8": _QUANT,
    "dequant_reduce_requant": _DRR, "drr_requant": _DRR, "drr_requant_hp": _DRR,
    "lp_tree_step": _DRR, "dequant_separate": _DRR, "lp_flat_sum": _DRR,
    "allreduce_local_flat": _TREE, "allreduce_local_tree": _TREE,
    "allreduce_local_lowprec": _LP,
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode",
                   help="step workload: decode | tree | lp_fp32 | lp_bf16 | flat_uniform")
    p.add_argument("--configs", default="cfg1,cfg3,cfg4,cfg5",
                   help="comma list of the per-config measurements to run beside the "
                        "step ('' = none); cfg2 is the decode step workload")
    p.add_argument("--kernel-reps", type=int, default=0,
                   help="launches per timed measurement, everywhere (0 = auto; for profiler runs)")
    p.add_argument("--warm", action="store_true",
                   help="reuse one batch every step (cache-warm; labelled)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ceilings", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="oracle time, split between the 1-thread and the N-thread legs")
    return p.parse_args()


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def sha_of(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "allreduce_reduction_rx_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _profile_field(path, key, name, field):
    """`field` of the line '- <key>: source_sha256=<sha> ... field=<v>' of a
    committed profile summary, when its source hash is the current one."""
    if not os.path.exists(path):
        return None
    kernel = name.split("@")[0]
    want = sha_of(KERNEL_SOURCES[kernel])
    for line in open(path):
        m = re.match(r"- ([\w@.]+): source_sha256=(\w+) (.*)$", line.strip())
        if m and m.group(1) == key:
            if m.group(2) != want:
                return None
            f = dict(kv.split("=", 1) for kv in m.group(3).split())
            return float(f[field]) if field in f else None
    return None


def trace_us(workload, name):
    """Average per-dispatch µs of `name` in the committed rocprofv3 kernel
    trace of this workload, or None (absent, or the source changed)."""
    return _profile_field(os.path.join(ROOT, "profiles", f"kernels_{workload}.md"), name, name,
                          "avg_us")


def read_traffic(workload, name):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary
    (profiles/traffic_<workload>.md), or None."""
    return _profile_field(os.path.join(ROOT, "profiles", f"traffic_{workload}.md"), name, name,
                          "hbm_bytes_per_launch")


def entry(nbytes, us, reps, workload=None, name=None, target=None):
    gbs = nbytes / (us * 1e-6) / 1e9
    d = {"bytes": int(nbytes), "us": round(us, 3), "GB/s": round(gbs, 1),
         "frac": round(gbs / PEAK_HBM_GBS, 4), "launches": reps}
    if workload and name:
        tu = trace_us(workload, name)
        if tu:
            d["us_trace"] = round(tu, 3)
            d["frac_trace"] = round(nbytes / (tu * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
    if target is not None:
        d["target_frac"] = target
    return d


def sha256_buffers(bufs):
    """SHA-256 of each host buffer's bytes (one thread per buffer)."""
    with ThreadPoolExecutor(max(1, min(len(bufs), 16))) as ex:
        return list(ex.map(lambda b: hashlib.sha256(memoryview(b).cast("B")).hexdigest(), bufs))


def cpu_threads():
    # the GPU machine gives one GPU's job 16 host threads, whatever the OS shows
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class Timer:
    """Back-to-back launches captured in one HIP graph, timed with HIP events
    on the stream the graph replays on (torch's current stream, which is the
    stream the binding launches on).

    With RX_BENCH_PHASE_LOG=<path> in the environment, every timed
    measurement appends one JSON line {"phase", "t0_ns", "t1_ns"} (host
    CLOCK_MONOTONIC, the device idle at both ends), so that a profiler's
    per-dispatch records can be attributed to the measurement they belong
    to."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.current_stream()
        self.a = torch.cuda.Event(enable_timing=True)
        self.z = torch.cuda.Event(enable_timing=True)
        path = os.environ.get("RX_BENCH_PHASE_LOG")
        self.log = open(path, "a") if path else None

    def phase(self, name, run):
        """run() as the measurement `name` (logged when the log is on)."""
        if self.log is None:
            return run()
        self.torch.cuda.synchronize()
        t0 = time.clock_gettime_ns(time.CLOCK_MONOTONIC)
        out = run()
        self.torch.cuda.synchronize()
        t1 = time.clock_gettime_ns(time.CLOCK_MONOTONIC)
        self.log.write(json.dumps({"phase": name, "t0_ns": t0, "t1_ns": t1}) + "\n")
        self.log.flush()
        return out

    def capture(self, calls):
        g = self.torch.cuda.CUDAGraph()
        with self.torch.cuda.graph(g):
            for c in calls:
                c()
        return g

    def timed(self, run, reps_inner):
        """ms per inner repetition of run()."""
        torch = self.torch
        torch.cuda.synchronize()
        self.a.record(self.stream)
        run()
        self.z.record(self.stream)
        torch.cuda.synchronize()
        return self.a.elapsed_time(self.z) / reps_inner

    def us_per_launch(self, calls, name=None):
        g = self.capture(calls)

        def run():
            g.replay()
            return self.timed(g.replay, len(calls)) * 1000.0

        us = self.phase(name, run) if name else run()
        del g
        return us


REPS_OVERRIDE = 0   # --kernel-reps: launches per measurement everywhere (0 = auto)


def nreps(default):
    return REPS_OVERRIDE or default


def auto_reps(nbytes, lo=8, hi=2000):
    """Enough launches for ~50 ms of HBM traffic at 4 TB/s."""
    return nreps(max(lo, min(hi, int(0.05 / max(1e-9, nbytes / 4e12)))))


def nsets_for(bytes_per_set, torch, cap=1024):
    free, _ = torch.cuda.mem_get_info()
    n = -(-ROTATE_BYTES // max(1, bytes_per_set))
    return max(1, min(cap, n, int(0.5 * free // max(1, bytes_per_set))))


def upload(host, torch, dev):
    import numpy as np
    out = []
    for h in host:
        t = torch.from_numpy(h.view(np.int16) if h.dtype == np.uint16 else h).to(dev)
        out.append(t.view(torch.bfloat16) if h.dtype == np.uint16 else t)
    return out


# ---------------------------------------------------------------------------
# the step workload
# ---------------------------------------------------------------------------

class Batch:
    """One set of device buffers for a step."""

    def __init__(self, w, srcs_dev, lp_block, torch):
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


def step_workload(args, torch, rx, G, timer):
    import numpy as np
    dev = torch.device("cuda:0")
    wname = args.workload
    w = G.WORKLOADS[wname]
    n, count = w.nsrc, w.count
    e = w.elem_bytes
    if w.fp8:
        lp_fmt, lp_block = w.fp8, w.block
    else:
        lp_fmt, lp_block = ("e5m2", 256) if w.dtype == G.BF16 else ("e4m3", 128)
    nb = -(-count // lp_block)
    tdt = torch.bfloat16 if w.dtype == G.BF16 else torch.float32

    host = w.sources()
    hashes = sha256_buffers(host)
    base = upload(host, torch, dev)
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
    # measured beside the step, not part of it
    bytes_k["lp_tree_step"] = 2 * n * (lp_chunk + 4 * (lp_chunk // lp_block))
    bytes_k["dequant_separate"] = (count + 4 * nb) + count * e
    bytes_k["lp_flat_sum"] = n * (count + 4 * nb) + count * e
    bytes_k["allreduce_local_flat"] = 2 * n * count * e
    bytes_k["allreduce_local_tree"] = 2 * n * count * e
    # the low-precision allreduce is one pass (every buffer read and written
    # once) when a block spans at most 64 16-byte vectors, else a quantize
    # pass into the workspace and a reduce pass
    one_pass = lp_block <= (256 if w.dtype == G.FP32 else 512)
    bytes_k["allreduce_local_lowprec"] = (2 * n * count * e if one_pass else
                                          n * (count * e + count + 4 * nb)
                                          + n * (count + 4 * nb) + n * count * e)
    per_batch_bytes = (n * count * e + count * e + n * count * e + n * (count + 4 * nb)
                       + count + 4 * nb + count * e + n * (count + 4 * nb))
    nsets = 1 if args.warm else nsets_for(per_batch_bytes, torch, cap=256)
    batches = [Batch(w, base, lp_block, torch)]
    for _ in range(nsets - 1):
        batches.append(Batch(w, [b.clone() for b in base], lp_block, torch))
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
    # depend on the values); one workspace per set, sets rotating over
    # >= 2 GiB like the batches
    ws_bytes = rx.rx_allreduce_local_workspace(n, count, lp_block)
    ar_set_bytes = n * count * e + ws_bytes
    n_ar = 1 if args.warm else nsets_for(ar_set_bytes, torch)
    ar_bufs = [[torch.zeros(count, dtype=tdt, device=dev) for _ in range(n)] for _ in range(n_ar)]
    ar_ws = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(n_ar)]

    def k_ar_flat(b, i):
        rx.rx_allreduce_local(ar_bufs[i % n_ar], rx.RX_ALGO_FLAT, lp_fmt, lp_block)

    def k_ar_tree(b, i):
        rx.rx_allreduce_local(ar_bufs[i % n_ar], rx.RX_ALGO_TREE, lp_fmt, lp_block)

    def k_ar_lp(b, i):
        rx.rx_allreduce_local(ar_bufs[i % n_ar], rx.RX_ALGO_LOWPREC, lp_fmt, lp_block,
                              ar_ws[i % n_ar])

    kernels_timed = kernels + [("lp_tree_step", k_lp_tree), ("dequant_separate", k_dequant),
                               ("lp_flat_sum", k_lp_flat), ("allreduce_local_flat", k_ar_flat),
                               ("allreduce_local_tree", k_ar_tree),
                               ("allreduce_local_lowprec", k_ar_lp)]

    # ---- whole-step timing: W untimed steps, then exactly K timed steps ----
    g_warm = timer.capture([lambda i=i: step(i) for i in range(max(1, args.warmup))])
    g_steps = timer.capture([lambda i=i: step(i) for i in range(args.steps)])
    if args.warmup:
        g_warm.replay()
    t_wall = time.perf_counter()
    step_ms = timer.phase(f"{wname}/step", lambda: timer.timed(g_steps.replay, args.steps))
    wall_s = time.perf_counter() - t_wall
    del g_warm, g_steps

    # ---- per-kernel timing: back-to-back launches of one kernel ----
    per_kernel = {}
    for name, fn in kernels_timed:
        reps = auto_reps(bytes_k[name], lo=50)
        us = timer.us_per_launch([lambda i=i: fn(batches[i % nsets], i) for i in range(reps)],
                                 f"{wname}/{name}")
        per_kernel[name] = entry(bytes_k[name], us, reps, wname, name)

    # ---- the tree step for each rank on its own ----
    by_rank = []
    for k in range(n):
        reps = per_kernel["tree_step"]["launches"]
        by_rank.append(round(timer.us_per_launch(
            [lambda i=i, k=k: rx.rx_reduce_scatter_chunk_bcast(batches[i % nsets].srcs, k,
                                                               batches[i % nsets].tree_dsts)
             for i in range(reps)], f"{wname}/tree_step@rank{k}"), 3))

    # ---- the tree step's memory pattern without its arithmetic ----
    chunks = [rx.rx_tree_chunk(count, n, w.dtype, k) for k in range(n)]
    tree_floor = tree_pattern_floor(rx, timer, lambda i: batches[i % nsets].srcs,
                                    lambda i: batches[i % nsets].tree_dsts, chunks, e,
                                    per_kernel["tree_step"]["launches"], wname)

    # ---- the flat reduce over the first k rank buffers, k = 1..N ----
    flat_by_nsrc = []
    for k in range(1, n + 1):
        reps = per_kernel["reduce_flat"]["launches"]
        flat_by_nsrc.append(round(timer.us_per_launch(
            [lambda i=i, k=k: rx.rx_reduce_flat(batches[i % nsets].srcs[:k],
                                                batches[i % nsets].flat_out)
             for i in range(reps)], f"{wname}/reduce_flat@nsrc{k}"), 3))

    # ---- invariant spot check of batch 0: the tree chunk equals the flat
    # result on that chunk ----
    b0 = batches[0]
    rx.rx_reduce_flat(b0.srcs, b0.flat_out)
    rx.rx_reduce_scatter_chunk_bcast(b0.srcs, 0, b0.tree_dsts)
    torch.cuda.synchronize()
    lo, hi = rx.rx_tree_chunk(count, n, w.dtype, 0)
    iv = torch.int16 if tdt == torch.bfloat16 else torch.int32
    tree_ok = all(torch.equal(d[lo:hi].view(iv), b0.flat_out[lo:hi].view(iv)) for d in b0.tree_dsts)

    us_single, us_events = single_launch_us(torch, rx, k_flat, batches, timer.stream)

    out = {
        "w": w, "host": host, "hashes": hashes, "lp_fmt": lp_fmt, "lp_block": lp_block,
        "step_ms": step_ms, "wall_s": wall_s, "step_bytes": step_bytes, "chunk": chunk,
        "nsets": nsets, "per_batch_bytes": per_batch_bytes, "per_kernel": per_kernel,
        "by_rank": by_rank, "flat_by_nsrc": flat_by_nsrc, "tree_ok": tree_ok,
        "us_single": us_single, "us_events": us_events, "kernels": [k for k, _ in kernels],
        "n_ar_sets": n_ar, "ar_set_bytes": ar_set_bytes, "tree_floor": tree_floor,
    }
    del batches, ar_bufs, ar_ws, base
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# the five message shapes
# ---------------------------------------------------------------------------

def describe(w):
    e_name = "BF16" if w.dtype == 1 else "FP32"
    s = f"{w.nsrc} x {w.count:,} {e_name} ({w.count * w.elem_bytes / 1024:.0f} KiB per rank), seed {w.seed}"
    if w.fp8:
        s += f", {w.fp8.upper()} blocks of {w.block}"
    return s


def cfg_flat_small(wname, torch, rx, G, timer):
    """cfg1: the pages' rank-id example and its U[-1,1) companion."""
    import numpy as np
    dev = torch.device("cuda:0")
    w = G.WORKLOADS[wname]
    host = w.sources()
    srcs = upload(host, torch, dev)
    dst = torch.empty(w.count, dtype=torch.float32, device=dev)
    nbytes = (w.nsrc + 1) * w.count * w.elem_bytes
    reps = nreps(2000)
    us = timer.us_per_launch([lambda: rx.rx_reduce_flat(srcs, dst)] * reps, f"{wname}/reduce_flat")
    rx.rx_reduce_flat(srcs, dst)
    torch.cuda.synchronize()
    d = {"workload": describe(w), "input_sha256": sha256_buffers(host),
         "cache": "warm (7.2 KB; every launch reads the same buffers)",
         "kernels": {"reduce_flat": entry(nbytes, us, reps, None, None)}}
    if wname == "flat_rank":
        d["check"] = "28.0 everywhere" if bool((dst == 28.0).all()) else "MISMATCH"
    return d


def cfg_tree(torch, rx, G, timer):
    """cfg3: the tree step on 8 x 4 MiB BF16, every rank, rotating sets."""
    dev = torch.device("cuda:0")
    w = G.WORKLOADS["tree"]
    n, count, e = w.nsrc, w.count, w.elem_bytes
    host = w.sources()
    hashes = sha256_buffers(host)
    base = upload(host, torch, dev)
    set_bytes = 2 * n * count * e
    nsets = nsets_for(set_bytes, torch)
    sets = [(base, [torch.empty_like(base[0]) for _ in range(n)])]
    for _ in range(nsets - 1):
        sets.append(([b.clone() for b in base], [torch.empty_like(base[0]) for _ in range(n)]))
    lo, hi = rx.rx_tree_chunk(count, n, w.dtype, 0)
    nbytes = 2 * n * (hi - lo) * e
    reps = nreps(1000)
    by_rank = []
    for k in range(n):
        by_rank.append(timer.us_per_launch(
            [lambda i=i, k=k: rx.rx_reduce_scatter_chunk_bcast(sets[i % nsets][0], k,
                                                               sets[i % nsets][1])
             for i in range(reps)], f"tree/tree_step@rank{k}"))
    med = sorted(by_rank)[n // 2]
    tree = entry(nbytes, med, reps, "tree", "tree_step", target=0.4)
    tree["us_by_rank"] = [round(x, 3) for x in by_rank]
    tree["statistic"] = "median over the 8 ranks"
    chunks = [rx.rx_tree_chunk(count, n, w.dtype, k) for k in range(n)]
    tree["pattern_floor"] = tree_pattern_floor(rx, timer, lambda i: sets[i % nsets][0],
                                               lambda i: sets[i % nsets][1], chunks, e, reps, "tree")
    tree["frac_of_pattern_floor"] = round(tree["pattern_floor"]["us"] / med, 4)
    tree["offset_layout"] = tree_offset_layout(torch, rx, timer, base, nsets, chunks, e, reps)
    fbytes = (n + 1) * count * e
    freps = auto_reps(fbytes, lo=100)
    flat_out = [torch.empty_like(base[0]) for _ in range(nsets)]
    us = timer.us_per_launch([lambda i=i: rx.rx_reduce_flat(sets[i % nsets][0], flat_out[i % nsets])
                              for i in range(freps)], "tree/reduce_flat")
    out = {"workload": describe(w) + f", chunk {hi - lo:,}", "input_sha256": hashes,
           "cache": f"cold (rotating {nsets} sets, {nsets * set_bytes / 2**30:.2f} GiB)",
           "kernels": {"tree_step": tree,
                       "reduce_flat": entry(fbytes, us, freps, "tree", "reduce_flat")}}
    del sets, base, flat_out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def cfg_lp(wname, torch, rx, G, timer, ceilings):
    """cfg4 / cfg5: quantizer, DRR-REQUANT with and without the
    high-precision output, separate dequantization, each rotating over
    >= 2 GiB (or one launch where a launch moves that much)."""
    dev = torch.device("cuda:0")
    w = G.WORKLOADS[wname]
    n, count, e, fmt, block = w.nsrc, w.count, w.elem_bytes, w.fp8, w.block
    nb = -(-count // block)
    tdt = torch.bfloat16 if w.dtype == G.BF16 else torch.float32
    t0 = time.perf_counter()
    host = w.sources()
    hashes = sha256_buffers(host)
    base = upload(host, torch, dev)
    del host
    gen_s = time.perf_counter() - t0
    kern = {}

    def codes_like():
        return ([torch.empty(count, dtype=torch.uint8, device=dev) for _ in range(n)],
                [torch.empty(nb, dtype=torch.float32, device=dev) for _ in range(n)])

    # quantizer: sources + codes + scales per set
    q_bytes = n * (count * e + count + 4 * nb)
    nq = nsets_for(q_bytes, torch)
    qsets = [(base,) + codes_like()]
    for _ in range(nq - 1):
        qsets.append(([b.clone() for b in base],) + codes_like())
    reps = auto_reps(q_bytes)
    us = timer.us_per_launch([lambda i=i: rx.rx_quant_fp8(qsets[i % nq][0], fmt, block,
                                                          qsets[i % nq][1], qsets[i % nq][2])
                              for i in range(reps)], f"{wname}/quant_fp8")
    kern["quant_fp8"] = entry(q_bytes, us, reps, wname, "quant_fp8", target=0.8)
    # flat reduce of the same message (the full-precision leg)
    f_bytes = (n + 1) * count * e
    flat_out = [torch.empty(count, dtype=tdt, device=dev) for _ in range(nq)]
    reps = auto_reps(f_bytes)
    us = timer.us_per_launch([lambda i=i: rx.rx_reduce_flat(qsets[i % nq][0], flat_out[i % nq])
                              for i in range(reps)], f"{wname}/reduce_flat")
    kern["reduce_flat"] = entry(f_bytes, us, reps, wname, "reduce_flat", target=0.8)
    rx.rx_quant_fp8(base, fmt, block, qsets[0][1], qsets[0][2])
    codes0, scales0 = qsets[0][1], qsets[0][2]
    del flat_out
    for s in qsets[1:]:
        del s
    qsets = None
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # DRR: codes + scales in, requantized codes + scales (+ hp) out
    in_bytes = n * (count + 4 * nb)
    out_q = count + 4 * nb
    d_set = in_bytes + out_q + count * e
    nd = nsets_for(d_set, torch)
    dsets = []
    for j in range(nd):
        c = codes0 if j == 0 else [x.clone() for x in codes0]
        s = scales0 if j == 0 else [x.clone() for x in scales0]
        dsets.append((c, s, torch.empty(count, dtype=torch.uint8, device=dev),
                      torch.empty(nb, dtype=torch.float32, device=dev),
                      torch.empty(count, dtype=tdt, device=dev)))
    hp_name = "drr_requant_bf16_out" if tdt == torch.bfloat16 else "drr_requant_fp32_out"
    for name, with_hp in (("drr_requant", False), (hp_name, True)):
        nbytes = in_bytes + out_q + (count * e if with_hp else 0)
        reps = auto_reps(nbytes)
        us = timer.us_per_launch(
            [lambda i=i, h=with_hp: rx.rx_dequant_reduce_requant(
                dsets[i % nd][0], dsets[i % nd][1], fmt, block, rx.RX_DRR_REQUANT,
                dsets[i % nd][2], dsets[i % nd][3], dsets[i % nd][4] if h else None)
             for i in range(reps)], f"{wname}/" + ("drr_requant_hp" if with_hp else "drr_requant"))
        kern[name] = entry(nbytes, us, reps, wname,
                           "drr_requant_hp" if with_hp else "drr_requant", target=0.8)
    # separate dequantization of the requantized message (N = 1, SUM), with
    # its own rotation: requantized codes + scales in, the message dtype out
    rx.rx_dequant_reduce_requant(codes0, scales0, fmt, block, rx.RX_DRR_REQUANT,
                                 dsets[0][2], dsets[0][3])
    dq_bytes = out_q + count * e
    nq2 = nsets_for(dq_bytes, torch)
    qsets2 = [(dsets[0][2], dsets[0][3], dsets[0][4])]
    for _ in range(nq2 - 1):
        qsets2.append((dsets[0][2].clone(), dsets[0][3].clone(),
                       torch.empty(count, dtype=tdt, device=dev)))
    reps = auto_reps(dq_bytes)
    us = timer.us_per_launch([lambda i=i: rx.rx_dequant_reduce_requant(
        [qsets2[i % nq2][0]], [qsets2[i % nq2][1]], fmt, block, rx.RX_DRR_SUM,
        out_hp=qsets2[i % nq2][2]) for i in range(reps)], f"{wname}/dequant_separate")
    kern["dequant_separate"] = entry(dq_bytes, us, reps, wname, "dequant_separate", target=0.8)

    del qsets2
    dsets = None
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    # the whole one-device low-precision allreduce, in place (one pass: every
    # buffer read once and written once), on buffers of zeros so repeated
    # in-place sums stay finite; no workspace (the one-pass form needs none)
    ar_bytes = 2 * n * count * e
    na = nsets_for(n * count * e, torch)
    ar = [[torch.zeros(count, dtype=tdt, device=dev) for _ in range(n)] for _ in range(na)]
    reps = auto_reps(ar_bytes)
    us = timer.us_per_launch([lambda i=i: rx.rx_allreduce_local_noalloc(
        ar[i % na], rx.RX_ALGO_LOWPREC, fmt, block) for i in range(reps)],
        f"{wname}/allreduce_local_lowprec")
    kern["allreduce_local_lowprec"] = entry(ar_bytes, us, reps, wname, "allreduce_local_lowprec",
                                            target=0.8)
    del ar

    if ceilings:
        ratio_kind = {
            "quant_fp8": ("narrow4" if e == 4 else "narrow2"),
            "reduce_flat": f"reduce{n}",
            "drr_requant": f"reduce{n}",
            hp_name: f"reduce{max(1, round(in_bytes / (out_q + count * e)))}",
            "dequant_separate": "copy",
            "allreduce_local_lowprec": "copy",
        }
        for name, kind in ratio_kind.items():
            c = ceilings.get(kind)
            if c:
                kern[name]["mixed_ceiling"] = kind
                kern[name]["frac_of_mixed_ceiling"] = round(kern[name]["GB/s"] / c["GB/s"], 4)
    out = {"workload": describe(w), "input_sha256": hashes,
           "cache": f"cold (quant rotates {nq} set(s) of {q_bytes / 2**30:.2f} GiB, DRR {nd} of "
                    f"{d_set / 2**30:.2f} GiB, dequant {nq2} of {dq_bytes / 2**30:.2f} GiB, "
                    f"allreduce {na} of {n * count * e / 2**30:.2f} GiB)",
           "generate_upload_s": round(gen_s, 1), "kernels": kern}
    del base, codes0, scales0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# ceilings and floors
# ---------------------------------------------------------------------------

def stream_ceilings(torch, rx, timer):
    """Read, write and copy rates of the library's plain 16-byte-per-lane
    streaming kernels over 1 GiB, and the mixed read/write ceilings (the
    hot-path kernels' access patterns with XOR in place of their arithmetic:
    reduce N:1 over N sources, 2:1 and 4:1 narrowing), best over 1, 2, 4
    and 8 workgroups per CU with and without nontemporal hints (the mixed ones
    also with and without the next-tile prefetch). Bytes counted: read +
    written."""
    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    sink = torch.empty(rx.rxtest_stream_sink_bytes(8) // 4, dtype=torch.float32, device="cuda:0")
    out = {}

    def best(kind, run_for, moved, reps=None, pfs=(None,)):
        reps = nreps(6) if reps is None else reps
        b = None
        for wgs in (1, 2, 4, 8):
            for nt in (False, True):
                for pf in pfs:
                    tag = f"ceiling/{kind}@wgs{wgs}nt{int(nt)}" + ("" if pf is None else f"pf{int(pf)}")
                    call = (lambda wgs=wgs, nt=nt: run_for(wgs, nt)) if pf is None else \
                        (lambda wgs=wgs, nt=nt, pf=pf: run_for(wgs, nt, pf))
                    us = timer.us_per_launch([call] * reps, tag)
                    gbs = moved / (us * 1e-6) / 1e9
                    if b is None or gbs > b["GB/s"]:
                        b = {"GB/s": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
                             "wgs_per_cu": wgs, "nontemporal": nt}
                        if pf is not None:
                            b["prefetch"] = pf
        return b

    out["read"] = best("read", lambda wgs, nt: rx.rxtest_stream(rx.RXTEST_READ, src, sink, nbytes, wgs, nt),
                       nbytes)
    out["write"] = best("write", lambda wgs, nt: rx.rxtest_stream(rx.RXTEST_WRITE, None, dst, nbytes, wgs, nt),
                        nbytes)
    out["copy"] = best("copy", lambda wgs, nt: rx.rxtest_stream(rx.RXTEST_COPY, src, dst, nbytes, wgs, nt),
                       2 * nbytes)
    if not hasattr(rx, "rxtest_stream_mixed"):
        del src, dst, sink
        torch.cuda.empty_cache()
        return out
    # mixed: 1 GiB read in total
    for k in (8, 3, 2):
        per = nbytes // k // 16 * 16
        srcs = [src.view(torch.uint8)[j * per:(j + 1) * per] for j in range(k)]
        out[f"reduce{k}"] = best(f"reduce{k}", lambda wgs, nt, pf, srcs=srcs, per=per: rx.rxtest_stream_mixed(
            rx.RXTEST_MIXED_REDUCE, srcs, dst.view(torch.uint8)[:per], per, wgs, nt, pf),
            (k + 1) * per, pfs=(False, True))
    for kind, k in ((rx.RXTEST_MIXED_NARROW2, 2), (rx.RXTEST_MIXED_NARROW4, 4)):
        out[f"narrow{k}"] = best(f"narrow{k}", lambda wgs, nt, pf, kind=kind, k=k: rx.rxtest_stream_mixed(
            kind, [src], dst.view(torch.uint8)[:nbytes // k], nbytes, wgs, nt, pf),
            nbytes + nbytes // k, pfs=(False, True))
    del src, dst, sink
    torch.cuda.empty_cache()
    return out


def tree_offset_layout(torch, rx, timer, base, nsets, chunks, e, reps):
    """The tree step and its pattern floor on rank buffers carved from one
    allocation at a stride of buffer size + 2 KiB. Separate allocations of a
    power-of-two size sit at one offset modulo that size, so chunk k of all
    2N buffers shares its low address bits; here each buffer starts 2 KiB
    further along. The ranks of a node hold their buffers in their own GPUs'
    memories, so the aliasing of the one-device layout has no counterpart
    there; this entry shows what the step costs without it."""
    n = len(base)
    nbytes = base[0].numel() * e
    stride = nbytes + 2048
    big = torch.empty(nsets * 2 * n * stride, dtype=torch.uint8, device=base[0].device)

    def view(i, j):
        o = (i * 2 * n + j) * stride
        return big[o:o + nbytes].view(base[0].dtype)

    sets = [([view(i, j) for j in range(n)], [view(i, n + j) for j in range(n)]) for i in range(nsets)]
    for srcs, _ in sets:
        for s, b in zip(srcs, base):
            s.copy_(b)
    by_rank = []
    for k in range(n):
        by_rank.append(timer.us_per_launch(
            [lambda i=i, k=k: rx.rx_reduce_scatter_chunk_bcast(sets[i % nsets][0], k, sets[i % nsets][1])
             for i in range(reps)], f"tree/tree_step_offset@rank{k}"))
    floor = tree_pattern_floor(rx, timer, lambda i: sets[i % nsets][0], lambda i: sets[i % nsets][1],
                               chunks, e, reps, "tree_offset")
    out = {"stride_bytes": stride, "us": round(sorted(by_rank)[n // 2], 3),
           "us_by_rank": [round(x, 3) for x in by_rank], "pattern_floor": floor}
    del sets, big
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def tree_pattern_floor(rx, timer, srcs_of, dsts_of, chunks, e, reps, tag):
    """The tree step's memory pattern without its arithmetic: each rank
    buffer's chunk copied into its own destination buffer (the same 2N
    streams in the same allocations and rotation as the tree step, the chunk
    following the rank as in the tree step's timing); best of one or two
    lanes per 16-byte vector in 64- or 128-thread workgroups. The floor the
    tree step's memory pattern sets, measured beside it."""
    n = len(chunks)
    best = None
    for lanes, wg in ((1, 64), (1, 128), (2, 64), (2, 128)):
        us = timer.us_per_launch(
            [lambda i=i, lanes=lanes, wg=wg: rx.rxtest_copy_streams(
                srcs_of(i), dsts_of(i), chunks[i % n][0] * e,
                (chunks[i % n][1] - chunks[i % n][0]) * e, lanes, wg) for i in range(reps)],
            f"floor/tree_streams@{tag}_lanes{lanes}wg{wg}")
        if best is None or us < best[0]:
            best = (us, lanes, wg)
    return {"us": round(best[0], 3), "lanes": best[1], "wg": best[2]}


def launch_floors(torch, rx, timer, in_bytes, reps=None):
    """What a plain streaming kernel costs per back-to-back launch at this
    message size, cold (graph replay, each launch on its own slice of a
    1 GiB rotation): a launch with no memory access, a read of in_bytes, and
    a copy of in_bytes (best of 1/2/4 workgroups per CU, with and without
    nontemporal hints)."""
    reps = nreps(256) if reps is None else reps
    total = 1 << 30
    slices = total // in_bytes
    src = torch.zeros(total // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.zeros_like(src)
    sink = torch.empty(rx.rxtest_stream_sink_bytes(8) // 4, dtype=torch.float32, device="cuda:0")
    per = in_bytes // 4
    out = {"bytes": in_bytes}
    out["empty_us"] = round(timer.us_per_launch(
        [lambda: rx.rxtest_stream(rx.RXTEST_EMPTY, None, None, 0, 1)] * reps, "floor/empty"), 3)
    for kind, name in ((rx.RXTEST_READ, "read_us"), (rx.RXTEST_COPY, "copy_us")):
        b = None
        for wgs in (1, 2, 4):
            for nt in (False, True):
                calls = []
                for i in range(reps):
                    k = i % slices
                    s_ = src[k * per:(k + 1) * per]
                    d_ = sink if kind == rx.RXTEST_READ else dst[k * per:(k + 1) * per]
                    calls.append(lambda s_=s_, d_=d_, wgs=wgs, nt=nt:
                                 rx.rxtest_stream(kind, s_, d_, in_bytes, wgs, nt))
                us = timer.us_per_launch(calls, f"floor/{name[:-3]}@wgs{wgs}nt{int(nt)}")
                b = us if b is None else min(b, us)
        out[name] = round(b, 3)
    del src, dst, sink
    torch.cuda.empty_cache()
    return out


def single_launch_us(torch, rx, fn, batches, stream, reps=None):
    """Median µs of one launch on its own (the GPU-side dispatch included),
    bracketed by its own HIP events. Each launch is queued behind a 512 MiB
    streaming read, so the host has enqueued the events and the launch before
    the GPU reaches them and no host-side call overhead is timed; the read
    also leaves the caches cold. Rotates over the cold batches."""
    reps = nreps(200) if reps is None else reps
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
    for a, z in evs:
        rx.rxtest_stream(rx.RXTEST_READ, busy, sink, nbytes, 2, True, stream)
        a.record(stream)
        z.record(stream)
    torch.cuda.synchronize()
    t0 = sorted(a.elapsed_time(z) * 1000.0 for a, z in evs[10:])
    del busy, sink
    torch.cuda.empty_cache()
    return round(ts[len(ts) // 2], 3), round(t0[len(t0) // 2], 3)


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, timed on the host cores
# ---------------------------------------------------------------------------

def cpu_baseline(w, host, lp_fmt, lp_block, seconds, step_bytes):
    """The oracle (plain C) running the same step on the same inputs: one
    host thread, then `cpu_threads()` threads over windows of whole blocks
    (the tree step, a single call, runs beside them). The oracle is
    elementwise and block-local, so the windowed run computes the same bits;
    that is checked on one step."""
    import numpy as np

    import oracle as O

    n = w.nsrc
    fmt = O.FMT[lp_fmt]
    dt = O.BF16 if w.dtype == 1 else O.FP32
    cnt = w.count
    sample = "full message"
    if cnt > (1 << 22):   # bound the sample
        cnt = 1 << 22
        sample = f"first {cnt:,} elements of each rank buffer"
    srcs = [np.ascontiguousarray(h[:cnt]) for h in host]
    e = w.elem_bytes
    nb = -(-cnt // lp_block)
    lo, hi = O.tree_chunk(cnt, n, dt, 0)
    sbytes = (n * cnt * e + cnt * e) + 2 * n * (hi - lo) * e + n * (cnt * e + cnt + 4 * nb) + \
        n * (cnt + 4 * nb) + (cnt + 4 * nb) + cnt * e

    def one_thread(i):
        dsts = [np.zeros(cnt, dtype=srcs[0].dtype) for _ in range(n)]
        flat = O.reduce_flat(srcs, dt)
        O.reduce_scatter_chunk_bcast(srcs, dt, i % n, dsts)
        codes, scales = O.quant_fp8(srcs, dt, fmt, lp_block)
        r = O.dequant_reduce_requant(codes, scales, fmt, lp_block, O.DRR_REQUANT, dt, True)
        return flat, dsts, codes, scales, r

    threads = cpu_threads()
    unit = lp_block * 8
    win = -(-(-(-cnt // threads)) // unit) * unit
    wins = [(a, min(a + win, cnt)) for a in range(0, cnt, win)]
    pool = ThreadPoolExecutor(threads)

    def many_threads(i):
        dsts = [np.zeros(cnt, dtype=srcs[0].dtype) for _ in range(n)]
        flat = np.empty(cnt, dtype=srcs[0].dtype)
        codes = [np.empty(cnt, np.uint8) for _ in range(n)]
        scales = [np.empty(nb, np.float32) for _ in range(n)]
        oc, osc = np.empty(cnt, np.uint8), np.empty(nb, np.float32)
        ohp = np.empty(cnt, dtype=srcs[0].dtype)
        tree = pool.submit(O.reduce_scatter_chunk_bcast, srcs, dt, i % n, dsts)

        def stage1(ab):
            a, b = ab
            x = [s[a:b] for s in srcs]
            flat[a:b] = O.reduce_flat(x, dt)
            c, s = O.quant_fp8(x, dt, fmt, lp_block)
            for j in range(n):
                codes[j][a:b] = c[j]
                scales[j][a // lp_block:-(-b // lp_block)] = s[j]
            r = O.dequant_reduce_requant(c, s, fmt, lp_block, O.DRR_REQUANT, dt, True)
            oc[a:b], osc[a // lp_block:-(-b // lp_block)], ohp[a:b] = r

        list(pool.map(stage1, wins))
        tree.result()
        return flat, dsts, codes, scales, (oc, osc, ohp)

    def run(fn, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn(reps)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return reps, el

    a = one_thread(3)
    b = many_threads(3)
    same = (np.array_equal(a[0], b[0]) and all(np.array_equal(x, y) for x, y in zip(a[1], b[1]))
            and all(np.array_equal(x, y) for x, y in zip(a[2], b[2]))
            and all(np.array_equal(x.view(np.uint32), y.view(np.uint32)) for x, y in zip(a[3], b[3]))
            and all(np.array_equal(x.view(np.uint8), y.view(np.uint8)) for x, y in zip(a[4], b[4])))
    r1, e1 = run(one_thread, seconds / 2)
    rn, en = run(many_threads, seconds / 2)
    pool.shutdown()
    cpu = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    g1, gn = sbytes * r1 / e1 / 1e9, sbytes * rn / en / 1e9
    return {"value": round(gn, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the step over the {sample} ({sbytes:,} algorithmic bytes per step): "
                      f"{rn} step(s) in {en:.1f} s on {threads} host threads, windows of whole "
                      f"blocks; {cpu}, {os.cpu_count()} logical CPUs visible",
            "one_thread": {"value": round(g1, 3), "unit": "GB/s", "cores": 1,
                           "sample": f"{r1} step(s) in {e1:.1f} s"},
            "threads_bit_identical_to_one": bool(same)}


# ---------------------------------------------------------------------------

def main():
    global REPS_OVERRIDE
    args = parse()
    REPS_OVERRIDE = args.kernel_reps
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only (got --gpus {args.gpus}); "
              "the multi-GPU collective is out of scope here", file=sys.stderr)
        sys.exit(2)

    import torch

    import allreduce_reduction_rx_amd as rx
    import rxgen as G

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    rx.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    timer = Timer(torch)

    def progress(msg):
        print(f"bench: {msg}", file=sys.stderr, flush=True)

    progress(f"step workload {args.workload}")
    s = step_workload(args, torch, rx, G, timer)
    w, n, count = s["w"], s["w"].nsrc, s["w"].count
    e = w.elem_bytes
    pk = s["per_kernel"]

    ceil = None
    if not args.no_ceilings:
        progress("ceilings")
        ceil = stream_ceilings(torch, rx, timer)
        for k in pk.values():
            k["frac_of_copy_ceiling"] = round(k["GB/s"] / ceil["copy"]["GB/s"], 4)
    floors = None
    if n * count * e <= (64 << 20):
        progress("launch floors")
        floors = launch_floors(torch, rx, timer, n * count * e)

    configs = {}
    want = [c for c in args.configs.split(",") if c]
    if args.workload == "decode":
        configs["cfg2"] = {"workload": describe(w), "input_sha256": s["hashes"],
                           "cache": f"cold (rotating {s['nsets']} batches)",
                           "kernels": {"reduce_flat": dict(pk["reduce_flat"], target_frac=0.4)}}
    if "cfg1" in want:
        progress("cfg1")
        configs["cfg1"] = cfg_flat_small("flat_rank", torch, rx, G, timer)
        configs["cfg1_uniform"] = cfg_flat_small("flat_uniform", torch, rx, G, timer)
    if "cfg3" in want:
        progress("cfg3")
        configs["cfg3"] = cfg_tree(torch, rx, G, timer)
    if "cfg4" in want:
        progress("cfg4")
        configs["cfg4"] = cfg_lp("lp_fp32", torch, rx, G, timer, ceil)
    if "cfg5" in want:
        progress("cfg5")
        configs["cfg5"] = cfg_lp("lp_bf16", torch, rx, G, timer, ceil)

    cpu = None
    if not args.no_cpu_baseline:
        progress("cpu baseline")
        cpu = cpu_baseline(w, s["host"], s["lp_fmt"], s["lp_block"], args.cpu_seconds,
                           s["step_bytes"])

    dominant = max(s["kernels"], key=lambda k: pk[k]["us"])
    dk = pk[dominant]
    value = s["step_bytes"] / (s["step_ms"] * 1e-3) / 1e9
    e_name = "BF16" if w.dtype == G.BF16 else "FP32"
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(s["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": e_name.lower(),
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {n} x {count} {e_name} rank buffers "
                        f"({count * e / 1024:.0f} KiB each), step = flat reduce + tree step "
                        f"(chunk {s['chunk']}) + FP8 quant ({s['lp_fmt']}, block {s['lp_block']}) + "
                        f"dequant-reduce-requant with {e_name} output",
            "nsrc": n, "count": count, "io_dtype": e_name.lower(), "accumulate": "f32",
            "fp8": s["lp_fmt"], "block": s["lp_block"],
            "cache": "warm (one batch reused)" if args.warm else
                     f"cold (rotating {s['nsets']} batches, "
                     f"{s['nsets'] * s['per_batch_bytes'] / 2**30:.2f} GiB; local allreduce rows "
                     f"{s['n_ar_sets']} sets, {s['n_ar_sets'] * s['ar_set_bytes'] / 2**30:.2f} GiB)",
            "step_bytes": s["step_bytes"],
        },
        "roofline": {
            "bound": "hbm", "kernel": dominant,
            "achieved": dk["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": dk["frac"],
            "frac_event": dk["frac"], "us_event": dk["us"],
            "frac_trace": dk.get("frac_trace"), "us_trace": dk.get("us_trace"),
            "traffic": read_traffic(args.workload, dominant),
        },
        "us_at_512KB": ({"event": pk["reduce_flat"]["us"],
                         "trace": pk["reduce_flat"].get("us_trace")}
                        if args.workload == "decode" else None),
        "configs": configs,
        "kernels": pk,
        "reduce_flat_us_by_nsrc": s["flat_by_nsrc"],
        "tree_step_by_rank_us": s["by_rank"],
        "tree_step_pattern_floor": s["tree_floor"],
        "us_reduce_flat_single_launch": s["us_single"],
        "us_event_pair_alone": s["us_events"],
        "launch_floors": floors,
        "tree_matches_flat": bool(s["tree_ok"]),
        "stream_ceilings": ceil,
        "input_sha256": s["hashes"],
        "wall_s": round(s["wall_s"], 4),
        "launch": "HIP graph replay",
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
