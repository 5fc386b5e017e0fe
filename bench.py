"""Benchmark: exact per-row top-K on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N]

A step is one launch of the whole selection path (row resolve, block64 sample,
histogram, crossing bin, compaction, refine / rescue, index writes) over one
batch.  The headline batch is the largest single-GPU workload, the prefill
packed causal tile: 4096 rows from 4 requests, row stride 16640 fp32, causal
window lengths 1..16384 starting at every ks % 4, K = 1024.  The same JSON
line carries the other workloads (decode 4 x 4096 K=512, decode varlen
64 x 131072 K=2048, long skewed decode BS 1 and 8, tie-heavy 8 x 262144
K=2048) and the per-row-kind tail of the tie-heavy batch.

Timing, per workload:
  * Inputs are resident in HBM.  Copies of the batch rotate so that between two
    reads of one copy at least 1 GiB of other scores is read (counting only the
    bytes the launches read, whatever --steps is), and a 1 GiB fill kernel runs
    right before the timed region: no timed launch finds its scores in the
    256 MB Infinity Cache or the L2s.
  * Timed region: K launches captured once as a HIP graph and replayed between
    torch.cuda.synchronize() calls and one pair of HIP events on the launch
    stream; region / K is the per-launch time `value`, ms_per_step and the
    roofline use.
  * Latency: at least 200 launches, each after its own 1 GiB fill and between
    its own event pair (cold), give p50 / p99; the same without the fill give
    the warm figures, and a replay of a graph on one copy the warm mean.

Prints ONE JSON line.  The CPU baseline is the test oracle (plain full sort per
row) on all host cores and on one core, over whole batches of the headline
workload for a bounded time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "top-K rows/s + achieved HBM GB/s vs peak; p50/p99 µs/row, K=512..2048"
PEAK_HBM_GBS = 8000.0  # MI355X published HBM3E bandwidth
ROTATE_BYTES = 1 << 30  # scores read between two reads of one copy
FLUSH_BYTES = 1 << 30   # fill before each cold sample and before the timed region
MIN_LATENCY_SAMPLES = 200
# GPU sleep queued ahead of a timed region's start event (about 1 ms): long
# enough for the host to submit the region's launches behind it
SUBMIT_SLEEP_CYCLES = int(3e6)
HEADLINE = 3
EXTRA = ((1, {}), (2, {}), (4, {"bs": 1}), (4, {"bs": 8}), (5, {}))
TAIL_RATIO_LIMIT = 4.0  # tie-heavy kinds alone: p50 at most this times the 64-level row's
# the kernels and the planner that shapes their launches (the counters depend
# on both)
KERNEL_SOURCES = ("exact_row_top_amd/csrc/gvr_kernels.hip", "exact_row_top_amd/csrc/gvr_common.h",
                  "exact_row_top_amd/csrc/gvr_device.h", "exact_row_top_amd/csrc/row_window.h",
                  "exact_row_top_amd/csrc/blockskip.hip", "exact_row_top_amd/csrc/topk_abi.cpp")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(workload_name: str):
    """Measured HBM bytes per launch from committed rocprofv3 counter runs,
    or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tab = json.load(f)
    ent = tab.get(workload_name)
    if not ent or ent.get("kernel_hash") != kernel_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


def latency_samples(steps: int) -> int:
    """Latency samples per workload: never fewer than 200, whatever --steps."""
    return max(MIN_LATENCY_SAMPLES, int(steps))


def rotation(read_bytes: int) -> int:
    """Copies to rotate so that >= ROTATE_BYTES of scores are read between two
    reads of one copy (read_bytes: scores one launch reads)."""
    return max(2, math.ceil(ROTATE_BYTES / max(int(read_bytes), 1)) + 1)


def read_bytes_of(w) -> int:
    nv = w.valid_lengths()
    return int(4 * nv[nv > w.k].sum())


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float = 10.0, single_s: float = 4.0):
    """The oracle on the host over whole batches, bounded: all cores, then one
    core (same rows, one thread)."""
    import oracle
    cores = oracle.online_cores()

    def timed(nthreads, budget):
        rows, reps = 0, 0
        t0 = time.perf_counter()
        while True:
            if w.mode == "decode":
                oracle.topk_decode(w.logits, w.n_valid, w.k, nthreads=nthreads)
            else:
                oracle.topk_prefill(w.logits, w.row_starts, w.row_ends, w.k, nthreads=nthreads)
            reps += 1
            rows += w.num_rows
            el = time.perf_counter() - t0
            if el >= budget:
                return rows, reps, el

    rows, reps, el = timed(0, budget_s)
    rows1, reps1, el1 = timed(1, single_s)
    return {
        "value": rows / el,
        "unit": "rows/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{reps} full batch(es) of {w.name} ({rows} rows, {el:.2f} s wall on {cores} "
                  f"threads)",
        "single_thread_rows_per_s": rows1 / el1,
        "single_thread_sample": f"{reps1} batch(es), {el1:.2f} s on 1 thread",
        "cpu_model": cpu_model(),
    }


def copy_calib(torch, steps: int):
    """A plain device copy of known size: 256 MiB read, 256 MiB written per
    launch.  Its FETCH_SIZE / WRITE_SIZE counter readings give the scale from
    counter units to bytes for the top-K kernel's readings."""
    n = 64 << 20
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(max(steps, 1)):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calib_bytes_read": n * 4, "copy_calib_bytes_written": n * 4,
                      "launches": max(steps, 1)}), flush=True)


class Runner:
    """One workload on the device: rotating copies, extents, output,
    workspace, and the launch of step i."""

    def __init__(self, torch, ert, w, hints=None, bmax_mode=None, warm_only=False):
        self.torch, self.ert, self.w = torch, ert, w
        x = torch.from_numpy(np.ascontiguousarray(w.logits)).cuda()
        self.ncopies = 1 if warm_only else rotation(read_bytes_of(w))
        self.copies = torch.empty((self.ncopies,) + tuple(x.shape), dtype=x.dtype, device="cuda")
        self.copies[:] = x
        if w.mode == "decode":
            self.ext = (torch.from_numpy(w.n_valid).cuda(),)
            self.fn = ert.topk_decode
        else:
            self.ext = (torch.from_numpy(w.row_starts).cuda(), torch.from_numpy(w.row_ends).cuda())
            self.fn = ert.topk_prefill
        self.kw = {}
        if hints is not None:
            self.kw["pre_idx"] = torch.from_numpy(hints).cuda()
        if bmax_mode is not None:
            # the block maxima come with the scores (the indexer GEMM's
            # epilogue writes them); produced here once per copy, untimed
            self.bmax = torch.stack([ert.block_max(self.copies[i]) for i in range(self.ncopies)])
            self.kw["blockskip"] = bmax_mode
        else:
            self.bmax = None
        self.out = torch.empty((w.num_rows, w.k), dtype=torch.int32, device="cuda")
        self.read_floor = False
        self.sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.ws = ert.new_workspace(w.num_rows, w.row_stride, w.k)
        torch.cuda.synchronize()

    def step(self, i, copy=None):
        c = (i % self.ncopies) if copy is None else copy
        if self.read_floor:
            self.ert.read_floor(self.copies[c], self.ext[0], self.w.k,
                                extents2=self.ext[1] if len(self.ext) > 1 else None,
                                sink=self.sink)
            return
        kw = dict(self.kw)
        if self.bmax is not None:
            kw["bmax"] = self.bmax[c]
        self.fn(self.copies[c], *self.ext, self.w.k, indices=self.out, workspace=self.ws, **kw)

    def bytes_resident(self) -> int:
        return self.copies.numel() * 4


def flush(torch, buf):
    buf.fill_(1.0)


def measure(torch, run: Runner, steps: int, warmup: int, flush_buf, eager: bool = False,
            warm_graph: bool = True):
    """Cold graph-region mean, cold and warm latency samples, warm graph mean."""
    for i in range(warmup):
        run.step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)

    def region(launch_all):
        flush(torch, flush_buf)
        torch.cuda.synchronize()
        # a GPU sleep ahead of the start event: the launches are queued
        # before the GPU reaches the event, so the region holds their
        # execution only, not the host's submission of the first ones
        torch.cuda._sleep(SUBMIT_SLEEP_CYCLES)
        t_start.record()
        launch_all()
        t_end.record()
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end) * 1e3  # us

    def graph_of(fn):
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                fn()
        torch.cuda.synchronize()
        g.replay()  # untimed: the first replay pays any one-time setup
        torch.cuda.synchronize()
        return g

    if eager:
        # K launches issued one by one (counter runs)
        def eager_all():
            for i in range(steps):
                run.step(warmup + i)
        region_us = region(eager_all)
    else:
        g = graph_of(lambda: [run.step(warmup + i) for i in range(steps)])
        region_us = region(g.replay)
        del g

    # latency samples: cold (each behind its own 1 GiB fill), then warm (the
    # same copy again and again, no fill), all queued behind a GPU sleep
    n_lat = latency_samples(steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(2 * n_lat)]
    torch.cuda._sleep(int(20e6))
    for i in range(n_lat):
        flush(torch, flush_buf)
        ev[i][0].record()
        run.step(i)
        ev[i][1].record()
    for i in range(n_lat):
        ev[n_lat + i][0].record()
        run.step(0, copy=0)
        ev[n_lat + i][1].record()
    torch.cuda.synchronize()
    per = np.array([s.elapsed_time(e) for s, e in ev]) * 1e3
    cold, warm = per[:n_lat], per[n_lat:]

    warm_us = None
    if warm_graph:
        gw = graph_of(lambda: [run.step(0, copy=0) for _ in range(steps)])
        torch.cuda.synchronize()
        torch.cuda._sleep(SUBMIT_SLEEP_CYCLES)
        t_start.record()
        gw.replay()
        t_end.record()
        torch.cuda.synchronize()
        warm_us = t_start.elapsed_time(t_end) * 1e3 / steps
        del gw
    return {
        "region_us": region_us,
        "us_per_launch": region_us / steps,
        "p50_us": float(np.percentile(cold, 50)),
        "p99_us": float(np.percentile(cold, 99)),
        "latency_samples": n_lat,
        "warm_us_per_launch": warm_us,
        "warm_p50_us": float(np.percentile(warm, 50)),
        "warm_p99_us": float(np.percentile(warm, 99)),
    }


def summary(w, m, alg_bytes=None):
    alg = w.algorithmic_bytes() if alg_bytes is None else alg_bytes
    us = m["us_per_launch"]
    gbs = alg / (us * 1e-6) / 1e9
    rows = w.num_rows
    return {
        "workload": w.name,
        "rows": rows,
        "k": w.k,
        "algorithmic_bytes": alg,
        "us_per_launch": us,
        "rows_per_s": rows / (us * 1e-6),
        "gbs": gbs,
        "frac": gbs / PEAK_HBM_GBS,
        "p50_us": m["p50_us"],
        "p99_us": m["p99_us"],
        "p50_us_per_row": m["p50_us"] / rows,
        "p99_us_per_row": m["p99_us"] / rows,
        "latency_samples": m["latency_samples"],
        "warm_us_per_launch": m["warm_us_per_launch"],
        "warm_p50_us": m["warm_p50_us"],
        "warm_p99_us": m["warm_p99_us"],
    }


def tail_protocol(torch, ert, workloads, steps, flush_buf):
    """Each tie-heavy row kind alone at BS = 1, cold: p50 / p99 and the ratio
    of its p50 to the 64-level row's (no kind may pass TAIL_RATIO_LIMIT)."""
    w5 = workloads.tie_heavy()
    kinds = {}
    for r, kind in enumerate(workloads.TIE_ROW_KINDS):
        w = workloads.Workload(f"tie_heavy_{kind}_1x{w5.row_stride}_k{w5.k}", "decode",
                               np.ascontiguousarray(w5.logits[r:r + 1]), w5.k,
                               n_valid=w5.n_valid[r:r + 1].copy())
        run = Runner(torch, ert, w, warm_only=True)
        m = measure(torch, run, steps, 5, flush_buf, warm_graph=False)
        kinds[kind] = {"p50_us": m["p50_us"], "p99_us": m["p99_us"],
                       "warm_p50_us": m["warm_p50_us"]}
        log(f"[bench] tail {kind}: cold p50 {m['p50_us']:.2f} p99 {m['p99_us']:.2f} us")
        del run
    base = kinds[workloads.TIE_ROW_KINDS[0]]["p50_us"]
    for v in kinds.values():
        v["p50_ratio_to_quantised64"] = v["p50_us"] / base
    worst = max(v["p50_ratio_to_quantised64"] for v in kinds.values())
    return {"kinds": kinds, "criterion": f"p50 <= {TAIL_RATIO_LIMIT} x quantised64 p50",
            "worst_ratio": worst, "pass": bool(worst <= TAIL_RATIO_LIMIT)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=HEADLINE,
                    help="1..5 (3, the prefill tile, is the headline); 6 = workload 2's shape "
                         "as a decode step with the previous step's top-K as hints; 7 / 8 = a "
                         "128 MiB decode batch with block maxima (rows with locality / i.i.d.)")
    ap.add_argument("--no-hints", action="store_true",
                    help="workload 6 without its hints (the same rows, sample-only guess)")
    ap.add_argument("--blockskip", type=int, default=0, choices=(-1, 0, 1),
                    help="workloads 7 / 8: 0 = the size gate decides, 1 = force the block-skip "
                         "pass, -1 = the ordinary path")
    ap.add_argument("--bs", type=int, default=1, help="batch size for workload 4")
    ap.add_argument("--no-extra", action="store_true",
                    help="only the chosen workload (no other workloads, no tail protocol)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline leg")
    ap.add_argument("--read-floor", action="store_true",
                    help="time the read floor instead of the selection: a launch that reads "
                         "exactly the scores the selection reads, in its launch shape, and "
                         "nothing else (a measurement aid)")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of a graph replay (for counter runs)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a plain 256 MiB device copy, the counter scale reference")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    if args.copy_calib:
        copy_calib(torch, args.steps)
        return

    import exact_row_top_amd as ert
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ert.load_library()
    flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    hints, bmax_mode = None, None
    if args.workload in (7, 8):
        w = workloads.decode_blockskip(smooth=2.0 if args.workload == 7 else 0.0)
        bmax_mode = args.blockskip
    elif args.workload == 6:
        w, hints = workloads.decode_step()
        if args.no_hints:
            hints = None
            w.name = w.name.replace("_hinted", "_unhinted")
    else:
        kw = {"bs": args.bs} if args.workload == 4 else {}
        w = workloads.config(args.workload, **kw)
    rows, k = w.num_rows, w.k
    alg_bytes = w.algorithmic_bytes()
    if hints is not None:
        # a long row's hint row is read once (short rows read none)
        alg_bytes += 4 * k * int((w.valid_lengths() > k).sum())
    log(f"[bench] workload {w.name}: {rows} rows, stride {w.row_stride}, k={k}, "
        f"algorithmic bytes/launch {alg_bytes}")
    run = Runner(torch, ert, w, hints=hints, bmax_mode=bmax_mode)
    bsk_info = None
    if bmax_mode is not None:
        st = torch.full((rows, ert.STATS_WORDS), -7, dtype=torch.int32, device="cuda")
        ert.topk_decode(run.copies[0], *run.ext, k, indices=run.out, workspace=run.ws,
                        row_stats=st, bmax=run.bmax[0], blockskip=bmax_mode)
        torch.cuda.synchronize()
        st = st.cpu().numpy()
        nvr = w.valid_lengths()
        longr = nvr > k
        nbr = (nvr + 31) // 32
        if bool(np.all(st[longr, 6] == 1) and np.all(st[longr, 8] > 0)):
            visited = int(st[longr, 8].sum())
            # what the pass must move: the block maxima and the visited blocks
            # of long rows, the output and the extents
            alg_bytes = 4 * int(nbr[longr].sum()) + 128 * visited + 4 * k * rows + 4 * rows
            bsk_info = {"blocks_visited": visited, "blocks": int(nbr[longr].sum()),
                        "row_bytes_per_launch": w.algorithmic_bytes()}
        else:
            bsk_info = {"path": "ordinary"}
    run.read_floor = args.read_floor
    if args.read_floor:
        w.name += "_read_floor"
    log(f"[bench] {run.ncopies} rotating copies ({run.bytes_resident() / 2**20:.0f} MiB, "
        f"{run.ncopies * read_bytes_of(w) / 2**20:.0f} MiB of scores read per rotation)")
    t0 = time.perf_counter()
    m = measure(torch, run, args.steps, args.warmup, flush_buf, eager=args.eager)
    wall = time.perf_counter() - t0
    ncopies = run.ncopies
    del run
    head = summary(w, m, alg_bytes)
    log(f"[bench] graph region {m['region_us']:.1f} us for {args.steps} launches -> "
        f"{m['us_per_launch']:.2f} us/launch ({head['gbs']:.0f} GB/s, {100 * head['frac']:.1f} % "
        f"of peak); cold p50 {m['p50_us']:.2f} p99 {m['p99_us']:.2f} us over {m['latency_samples']} "
        f"samples; warm {m['warm_us_per_launch']:.2f} us/launch; wall {wall:.1f} s")

    ms_per_step = m["us_per_launch"] / 1e3
    res = {
        "metric": METRIC,
        "value": rows / (ms_per_step / 1e3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "rows": rows,
            "row_stride": w.row_stride,
            "k": k,
            "mode": w.mode,
            "algorithmic_bytes_per_launch": alg_bytes,
            "cache": (f"cold: {ncopies} rotating copies (>= {ROTATE_BYTES >> 20} MiB of scores "
                      f"read between two reads of one copy) and a {FLUSH_BYTES >> 20} MiB fill "
                      f"before the timed region and before each latency sample"),
            "parallelism": "single GPU",
        },
        **({"blockskip": bsk_info} if bsk_info is not None else {}),
        "p50_us_per_row": head["p50_us_per_row"],
        "p99_us_per_row": head["p99_us_per_row"],
        "p50_us_per_launch": m["p50_us"],
        "p99_us_per_launch": m["p99_us"],
        "latency_samples": m["latency_samples"],
        "warm_us_per_launch": m["warm_us_per_launch"],
        "warm_p50_us_per_launch": m["warm_p50_us"],
        "warm_p99_us_per_launch": m["warm_p99_us"],
        "timing": "eager launches" if args.eager else "graph replay",
        "roofline": {
            "bound": "hbm",
            "achieved": head["gbs"],
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": head["frac"],
            "traffic": traffic_for(w.name),
            "kernel": ("read_floor_kernel" if args.read_floor else
                       "topk_blockskip_kernel" if bsk_info and "blocks_visited" in bsk_info
                       else "gvr_topk_kernel"),
            "kernel_source_hash": kernel_hash(),
        },
    }
    if not args.no_extra and args.workload == HEADLINE and not args.read_floor:
        extra = {}
        for cfg, kw in EXTRA:
            we = workloads.config(cfg, **kw)
            re_ = Runner(torch, ert, we)
            me = measure(torch, re_, args.steps, args.warmup, flush_buf)
            del re_
            extra[we.name] = summary(we, me)
            extra[we.name]["traffic"] = traffic_for(we.name)
            log(f"[bench] {we.name}: {me['us_per_launch']:.2f} us/launch cold "
                f"({extra[we.name]['gbs']:.0f} GB/s), p50 {me['p50_us']:.2f} p99 "
                f"{me['p99_us']:.2f} us, warm {me['warm_us_per_launch']:.2f} us")
        res["configs"] = extra
        res["tail"] = tail_protocol(torch, ert, workloads, args.steps, flush_buf)
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
