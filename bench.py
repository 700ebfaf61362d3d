#!/usr/bin/env python3
"""Throughput of the MoE dispatch/combine hot path on one MI355X.

One step = the whole path over one batch of synthetic input already resident
in HBM: ep_dispatch_layout (layout counts and the dispatch plan) ->
ep_dispatch_from_layout (the row permutation) -> (expert stage of the
workload, if any) -> ep_combine, all on one stream.  W untimed warmup steps,
then K timed steps bracketed by stream synchronisation and HIP events, three
ways: replayed from HIP graphs of 10 captured steps (the reported
ms_per_step), eager back to back (eager_ms_per_step), and eager with events
between the calls (the per-call durations in phase_us: median over steps);
phase_us_flushed repeats the calls each after a 512 MiB copy that evicts the
memory-side cache (cold-cache durations).  The workloads'
expert stage (identity, per-expert scaling, or fp8 -> mxfp8 re-encoding)
runs during warmup and is not part of the timed step.  A batch of at most
2048 (token, slot) pairs is laid out and dispatched by one
ep_dispatch_with_layout (ep_dispatch_ranks_with_layout) call, which the
library runs as a single launch (phases "layout+dispatch", "combine").  With --layout ranks
the step is the (token, rank) path: ep_dispatch_layout (planning one row per
token per rank it reaches) -> ep_dispatch_ranks -> ep_combine_ranks, with
ep_expert_reduce_ranks (the weighted per-rank partials) as the expert stage.

Prints one JSON line:
  value         algorithmic HBM bytes of the step / step time (GB/s)
  tokens_per_s  tokens of the batch / step time
  dispatch_combine_gbs  the dispatch and combine calls' algorithmic bytes / their
                summed per-call durations (the layout pass left out)
  phase_gbs     each call's algorithmic bytes / its per-call duration
  rel_l2_vs_fp32  relative L2 distance of y from the unquantized fp32 result
  roofline      the longest-running call against the 8 TB/s HBM peak, with
                hardware byte counts when they were measured for this kernel,
                and against a plain 1 GiB device copy timed in the same run
  cpu_baseline  the CPU oracle (single thread) on the same workload
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--layout pairs|ranks]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine HBM GB/s and tokens/s at T=4096,H=7168,E=256,top-8"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published peak

GRAPH_STEPS = 10   # steps captured per HIP graph
SINGLE_LAUNCH_PAIRS = 2048   # batches the library lays out and dispatches in one launch
FLUSH_BYTES = 512 << 20      # copy that evicts the 256 MB memory-side cache
COPY_REF_BYTES = 1 << 30     # plain copy timed as the box's streaming reference
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash() -> str:
    """sha256 over the code of the step's kernels (layout, dispatch, combine,
    both receive layouts) and their device headers, with comments and
    whitespace removed: an edit that changes no code keeps the hash."""
    import hashlib
    import re

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "combine_dispatch_layout_02_amd", "csrc")
    for name in ("plan.hip", "dispatch.hip", "combine.hip", "ranks.hip", "ep_device.h", "ep_internal.h",
                 "small_layout.h"):
        text = open(os.path.join(csrc, name)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (rocprofv3 FETCH_SIZE / WRITE_SIZE, each scaled by its reading on a plain
    copy of known size), or None when there is none for this workload or the
    kernel sources changed since the counters were taken."""
    path = os.path.join(PROFILES, f"counters_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("#") or "=" not in line:
            continue
        parts = dict(p.split("=", 1) for p in line.split())
        if "kernel" in parts:
            fields[parts["kernel"]] = parts
        else:
            fields.update(parts)
    if fields.get("kernel_sources_sha256") != kernel_source_hash():
        return None
    for name, parts in fields.items():
        if isinstance(parts, dict) and name.startswith(kernel):
            return int(float(parts["traffic_bytes"]))
    return None


class HipEvents:
    """Timing events created with hipEventDisableSystemFence: recording them
    does not write back / invalidate the caches, so the brackets around one
    call measure that call and do not slow the next one down."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
            try:
                self.hip = ctypes.CDLL(name)
                break
            except OSError:
                continue
        self.c = ctypes
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = self.c.c_void_p()
            if self.hip.hipEventCreateWithFlags(self.c.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            evs.append(e)
        return evs

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, self.c.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        out = self.c.c_float()
        if self.hip.hipEventElapsedTime(self.c.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill2n")
    ap.add_argument("--layout", choices=("pairs", "rank_major", "ranks"), default="pairs",
                    help="receive layout: one row per (token, expert) pair at compacted offsets (default); "
                         "the same rows at fixed per-rank blocks (RANK_MAJOR, capacity = the largest rank's "
                         "pair count); or one row per (token, rank) with per-rank partials "
                         "(ep_dispatch_ranks / ep_combine_ranks)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush-steps", type=int, default=10,
                    help="also time each call after a 512 MiB cache-evicting copy, over this many steps "
                         "(phase_us_flushed; 0 to skip)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-graph", action="store_true",
                    help="time the eager loop only (default: K steps replayed from HIP graphs of %d steps)" % GRAPH_STEPS)
    ap.add_argument("--sweep", action="store_true",
                    help="time the step at T = 1, 2, 4, ..., 8192 tokens (the workload's other sizes fixed) "
                         "and print one JSON line with the series")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run the plain copy kernel on this many MiB, --steps times (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU's share of the exchange (destinations are "
                                   "regions of one GPU's memory); runs on more than one GPU are not "
                                   "supported (use --gpus 1)"}))
        sys.exit(2)

    import torch

    from combine_dispatch_layout_02_amd import ep

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ep.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(args.steps):
            ep.ep_calib_copy(src, dst, n)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "launches": args.steps}))
        return

    if args.sweep:
        series = []
        for T in [2 ** i for i in range(14)]:
            o = measure(args.workload, args.steps, args.warmup, not args.no_graph, args.layout, T=T)
            o.pop("_inp")
            series.append({"tokens": T, "us_per_step": round(o["ms_per_step"] * 1000, 2),
                           "tokens_per_s": o["tokens_per_s"], "gbs": o["value"], "phase_us": o["phase_us"]})
        print(json.dumps({"metric": "step time vs tokens per source (" + args.workload + " shape, "
                                    + args.layout + " layout)",
                          "unit": "us", "series": series}), flush=True)
        return
    out = measure(args.workload, args.steps, args.warmup, not args.no_graph, args.layout, args.flush_steps)
    inp = out.pop("_inp")
    if not args.no_cpu_baseline:
        cfg = dict(inp, rank_rows=args.layout == "ranks", rank_capacity=out["config"]["rank_capacity"])
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds, out["step_algorithmic_bytes"])
    print(json.dumps(out), flush=True)


def measure(workload: str, steps: int, warmup: int, graph: bool = False, layout_kind: str = "pairs",
            flush_steps: int = 0, **overrides) -> dict:
    """Time `steps` steps of the path on `workload` (inputs resident in HBM);
    keyword overrides change the workload's shape (e.g. T=...).  layout_kind
    "ranks" times the (token, rank) path: layout, ep_dispatch_ranks,
    ep_combine_ranks (bf16 partials; the expert stage returns them)."""
    import numpy as np
    import torch

    from combine_dispatch_layout_02_amd import ep, workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    inp = workloads.make_inputs(workload, **overrides)
    T, H, E, R, N, k = (inp[n] for n in ("T", "H", "E", "R", "N", "k"))
    fp8 = inp["x_fmt"] == "fp8"
    nv = inp.get("y_fmt") == "nvfp4"
    ranks = layout_kind == "ranks"
    if ranks and nv:
        raise ValueError("the (token, rank) path returns bf16 partials; use a bf16-payload workload")
    M = 0
    if layout_kind == "rank_major" and (fp8 or nv or inp["expert"] == "scale"):
        raise ValueError("the workloads' expert stages use the compacted layout; RANK_MAJOR runs bf16 "
                         "identity workloads (prefill2n, skewed, tiny)")
    if layout_kind == "rank_major":   # capacity per rank: the largest rank's pair count (nothing dropped)
        ids = inp["topk_idx"]
        ok = (ids >= 0) & (ids < E)
        M = int(np.bincount(ids[ok] // (E // R), minlength=R).max())
    yf = ep.EP_FMT_NVFP4 if nv else (ep.EP_FMT_MXFP8 if (fp8 and not ranks) else ep.EP_FMT_BF16)
    shape = ep.make_shape(T, H, E, R, N, k, ep.EP_FMT_FP8_S128 if fp8 else ep.EP_FMT_BF16, yf,
                          rank_capacity=M, rank_rows=1 if ranks else 0)
    rows = shape.rows
    ws = ep.Workspace(shape, dev)

    # inputs resident in HBM before timing
    x = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    w = torch.from_numpy(inp["topk_w"]).to(dev)
    factor = None if inp["expert_factor"] is None else torch.from_numpy(inp["expert_factor"]).to(dev)
    if fp8:   # input quantization is outside the timed step
        xin, xs = ep.quant_fp8_s128(x)
    else:
        xin, xs = x, None

    # every output allocated once, outside the timed region
    lay = dict(r=torch.empty(R, dtype=torch.int32, device=dev), e=torch.empty(E, dtype=torch.int32, device=dev),
               m=torch.empty((T, R), dtype=torch.uint8, device=dev), n=torch.empty(N, dtype=torch.int32, device=dev),
               a=torch.empty(1, dtype=torch.int64, device=dev))
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def layout():
        ep.ep_dispatch_layout(shape, idx, lay["r"], lay["e"], lay["m"], lay["n"], lay["a"], ws)

    if ranks:
        cap = shape.rank_rows_cap
        recv_x = torch.empty((cap, H), dtype=xin.dtype, device=dev)
        recv_s = torch.empty((cap, H // 128), dtype=torch.float32, device=dev) if fp8 else None
        src = torch.empty(cap, dtype=torch.int32, device=dev)
        r_idx = torch.empty((cap, k), dtype=torch.int32, device=dev)
        r_w = torch.empty((cap, k), dtype=torch.float32, device=dev)
        trs = torch.empty((T, R), dtype=torch.int32, device=dev)
        roff = torch.empty(R + 1, dtype=torch.int32, device=dev)
        part = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)

        def dispatch():   # reuses the plan the layout call of this step left in the workspace
            ep.ep_dispatch_ranks(shape, xin, xs, idx, w, recv_x, recv_s, src, r_idx, r_w, trs, roff, ws)

        def layout_dispatch():   # one call; a single launch for batches of <= 2048 pairs
            ep.ep_dispatch_ranks_with_layout(shape, xin, xs, idx, w, lay["r"], lay["e"], lay["m"], lay["n"],
                                             lay["a"], recv_x, recv_s, src, r_idx, r_w, trs, roff, ws)

        def expert():
            ep.ep_expert_reduce_ranks(shape, recv_x, recv_s, roff, r_idx, r_w,
                                      factor if inp["expert"] == "scale" else None, part)

        def combine():
            ep.ep_combine_ranks(shape, part, trs, y)
    else:
        recv_x = torch.empty((rows, H), dtype=xin.dtype, device=dev)
        recv_s = torch.empty((rows, H // 128), dtype=torch.float32, device=dev) if fp8 else None
        src = torch.empty(rows, dtype=torch.int32, device=dev)
        rw = torch.empty(rows, dtype=torch.float32, device=dev)
        slot = torch.empty((T, k), dtype=torch.int32, device=dev)
        off = torch.empty(E + 1, dtype=torch.int32, device=dev)
        if fp8:
            eo = torch.empty((rows, H), dtype=torch.uint8, device=dev)
            eos = torch.empty((rows, H // 32), dtype=torch.uint8, device=dev)
        elif nv:
            eo = torch.empty((rows, H // 2), dtype=torch.uint8, device=dev)
            eos = torch.empty((rows, H // 16), dtype=torch.int16, device=dev)
        elif inp["expert"] == "scale":
            eo, eos = torch.empty_like(recv_x), None
        else:
            eo, eos = recv_x, None   # identity expert: combine reads the receive buffer itself

        def dispatch():   # reuses the plan the layout call of this step left in the workspace
            ep.ep_dispatch(shape, xin, xs, idx, w, recv_x, recv_s, src, rw, slot, off, ws, from_layout=True)

        def layout_dispatch():   # one call; a single launch for batches of <= 2048 pairs
            ep.ep_dispatch_with_layout(shape, xin, xs, idx, w, lay["r"], lay["e"], lay["m"], lay["n"], lay["a"],
                                       recv_x, recv_s, src, rw, slot, off, ws)

        def expert():
            if fp8:
                ep.ep_expert_requant_mxfp8(shape, off, factor, recv_x, recv_s, eo, eos)
            elif nv:
                ep.ep_expert_requant_nvfp4(shape, off, factor, recv_x, eo, eos)
            elif inp["expert"] == "scale":
                ep.ep_expert_scale_bf16(shape, off, factor, recv_x, eo)

        def combine():
            ep.ep_combine(shape, eo, eos, slot, w, y)

    # the expert stage stands in for the expert computation between dispatch
    # and combine: it runs in warmup (its output does not change from step to
    # step, the inputs being the same) and stays out of the timed step
    phases = [("layout", layout), ("dispatch", dispatch), ("combine", combine)]
    single_launch = M == 0 and T * k <= SINGLE_LAUNCH_PAIRS
    if single_launch:   # the library runs layout + dispatch of such a batch as one kernel
        phases = [("layout+dispatch", layout_dispatch), ("combine", combine)]

    def step():
        for _, fn in phases:
            fn()

    for _ in range(max(1, warmup)):
        for name, fn in phases:
            fn()
            if name != "combine" and name != "layout":
                expert()
    ws.check()
    torch.cuda.synchronize()
    V = int((inp["topk_idx"] >= 0).sum() - (inp["topk_idx"] >= E).sum())   # valid pairs
    y_ref = y.clone()   # every step recomputes the same y from the same inputs
    hev = HipEvents()

    def timed(run_steps) -> float:
        """ms per step of `steps` steps, stream-synchronised on both sides."""
        a0, a1 = hev.create(2)
        torch.cuda.synchronize()
        hev.record(a0, stream)
        run_steps()
        hev.record(a1, stream)
        torch.cuda.synchronize()
        ms = hev.ms(a0, a1) / steps
        hev.destroy([a0, a1])
        return ms

    # (1) eager: K steps back to back on the stream
    def eager():
        for _ in range(steps):
            step()
    eager_ms = timed(eager)
    ws.check()

    # (2) per-call durations: K more steps with events between the calls
    ev = [hev.create(len(phases) + 1) for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        hev.record(ev[s][0], stream)
        for i, (_, fn) in enumerate(phases):
            fn()
            hev.record(ev[s][i + 1], stream)
    torch.cuda.synchronize()
    # median over the steps: a host-side submission stall (e.g. a pause of the
    # interpreter) leaves the GPU idle between two events and inflates one
    # sample; the median keeps the kernel's own duration
    samples = {name: sorted(1000.0 * hev.ms(ev[s][i], ev[s][i + 1]) for s in range(steps))
               for i, (name, _) in enumerate(phases)}
    phase_us = {name: statistics.median(v) for name, v in samples.items()}
    phase_stats = {name: {"min": round(v[0], 2), "p90": round(v[min(len(v) - 1, int(0.9 * len(v)))], 2)}
                   for name, v in samples.items()}
    for e in ev:
        hev.destroy(e)

    # (2b) the same calls, each after a flush of the memory-side cache (a
    # 512 MiB copy, more than the 256 MB cache holds, outside the events): the
    # cold-cache duration of each call
    phase_us_flushed = None
    if flush_steps:
        fl_src = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        fl_dst = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        evf = [hev.create(2 * len(phases)) for _ in range(flush_steps)]
        torch.cuda.synchronize()
        for s_ in range(flush_steps):
            for i, (_, fn) in enumerate(phases):
                ep.ep_calib_copy(fl_src, fl_dst, FLUSH_BYTES)
                hev.record(evf[s_][2 * i], stream)
                fn()
                hev.record(evf[s_][2 * i + 1], stream)
        torch.cuda.synchronize()
        phase_us_flushed = {name: 1000.0 * statistics.median(hev.ms(evf[s_][2 * i], evf[s_][2 * i + 1])
                                                             for s_ in range(flush_steps))
                            for i, (name, _) in enumerate(phases)}
        for e in evf:
            hev.destroy(e)
        del fl_src, fl_dst

    # (3) HIP graph: G steps captured once, replayed K/G times (launch gaps
    # between steps vanish inside a graph, as in a captured serving loop)
    graph_ms, G = None, 0
    if graph:
        G = max(1, min(GRAPH_STEPS, steps))
        while steps % G:
            G -= 1
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(G):
                step()
        for _ in range(2):   # replays, with eager work and syncs in between, must match the eager result
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(y.view(torch.int16), y_ref.view(torch.int16)):
                raise RuntimeError("graph replay differs from the eager step")
            step()
            torch.cuda.synchronize()

        def replays():
            for _ in range(steps // G):
                g.replay()
        graph_ms = timed(replays)
        if not torch.equal(y.view(torch.int16), y_ref.view(torch.int16)):
            raise RuntimeError("graph replays differ from the eager step")
    ms_step = graph_ms if graph_ms is not None else eager_ms

    # the same box's plain device copy (1 GiB read + 1 GiB written), as a
    # measured streaming reference next to the published peak
    cp_src = torch.empty(COPY_REF_BYTES, dtype=torch.uint8, device=dev)
    cp_dst = torch.empty(COPY_REF_BYTES, dtype=torch.uint8, device=dev)
    ep.ep_calib_copy(cp_src, cp_dst, COPY_REF_BYTES)
    c0, c1 = hev.create(2)
    torch.cuda.synchronize()
    hev.record(c0, stream)
    for _ in range(5):
        ep.ep_calib_copy(cp_src, cp_dst, COPY_REF_BYTES)
    hev.record(c1, stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * COPY_REF_BYTES * 5 / (hev.ms(c0, c1) * 1e-3) / 1e9
    hev.destroy([c0, c1])
    del cp_src, cp_dst

    # accuracy of the step's y against the unquantized fp32 result, computed
    # in float64 from the inputs: sum over valid slots of w * s_e * x (s_e = 1
    # for the identity expert)
    xf = x.double()
    y32 = torch.zeros_like(xf)
    fac = factor.double() if (factor is not None and inp["expert"] == "scale") else None
    for j in range(k):
        e = idx[:, j]
        ok = (e >= 0) & (e < E)
        wj = torch.where(ok, w[:, j].double(), torch.zeros_like(w[:, j], dtype=torch.float64))
        if fac is not None:
            wj = wj * fac[torch.where(ok, e, torch.zeros_like(e))]
        y32 += wj[:, None] * xf
    rel_l2 = float(torch.linalg.vector_norm(y.double() - y32) / torch.linalg.vector_norm(y32).clamp_min(1e-300))
    del xf, y32

    # algorithmic bytes (library accounting on host copies of the layout)
    acc = ep.ep_accounting(shape, 0, lay["r"].cpu().numpy(), lay["n"].cpu().numpy(), int(lay["a"].item()), V)
    if ranks:
        algo_bytes = {"layout": acc["hbm_layout_bytes"], "dispatch": acc["hbm_dispatch_ranks_bytes"],
                      "combine": acc["hbm_combine_ranks_bytes"]}
        kernels = {"dispatch": "ep_dispatch_ranks_kernel", "combine": "ep_combine_ranks_kernel"}
    else:
        algo_bytes = {"layout": acc["hbm_layout_bytes"], "dispatch": acc["hbm_dispatch_bytes"],
                      "combine": acc["hbm_combine_bytes"]}
        kernels = {"dispatch": "ep_dispatch_copy_kernel", "combine": "ep_combine_" +
                   ("mxfp8" if fp8 else ("nvfp4" if nv else "bf16")) + "_kernel"}
    step_bytes = sum(algo_bytes.values())
    step_s = ms_step / 1000.0
    if single_launch:
        algo_bytes = {"layout+dispatch": algo_bytes["layout"] + algo_bytes["dispatch"],
                      "combine": algo_bytes["combine"]}
        kernels["layout+dispatch"] = kernels["dispatch"]
    dom = max((p for p in algo_bytes if p != "layout"), key=lambda p: phase_us[p])
    achieved = algo_bytes[dom] / (phase_us[dom] * 1e-6) / 1e9
    traffic = measured_traffic(workload + ("_ranks" if ranks else ""), kernels[dom])

    out = {
        "metric": METRIC,
        "value": round(step_bytes / step_s / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8/bf16" if ranks else "fp8/mxfp8") if fp8 else ("bf16/nvfp4" if nv else "bf16"),
        "data": "synthetic",
        "config": {"workload": workload, "tokens": T, "hidden": H, "experts": E, "virtual_ranks": R,
                   "virtual_nodes": N, "topk": k, "routing": inp["routing"], "expert": inp["expert"],
                   "x_format": inp["x_fmt"], "valid_pairs": V,
                   "receive_layout": "(token, rank) rows" if ranks else
                   ("(token, expert) rows, RANK_MAJOR" if M else "(token, expert) rows"),
                   "rank_capacity": M, "receive_rows": int(acc["nvl_tokens"]) if ranks else V},
        "tokens_per_s": round(T / step_s, 1),
        "dispatch_combine_gbs": round(sum(algo_bytes[p] for p in algo_bytes if p != "layout")
                                      / (sum(phase_us[p] for p in phase_us if p != "layout") * 1e-6) / 1e9, 1),
        "rel_l2_vs_fp32": round(rel_l2, 6),
        "phase_us": {p: round(v, 2) for p, v in phase_us.items()},
        "phase_gbs": {p: round(algo_bytes[p] / (phase_us[p] * 1e-6) / 1e9, 1) for p in algo_bytes},
        "phase_us_min_p90": phase_stats,
        "phase_us_flushed": None if phase_us_flushed is None else
        {p: round(v, 2) for p, v in phase_us_flushed.items()},
        "step_algorithmic_bytes": int(step_bytes),
        "eager_ms_per_step": round(eager_ms, 4),
        "timing": ("steps replayed from a HIP graph of %d steps" % G) if graph_ms is not None else "eager",
        "roofline": {"bound": "hbm", "kernel": kernels[dom], "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": int(algo_bytes[dom]),
                     "measured_copy_gbs": round(copy_gbs, 1), "frac_of_copy": round(achieved / copy_gbs, 4)},
        "pages_accounting": {"rdma_algo_tokens": acc["rdma_algo_tokens"],
                             "rdma_physical_tokens": acc["rdma_physical_tokens"],
                             "nvl_tokens": acc["nvl_tokens"],
                             "dispatch_rdma_bytes_bf16": acc["dispatch_rdma_bytes_bf16"],
                             "dispatch_nvl_bytes_bf16": acc["dispatch_nvl_bytes_bf16"]},
    }
    out["_inp"] = inp
    return out


def cpu_baseline(inp, seconds, step_bytes):
    """The CPU oracle as it stands (plain C, one thread) on the same workload:
    whole passes (layout, slots, dispatch rows, expert stage, combine) repeated
    until `seconds` of CPU work, at least one pass; then one more pass timed
    part by part (layout, slots + dispatch rows, combine)."""
    import oracle

    reps, t_start = 0, time.perf_counter()
    while True:
        oracle.run_path(inp)
        reps += 1
        if time.perf_counter() - t_start >= seconds:
            break
    dt = (time.perf_counter() - t_start) / reps
    parts = {}
    if not inp.get("rank_rows") and inp.get("x_fmt", "bf16") == "bf16" and inp.get("y_fmt", "bf16") == "bf16":
        idx, w = inp["topk_idx"], inp["topk_w"]
        t0 = time.perf_counter()
        oracle.layout(idx, inp["E"], inp["R"], inp["N"])
        t1 = time.perf_counter()
        sl = oracle.slots(idx, w, inp["E"])
        recv = oracle.dispatch_rows(inp["x"], sl["token_slot"])
        t2 = time.perf_counter()
        oracle.combine_bf16(recv, sl["token_slot"], w)
        t3 = time.perf_counter()
        parts = {"layout_s": round(t1 - t0, 4), "slots_dispatch_s": round(t2 - t1, 4), "combine_s": round(t3 - t2, 4)}
    return {"value": round(inp["T"] / dt, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "gbs": round(step_bytes / dt / 1e9, 3), "parts": parts,
            "sample": f"{reps} full passes of workload {inp['name']} (T={inp['T']}), {dt:.3f} s per pass"}


if __name__ == "__main__":
    main()
