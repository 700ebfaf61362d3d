#!/usr/bin/env python3
"""Throughput of the MoE dispatch/combine hot path on one MI355X.

One step = the whole path over one batch of synthetic input already resident
in HBM, all on one stream: layout -> dispatch -> (the workload's expert
stage, if any) -> combine.  Token-major rows: one ep_dispatch_with_layout
call (layout counts, plan and row permutation; a single launch up to 2048
(token, slot) pairs, else a count launch and the copy that scans the
counts) -> ep_combine; phases "layout+dispatch" and "combine".  --layout
ranks times the (token, rank) path the same way: ep_dispatch_ranks_with_layout
(one row per token per rank it reaches) -> ep_combine_ranks, with
ep_expert_reduce_ranks (the weighted per-rank partials) as the expert stage.
--split-layout times ep_dispatch_layout -> ep_dispatch_from_layout (or
ep_dispatch_ranks; the layout call's plan reused) -> the combine instead.
--layout rank_major gives the token-major rows fixed per-rank blocks
(rank_capacity).
The expert stage (identity, per-expert scaling, fp8 -> mxfp8 or bf16 ->
nvfp4 re-encoding) runs during warmup and is not part of the timed step.
W untimed warmup steps, then K timed steps bracketed by stream
synchronisation and HIP events, three ways: replayed from HIP graphs of 10
captured steps (the reported ms_per_step), eager back to back
(eager_ms_per_step), and eager with events between the calls (the per-call
durations in phase_us: median over steps).

Warm and cold.  The 256 MB memory-side cache (MALL) of MI355X is a
write-back cache: plain stores leave dirty lines there, written back to HBM
when something evicts them (non-temporal stores leave none).  Back to back
on the same buffers (the warm `value`), the receive rows and x that one
step leaves in it are read by the combine from it and
rewritten by the next step's dispatch before they ever reach HBM, so the
warm figure counts up to ~256 MB of "HBM" writes per step that HBM never
sees.  The cold figures charge them: `cold` times HIP graphs of [a 512 MiB
plain-read flush, step] minus graphs of [flush] alone.  The flush leaves the
cache clean and evicts everything the step left there, so the write-back of
the step's dirty lines lands in the flush that follows it and is counted in
the difference.  cold.phase_us does the same for each call alone; within
a step the combine reads rows the dispatch just left in the cache, so the
cold step can take less than its calls alone.

Prints one JSON line:
  value         algorithmic HBM bytes of the step / warm step time (GB/s)
  tokens_per_s  tokens of the batch / warm step time
  cold          ms_per_step, value, tokens_per_s, phase_us and phase_gbs with
                the memory-side cache flushed before each step and the
                step's write-back charged (see above)
  dispatch_combine_gbs  the dispatch and combine calls' algorithmic bytes / their
                summed per-call durations (the layout pass left out)
  phase_gbs     each call's algorithmic bytes / its warm per-call duration
  rel_l2_vs_fp32  relative L2 distance of y from the unquantized fp32 result
  roofline      the longest-running call against the 8 TB/s HBM peak (warm,
                MALL-assisted: frac; cold: cold_frac), with hardware byte
                counts when they were measured for this kernel; each row
                call's cold rate against 8 TB/s and against the ceiling that
                matches its mix of reads and writes (ceilings, below)
  ceilings      the box's streaming read, write and copy rates, measured in
                the same run: back-to-back launches alternating over 1 GiB
                buffers (so write-backs are charged), best over a few launch
                shapes
  cpu_baseline  the CPU oracle on the same workload, one thread and all cores
  kernel_sources_sha256  hash of the step kernels' code (comments and
                whitespace removed), as stated in the profiles/ summaries
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--layout pairs|rank_major|ranks] [--split-layout] [--sweep]
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
FLUSH_BYTES = 512 << 20      # plain read that evicts the 256 MB memory-side cache and leaves it clean
FLUSH_CHUNK, FLUSH_WAVES = 16384, 4096
CEIL_BYTES = 1 << 30         # streaming ceilings: launches alternate over buffers of this size
CEIL_LAUNCHES = 8
CEIL_SHAPES = [(c, w) for c in (4096, 16384, 65536) for w in (4096, 16384, 65536)]
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
    ap.add_argument("--split-layout", action="store_true",
                    help="time ep_dispatch_layout + ep_dispatch_from_layout / ep_dispatch_ranks (the plan reused) "
                         "instead of one ep_dispatch_with_layout / ep_dispatch_ranks_with_layout call")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache step and per-call timings (graphs with a 512 MiB read flush "
                         "before each step)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the streaming read / write / copy ceilings")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="CPU work for the oracle baseline, split between its one-thread and all-core timings")
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
            o = measure(args.workload, args.steps, args.warmup, not args.no_graph, args.layout,
                        split_layout=args.split_layout, T=T)
            o.pop("_inp")
            series.append({"tokens": T, "us_per_step": round(o["ms_per_step"] * 1000, 2),
                           "tokens_per_s": o["tokens_per_s"], "gbs": o["value"], "phase_us": o["phase_us"]})
        print(json.dumps({"metric": "step time vs tokens per source (" + args.workload + " shape, "
                                    + args.layout + " layout)",
                          "unit": "us", "series": series}), flush=True)
        return
    out = measure(args.workload, args.steps, args.warmup, not args.no_graph, args.layout,
                  cold=not args.no_cold and not args.no_graph, ceilings=not args.no_ceilings,
                  split_layout=args.split_layout)
    inp = out.pop("_inp")
    if not args.no_cpu_baseline:
        cfg = dict(inp, rank_rows=args.layout == "ranks", rank_capacity=out["config"]["rank_capacity"])
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds, out["step_algorithmic_bytes"])
    print(json.dumps(out), flush=True)


def measure(workload: str, steps: int, warmup: int, graph: bool = False, layout_kind: str = "pairs",
            cold: bool = False, ceilings: bool = False, split_layout: bool = False, **overrides) -> dict:
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
    # token-major rows: one ep_dispatch_with_layout call (a single launch up to
    # 2048 pairs of the compacted layout, else the count launch and the copy
    # that scans the counts); split_layout times ep_dispatch_layout +
    # ep_dispatch_from_layout instead, except for single-launch batches
    single_launch = not split_layout or (M == 0 and T * k <= SINGLE_LAUNCH_PAIRS)
    if single_launch:
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

    # (4) cold: the memory-side cache flushed (512 MiB plain read: evicts
    # everything, writes back what was dirty, leaves the cache clean) before
    # every step; graphs of [flush, step] (and of [flush, one call]) minus
    # graphs of [flush] alone, so the write-back of what the step or call
    # leaves dirty in the cache (it happens during the next flush) is
    # charged to it
    cold_res = None
    if cold and graph_ms is not None:
        cold_res = cold_timing(phases, steps, G, hev, stream, dev)
        if not torch.equal(y.view(torch.int16), y_ref.view(torch.int16)):
            raise RuntimeError("cold graph replays differ from the eager step")

    ceil = stream_ceilings(hev, stream, dev) if ceilings else None

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
        calls = {"layout": "layout", "dispatch": "dispatch_ranks", "combine": "combine_ranks"}
        kernels = {"dispatch": "ep_dispatch_ranks_kernel", "combine": "ep_combine_ranks_kernel"}
    else:
        calls = {"layout": "layout", "dispatch": "dispatch", "combine": "combine"}
        kernels = {"dispatch": "ep_dispatch_copy_kernel", "combine": "ep_combine_" +
                   ("mxfp8" if fp8 else ("nvfp4" if nv else "bf16")) + "_kernel"}
    rw = {p: (acc[f"hbm_{c}_read_bytes"], acc[f"hbm_{c}_write_bytes"]) for p, c in calls.items()}
    if single_launch:
        rw = {"layout+dispatch": (rw["layout"][0] + rw["dispatch"][0], rw["layout"][1] + rw["dispatch"][1]),
              "combine": rw["combine"]}
        kernels["layout+dispatch"] = kernels["dispatch"]
    algo_bytes = {p: r + w_ for p, (r, w_) in rw.items()}
    step_bytes = sum(algo_bytes.values())
    step_s = ms_step / 1000.0
    rows_calls = [p for p in algo_bytes if p != "layout"]
    dom = max(rows_calls, key=lambda p: phase_us[p])
    achieved = algo_bytes[dom] / (phase_us[dom] * 1e-6) / 1e9
    traffic = measured_traffic(workload + ("_ranks" if ranks else ""), kernels[dom])
    roofline = {"bound": "hbm", "kernel": kernels[dom], "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": int(algo_bytes[dom]),
                "mall_assisted": True}   # warm: back-to-back calls on the same buffers
    cold_out = None
    if cold_res is not None:
        cs = cold_res["step_us"] * 1e-6
        cph = cold_res["phase_us"]
        cold_out = {"ms_per_step": round(cold_res["step_us"] / 1000.0, 4),
                    "value": round(step_bytes / cs / 1e9, 2), "tokens_per_s": round(T / cs, 1),
                    "frac": round(step_bytes / cs / 1e9 / HBM_PEAK_GBS, 4),
                    "phase_us": {p: round(v, 2) for p, v in cph.items()},
                    "phase_gbs": {p: round(algo_bytes[p] / (cph[p] * 1e-6) / 1e9, 1) for p in algo_bytes},
                    "flush_us": round(cold_res["flush_us"], 2),
                    "method": "HIP graphs of [512 MiB plain-read flush, step] (phase_us: [flush, one call]) "
                              "minus graphs of [flush]: every step (call) starts with a clean memory-side "
                              "cache and the write-back of what it leaves dirty there is charged to it"}
        cdom = max(rows_calls, key=lambda p: cph[p])
        cach = algo_bytes[cdom] / (cph[cdom] * 1e-6) / 1e9
        roofline.update({"cold_kernel": kernels[cdom], "cold_achieved": round(cach, 1),
                         "cold_frac": round(cach / HBM_PEAK_GBS, 4),
                         "cold_step_frac": round(step_bytes / cs / 1e9 / HBM_PEAK_GBS, 4)})
        calls_out = {}
        for p in rows_calls:
            g = algo_bytes[p] / (cph[p] * 1e-6) / 1e9
            c = {"kernel": kernels[p], "cold_gbs": round(g, 1), "frac": round(g / HBM_PEAK_GBS, 4),
                 "read_bytes": int(rw[p][0]), "write_bytes": int(rw[p][1])}
            if ceil is not None:
                m = mix_ceiling(rw[p][0], rw[p][1], ceil)
                c.update({"ceiling_gbs": round(m, 1), "frac_of_ceiling": round(g / m, 4)})
            calls_out[p] = c
        roofline["calls"] = calls_out

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
        "cold": cold_out,
        "dispatch_combine_gbs": round(sum(algo_bytes[p] for p in rows_calls)
                                      / (sum(phase_us[p] for p in rows_calls) * 1e-6) / 1e9, 1),
        "rel_l2_vs_fp32": round(rel_l2, 6),
        "phase_us": {p: round(v, 2) for p, v in phase_us.items()},
        "phase_gbs": {p: round(algo_bytes[p] / (phase_us[p] * 1e-6) / 1e9, 1) for p in algo_bytes},
        "phase_us_min_p90": phase_stats,
        "step_algorithmic_bytes": int(step_bytes),
        "eager_ms_per_step": round(eager_ms, 4),
        "timing": ("steps replayed from a HIP graph of %d steps" % G) if graph_ms is not None else "eager",
        "kernel_sources_sha256": kernel_source_hash(),
        "roofline": roofline,
        "ceilings": ceil,
        "pages_accounting": {"rdma_algo_tokens": acc["rdma_algo_tokens"],
                             "rdma_physical_tokens": acc["rdma_physical_tokens"],
                             "nvl_tokens": acc["nvl_tokens"],
                             "dispatch_rdma_bytes_bf16": acc["dispatch_rdma_bytes_bf16"],
                             "dispatch_nvl_bytes_bf16": acc["dispatch_nvl_bytes_bf16"]},
    }
    out["_inp"] = inp
    return out


def _graph(body, reps: int):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            body()
    return g


def cold_timing(phases, steps: int, G: int, hev, stream, dev) -> dict:
    """Cold-cache step and per-call durations (us), write-back charged.

    Graphs of G copies of [512 MiB plain-read flush, body]: a plain read of
    more than the memory-side cache holds evicts every line, writing back the
    dirty ones, and leaves the cache clean; so each copy's body starts cold,
    and what it leaves dirty in the cache is written back during the next
    copy's flush, inside the same graph.  Subtracting the graph of G flushes
    alone leaves the body's duration with its write-back.  Bodies: the whole
    step (the cold step), and each call alone (its inputs are those of the
    last step, still in place, so every call starts from HBM; the calls of
    one step share the cache, so the step can take less than its calls
    alone).  Each graph is replayed K/G times per timing, three rounds
    alternating over the graphs, median."""
    import torch

    from combine_dispatch_layout_02_amd import ep

    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    sink = torch.empty(256, dtype=torch.uint8, device=dev)

    def flush():
        ep.ep_stream(ep.EP_STREAM_READ, flush_buf, sink, FLUSH_BYTES, FLUSH_CHUNK, FLUSH_WAVES)

    def body_of(fns):
        def body():
            flush()
            for fn in fns:
                fn()
        return body

    bodies = [[], [fn for _, fn in phases]] + [[fn] for _, fn in phases]
    graphs = [_graph(body_of(b), G) for b in bodies]
    reps = max(1, steps // G)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    samples = [[] for _ in graphs]
    for _ in range(3):
        for i, g in enumerate(graphs):
            a0, a1 = hev.create(2)
            torch.cuda.synchronize()
            hev.record(a0, stream)
            for _ in range(reps):
                g.replay()
            hev.record(a1, stream)
            torch.cuda.synchronize()
            samples[i].append(1000.0 * hev.ms(a0, a1) / (reps * G))
            hev.destroy([a0, a1])
    us = [statistics.median(v) for v in samples]
    del graphs
    return {"flush_us": us[0], "step_us": us[1] - us[0],
            "phase_us": {name: us[2 + i] - us[0] for i, (name, _) in enumerate(phases)}}


def stream_ceilings(hev, stream, dev) -> dict:
    """The box's streaming read, write and copy rates (GB/s): CEIL_LAUNCHES
    back-to-back launches of ep_stream alternating over two sets of 1 GiB
    buffers, so the cache holds nothing a launch reuses and the dirty lines
    each launch leaves are written back during the next one.  Each of read,
    write and copy is timed with plain and with non-temporal accesses, best
    over the launch shapes CEIL_SHAPES (chunk bytes x waves); "read", "write"
    and "copy" are the better of the two."""
    import torch

    from combine_dispatch_layout_02_amd import ep

    bufs = [torch.empty(CEIL_BYTES, dtype=torch.uint8, device=dev) for _ in range(4)]
    sink = torch.empty(256, dtype=torch.uint8, device=dev)
    kinds = {"read": ep.EP_STREAM_READ, "read_nt": ep.EP_STREAM_READ_NT, "write": ep.EP_STREAM_WRITE,
             "write_nt": ep.EP_STREAM_WRITE_NT, "copy": ep.EP_STREAM_COPY, "copy_nt": ep.EP_STREAM_COPY_NT}
    best = {}
    for name, kind in kinds.items():
        cls = name.split("_")[0]
        for chunk, waves in CEIL_SHAPES:
            def launch(i):
                a, b = (bufs[0], bufs[1]) if i % 2 == 0 else (bufs[2], bufs[3])
                if cls == "read":
                    ep.ep_stream(kind, a, sink, CEIL_BYTES, chunk, waves)
                elif cls == "write":
                    ep.ep_stream(kind, None, a, CEIL_BYTES, chunk, waves)
                else:
                    ep.ep_stream(kind, a, b, CEIL_BYTES, chunk, waves)
            launch(1)
            a0, a1 = hev.create(2)
            torch.cuda.synchronize()
            hev.record(a0, stream)
            for i in range(CEIL_LAUNCHES):
                launch(i)
            hev.record(a1, stream)
            torch.cuda.synchronize()
            moved = CEIL_BYTES * CEIL_LAUNCHES * (2 if cls == "copy" else 1)
            gbs = moved / (hev.ms(a0, a1) * 1e-3) / 1e9
            hev.destroy([a0, a1])
            if name not in best or gbs > best[name]["gbs"]:
                best[name] = {"gbs": round(gbs, 1), "chunk_bytes": chunk, "waves": waves}
    del bufs
    out = {cls: dict(max((best[cls], best[cls + "_nt"]), key=lambda v: v["gbs"]),
                     non_temporal=best[cls + "_nt"]["gbs"] > best[cls]["gbs"]) for cls in ("read", "write", "copy")}
    out["by_kind"] = best
    return out


def mix_ceiling(read_bytes: float, write_bytes: float, ceil: dict) -> float:
    """Ceiling (GB/s) for a call that reads and writes these bytes: the read
    and write streams' rates, each for its share of the bytes, one after the
    other -- the rate of a stream with the same mix if reads and writes cannot
    overlap on the memory bus."""
    t = read_bytes / ceil["read"]["gbs"] + write_bytes / ceil["write"]["gbs"]
    return (read_bytes + write_bytes) / t if t > 0 else 0.0


def host_cores() -> int:
    """Cores this process may use: the CPU share the job was given
    (OMP_NUM_THREADS when set, else the affinity mask)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def _oracle_rate(oracle, inp, seconds):
    reps, t_start = 0, time.perf_counter()
    while True:
        oracle.run_path(inp)
        reps += 1
        if time.perf_counter() - t_start >= seconds:
            break
    return reps, (time.perf_counter() - t_start) / reps


def cpu_baseline(inp, seconds, step_bytes):
    """The CPU oracle as it stands on the same workload: whole passes (layout,
    slots, dispatch rows, expert stage, combine) repeated until `seconds` of
    work, at least one pass; once with one thread, once with the row-level
    calls (dispatch rows, expert stage, combine) split over every core this
    process may use (the oracle's threads() mode: the same C code per token
    block, identical bytes).  The reported value is the all-core one; the
    one-thread figure sits beside it, each with its core count, and one more
    single-thread pass is timed part by part (layout, slots + dispatch rows,
    combine)."""
    import oracle

    cores = host_cores()
    reps1, dt1 = _oracle_rate(oracle, inp, seconds / 2)
    with oracle.threads(cores):
        repsn, dtn = _oracle_rate(oracle, inp, seconds / 2)
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
    return {"value": round(inp["T"] / dtn, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "gbs": round(step_bytes / dtn / 1e9, 3),
            "sample": f"{repsn} full passes of workload {inp['name']} (T={inp['T']}) on {cores} threads, "
                      f"{dtn:.3f} s per pass",
            "single_thread": {"value": round(inp["T"] / dt1, 1), "unit": "tokens/s", "cores": 1,
                              "gbs": round(step_bytes / dt1 / 1e9, 3), "parts": parts,
                              "sample": f"{reps1} full passes, {dt1:.3f} s per pass"}}


if __name__ == "__main__":
    main()
