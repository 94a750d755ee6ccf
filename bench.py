#!/usr/bin/env python3
"""Benchmark of the fused MXFP4 MoE hot path on one MI355X.

One step = the whole path over one batch: moe_sort (routing sort) -> moe_quant_act (fp8 / fp4
workloads only) -> moe_fused (Stage1 + Stage2 + combine, one launch per stage).  Inputs
(weights, activations and a set of rotating routings) are resident in HBM before timing starts;
consecutive steps use different routings so the experts they touch change and the weight stream
is not served from the last-level cache.  Per workload it also measures:

* each part alone over the same rotating routings (moe_fused over pre-sorted layouts, the sort,
  the quantization) and the two stage calls (Stage1; Stage2 + combine), timed with HIP events
  on the stream the library launches on (torch's current stream), each timed pass preceded by
  about 20 ms of untimed calls so that it measures the steady state;
* moe_fused replayed from a HIP graph of N calls over the rotating layouts, median of 3;
* the roofline of its dominant kernel: algorithmic bytes (HBM-bound workloads) or flops
  (MFMA-bound ones) per launch over that stage call's average time;
* the oracle on the host (float64 NumPy) on a bounded sample, scaled to one call.

Prints one JSON line.  `value` is the headline workload's µs per step.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dec-1] [--no-tiers]
                  [--no-cpu-baseline]
  python bench.py --counter-probe            launches for the rocprofv3 --pmc passes
  python bench.py --counter-summarize FETCH_DIR WRITE_DIR MFMA_DIR   -> profiles/counters.json
"""
import argparse
import hashlib
import json
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "fused MoE µs/call, TFLOP/s and weight GB/s (% roofline) at 1/256/8192 tokens"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}   # dense; fp8 x fp4 at the fp8 rate
# the pages' us1 + us2 (Stage1 + Stage2 kernels, no sort) at the shape 3584 x 384, 896 experts,
# top-16 on gfx950 (github ROCm/aiter PR 4463 "Performance"): context, not this metric's scope
PAGES_US = {"dec-1": 28.3, "dec-4": 42.7, "dec-16": 107.3, "mid-64": 229.1, "mid-256": 329.8, "mid-1024": 365.7,
            "pre-a16-2048": 651.3, "pre-a16-4096": 1087.3, "pre-a16-8192": 1994.4, "pre-a16-16384": 3600.3,
            "pre-a8-8192": 1249.4}
WARM_MS = 20.0   # untimed device work between the spin gate and each timed pass
TIERS = ["dec-4", "dec-16", "mid-64", "mid-256", "mid-1024", "ep-8192", "pre-16384", "pre-a16-2048",
         "pre-a16-4096", "pre-a16-8192", "pre-a16-16384", "pre-a8-8192"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of every HIP source and header: a counter record is valid only for the code it measured."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_moe_expert_sort_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    with open(os.path.join(ROOT, "include", "moe_mi355x.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def per_expert_bytes(D, I):
    w1 = 2 * I * (D // 2) + 2 * I * (D // 32)
    w2 = D * (I // 2) + D * (I // 32)
    return w1, w2


def act_bytes(a_dtype, cols):
    return {"bf16": 2 * cols, "fp8": cols + cols // 32, "fp4": cols // 2 + cols // 32}[a_dtype]


def routing_stats(wl, ids):
    """Algorithmic work of one call on one routing: the quantities the roofline divides.
    Weight bytes count each touched expert once; activation rows are read once, the
    intermediate written once and read once, each routed row's Stage2 output written once and
    read once by the combine (bf16), the output written once."""
    D, I, E = wl.model_dim, wl.inter_dim, wl.experts
    local = (ids >= 0) & (ids < E)
    rows = int(local.sum())
    touched = int(np.unique(ids[local]).size)
    w1b, w2b = per_expert_bytes(D, I)
    x_b = wl.tokens * act_bytes(wl.a_dtype, D)
    inter_b = rows * act_bytes(wl.a_dtype, I)
    rowout_b = rows * D * 2
    out_b = wl.tokens * D * 2
    return {"rows": rows, "touched": touched, "weight_bytes": touched * (w1b + w2b),
            "flops": 6.0 * rows * D * I, "stage1_flops": 4.0 * rows * D * I, "stage2_flops": 2.0 * rows * D * I,
            "stage1_bytes": touched * w1b + x_b + inter_b,
            "stage2_bytes": touched * w2b + inter_b + 2 * rowout_b + out_b,
            "fused_bytes": touched * (w1b + w2b) + x_b + 2 * inter_b + 2 * rowout_b + out_b}


class Workbench:
    """Device-resident inputs and preallocated buffers of one workload."""

    def __init__(self, wl, n_routings, weights_d):
        import torch
        import quantized_moe_expert_sort_amd as qm
        from quantized_moe_expert_sort_amd import inputs as gen
        self.wl, self.qm, self.torch, self.gen = wl, qm, torch, gen
        self.w = weights_d
        self.routings, self.stats, self.host = [], [], []
        D, I, K, E = wl.model_dim, wl.inter_dim, wl.topk, wl.experts
        for r in range(n_routings):
            p = gen.make_problem(wl, routing_seed=r, with_weights=False)
            self.stats.append(routing_stats(wl, p["topk_ids"]))
            self.host.append(p)
            x = torch.from_numpy(p["x"].view(np.int16)).cuda()
            self.routings.append((x, torch.from_numpy(p["topk_ids"]).cuda(), torch.from_numpy(p["topk_w"]).cuda()))
        T, bm = wl.tokens, wl.block_m
        self.layout = qm.MoeLayout(T, K, E, bm, with_weights=False)
        self.sort_ws = torch.empty(max(qm.sort_ws_bytes(T, K, E), 1), dtype=torch.uint8, device="cuda")
        d = qm.DTYPES[wl.a_dtype]
        self.fused_ws = torch.empty(qm.fused_ws_bytes(T, D, I, self.layout.cap, bm, d, qm.ACT_SITUV2),
                                    dtype=torch.uint8, device="cuda")
        self.out = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
        if wl.a_dtype != "bf16":
            self.q = torch.empty((T, D if wl.a_dtype == "fp8" else D // 2), dtype=torch.uint8, device="cuda")
            self.qs = torch.empty((T, D // 32), dtype=torch.uint8, device="cuda")
        self.per = None

    def step(self, i):
        """One pass of the whole path on routing i: sort, activation quant, fused operator."""
        qm, wl, gen = self.qm, self.wl, self.gen
        x, ids, w = self.routings[i % len(self.routings)]
        qm.moe_sort(ids, None, 0, wl.experts, wl.block_m, with_weights=False, layout=self.layout, ws=self.sort_ws)
        if wl.a_dtype == "bf16":
            xa, xs = x, None
        else:
            xa, xs = qm.moe_quant_act(x, wl.a_dtype, self.q, self.qs)
        qm.moe_fused(xa, xs, wl.a_dtype, *self.w, w, self.layout, wl.experts, "situv2", gen.BETA,
                     gen.LINEAR_BETA, out=self.out, ws=self.fused_ws)

    def prepare_stages(self):
        """Per-routing sorted layouts, quantized activations and workspaces, so that one stage can
        be launched back to back over rotating routings."""
        torch, qm, wl = self.torch, self.qm, self.wl
        self.per = []
        for x, ids, w in self.routings:
            lay = qm.moe_sort(ids, None, 0, wl.experts, wl.block_m, with_weights=False)
            xa, xs = (x, None) if wl.a_dtype == "bf16" else qm.moe_quant_act(x, wl.a_dtype)
            ws = torch.empty_like(self.fused_ws)
            self.per.append((xa, xs, w, lay, ws))
        torch.cuda.synchronize()

    def stage(self, i, stages):
        gen = self.gen
        xa, xs, w, lay, ws = self.per[i % len(self.per)]
        self.qm.moe_fused(xa, xs, self.wl.a_dtype, *self.w, w, lay, self.wl.experts, "situv2", gen.BETA,
                          gen.LINEAR_BETA, out=self.out, ws=ws, stages=stages)

    def device_ms(self, fn, steps, start, warm_ms=WARM_MS):
        """Device time per call of fn(i), i = start .. start+steps-1.  The calls are enqueued behind
        a spin kernel so that the GPU runs them back to back (as under graph replay or any launcher
        that stays ahead of the device) rather than waiting on Python between launches; if the spin
        ends before the host has enqueued everything, it is lengthened and the pass repeated.
        Untimed calls worth about warm_ms of device time run between the spin and the timed calls:
        after the near-idle spin the heavy kernels run up to ~25% slower for the next ~10 ms (a
        clock / power transient seen in kernel traces), which would otherwise be timed."""
        torch = self.torch
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        host = time.perf_counter()
        for i in range(steps):
            fn(start + i)
        torch.cuda.synchronize()
        host_ms = (time.perf_counter() - host) * 1e3
        warm = int(min(max(2, np.ceil(warm_ms * steps / max(host_ms, 1e-3))), 50 * steps))
        spin_ms = max(5.0, 3.0 * host_ms * (warm + steps) / steps)
        for _ in range(4):
            gate = torch.cuda.Event()
            torch.cuda._sleep(int(spin_ms * self.cyc_per_ms))
            gate.record()
            for i in range(warm):
                fn(start - warm + i)
            t0.record()
            for i in range(steps):
                fn(start + i)
            t1.record()
            starved = gate.query()
            torch.cuda.synchronize()
            if not starved:
                break
            spin_ms *= 3
        return t0.elapsed_time(t1) / steps, host_ms / steps, bool(starved)

    def graph_ms(self, n_calls, repeats=3):
        """moe_fused replayed from one HIP graph of n_calls calls over the rotating pre-sorted
        layouts: median over `repeats` replays of the replay time / n_calls."""
        torch, qm = self.torch, self.qm
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(min(n_calls, 3)):
                self.stage(i, qm.STAGE_ALL)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n_calls):
                self.stage(i, qm.STAGE_ALL)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(repeats):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) / n_calls)
        del g
        return float(np.median(times)), [round(t * 1e3, 3) for t in times]

    def sort_only(self, i):
        wl = self.wl
        _, ids, _ = self.routings[i % len(self.routings)]
        self.qm.moe_sort(ids, None, 0, wl.experts, wl.block_m, with_weights=False, layout=self.layout,
                         ws=self.sort_ws)

    def quant_only(self, i):
        x, _, _ = self.routings[i % len(self.routings)]
        self.qm.moe_quant_act(x, self.wl.a_dtype, self.q, self.qs)

    def run(self, steps, warmup, graph_calls):
        torch, qm = self.torch, self.qm
        self.cyc_per_ms = spin_cycles_per_ms()
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        ms, host_ms, starved = self.device_ms(self.step, steps, warmup)
        self.prepare_stages()
        for i in range(warmup):
            self.stage(i, qm.STAGE_ALL)
        fz, _, stf = self.device_ms(lambda i: self.stage(i, qm.STAGE_ALL), steps, 0)
        s1, _, st1 = self.device_ms(lambda i: self.stage(i, qm.STAGE_1), steps, 0)
        s2, _, st2 = self.device_ms(lambda i: self.stage(i, qm.STAGE_2), steps, 0)
        so, _, sts = self.device_ms(self.sort_only, steps, 0)
        qa, stq = 0.0, False
        if self.wl.a_dtype != "bf16":
            qa, _, stq = self.device_ms(self.quant_only, steps, 0)
        gms, greps = self.graph_ms(graph_calls)
        # the stage statistics of the routings the timed calls used
        idx = [(warmup + i) % len(self.routings) for i in range(steps)]
        st = [self.stats[j] for j in idx]
        mean = lambda k: float(np.mean([s[k] for s in st]))
        r = {k: mean(k) for k in st[0]}
        r.update({"ms_per_step": ms, "host_ms_per_step": host_ms,
                  "host_bound": bool(starved or stf or st1 or st2 or sts or stq),
                  "fused_ms": fz, "stage1_ms": s1, "stage2_ms": s2, "sort_ms": so, "quant_ms": qa,
                  "graph_ms": gms, "graph_calls": graph_calls, "graph_repeats_us": greps})
        return r


def spin_cycles_per_ms():
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    a.record()
    torch.cuda._sleep(2_000_000)
    b.record()
    torch.cuda.synchronize()
    return 2_000_000 / max(a.elapsed_time(b), 1e-3)


def is_hbm_bound(wl, r):
    """The workload's bound from its own measured work: HBM when streaming the touched weights
    at 8 TB/s takes longer than the flops at the dtype's MFMA peak."""
    return r["weight_bytes"] / (HBM_PEAK_GBPS * 1e9) >= r["flops"] / (MFMA_PEAK_TFLOPS[wl.a_dtype] * 1e12)


# kernels behind each stage call, by path: the grouped large-batch path from 2048 tokens when
# model_dim % 512 == 0 (with fp8 / fp4 activations the hot-expert table and token-major Stage2
# are launched before the grouped Stage2, which keeps a group's rows in LDS up to inter_dim
# 384); Stage2 and the combine in one kernel for at most 32 routed rows
def stage_kernels(wl):
    grouped = wl.tokens >= 2048 and wl.block_m == 32 and wl.model_dim % 512 == 0
    if grouped:
        s2 = "grouped_stage2_res_kernel" if wl.inter_dim <= 384 else "grouped_stage2_kernel"
        hot = ["hot_table_kernel", "hot_stage2_kernel"] if wl.a_dtype != "bf16" else []
        return (["group_kernel", "grouped_stage1_kernel"], hot + [s2, "combine_kernel"])
    if wl.tokens * wl.topk <= 32:
        return (["stage1_kernel"], ["stage2_small_kernel"])
    return (["stage1_kernel"], ["stage2_kernel", "combine_kernel"])


def roofline(wl, r, traffic_key=None):
    """Roofline of the dominant stage call (the longer of Stage1 and Stage2 + combine)."""
    hbm = is_hbm_bound(wl, r)
    k1, k2 = stage_kernels(wl)
    if r["stage1_ms"] >= r["stage2_ms"]:
        ks, ms, by, fl = k1, r["stage1_ms"], r["stage1_bytes"], r["stage1_flops"]
    else:
        ks, ms, by, fl = k2, r["stage2_ms"], r["stage2_bytes"], r["stage2_flops"]
    if hbm:
        a = by / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBPS, 4), "per_launch_bytes": round(by)}
    else:
        peak = MFMA_PEAK_TFLOPS[wl.a_dtype]
        a = fl / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(a, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(a / peak, 4), "per_launch_flops": round(fl)}
    roof["kernel"] = " + ".join(ks)
    roof["launch_us"] = round(ms * 1e3, 3)
    # HBM bytes of the call's kernels from the committed counter record (null unless every one
    # of them was measured on this source)
    recs = [counter_record(f"{k}:{wl.name}") for k in ks]
    tr = [None if x is None else x.get("hbm_bytes_per_launch") for x in recs]
    roof["traffic"] = None if any(t is None for t in tr) else int(sum(tr))
    busy = {k: x["mfma_util"] for k, x in zip(ks, recs) if x is not None and x.get("mfma_util") is not None}
    if busy:
        roof["mfma_busy_counter"] = busy     # MFMA-busy share of SIMD cycles, per kernel of the call
    return roof


def summarize(wl, r):
    fz = r["fused_ms"]
    tflops = r["flops"] / (fz * 1e-3) / 1e12
    gbps = r["weight_bytes"] / (fz * 1e-3) / 1e9
    peak_t = MFMA_PEAK_TFLOPS[wl.a_dtype]
    k1, k2 = stage_kernels(wl)
    s = {"us_per_step": round(r["ms_per_step"] * 1e3, 3), "fused_us": round(fz * 1e3, 3),
         "fused_graph_us": round(r["graph_ms"] * 1e3, 3), "graph_calls": r["graph_calls"],
         "graph_replays_us": r["graph_repeats_us"],
         "sort_us": round(r["sort_ms"] * 1e3, 3), "quant_us": round(r["quant_ms"] * 1e3, 3),
         "fused_tflops": round(tflops, 3), "fused_mfma_frac": round(tflops / peak_t, 5),
         "fused_weight_gbps": round(gbps, 1), "fused_weight_hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
         "fused_algorithmic_gbps": round(r["fused_bytes"] / (fz * 1e-3) / 1e9, 1),
         "stage_calls_us": {" + ".join(k1): round(r["stage1_ms"] * 1e3, 3),
                            " + ".join(k2): round(r["stage2_ms"] * 1e3, 3)},
         "bound": "hbm" if is_hbm_bound(wl, r) else "mfma",
         "touched_experts": round(r["touched"], 1), "routed_rows": round(r["rows"], 1),
         "eager_host_us_per_step": round(r["host_ms_per_step"] * 1e3, 3), "host_bound": r["host_bound"],
         "roofline": roofline(wl, r)}
    if wl.name in PAGES_US:
        s["pages_fused_us_context"] = PAGES_US[wl.name]
    return s


# ---------------------------------------------------------------------------------- counters

COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
COPY_PROBE_BYTES = 1 << 30      # elementwise float32 negation of 1 GiB: reads and writes 1 GiB
# (workload, stage call) pairs launched by --counter-probe: the headline's dominant kernel and
# those of the largest tiers
PROBES = [(w, st) for w in ("dec-1", "dec-4", "dec-16", "mid-256", "mid-1024", "pre-16384", "pre-a8-8192",
                            "pre-a16-8192", "ep-8192") for st in (1, 2)]
KERNEL_KEYS = ("grouped_stage1_kernel", "grouped_stage2_res_kernel", "grouped_stage2_kernel", "hot_stage2_kernel",
               "hot_table_kernel", "stage2_small_kernel", "stage2_kernel",
               "stage1_kernel", "combine_kernel", "group_kernel")


def counter_record(key):
    """Counter figures per launch of one kernel on one workload ('kernel:workload'), if the
    committed record was taken on this source."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("kernels", {}).get(key)


def counter_probe(n_launch=12):
    """Launches for the counter passes: the copy probe (3 launches, known bytes) and n_launch
    calls of each PROBES stage over pre-sorted rotating layouts, one workload after another."""
    import torch
    import quantized_moe_expert_sort_amd as qm
    from quantized_moe_expert_sort_amd import inputs as gen
    torch.cuda.set_device(0)
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    weights = {}
    order = []
    for name, stage in PROBES:
        if name not in order:
            order.append(name)
    for name in order:
        wl = gen.WORKLOADS[name]
        key = (wl.experts, wl.inter_dim)
        if key not in weights:
            weights.clear()
            torch.cuda.empty_cache()
            weights[key] = qm.device_weights(*gen.make_weights(wl.seed, wl.experts, wl.model_dim, wl.inter_dim))
        wb = Workbench(wl, 64 if wl.tokens <= 16 else 4, weights[key])
        wb.prepare_stages()
        for stage in (1, 2):
            if (name, stage) not in PROBES:
                continue
            if stage == 2:   # Stage2 reads the intermediate each layout's Stage1 left in its workspace
                for i in range(len(wb.per)):
                    wb.stage(i, qm.STAGE_1)
                torch.cuda.synchronize()
            # a marker launch between workloads and stages: the summary splits the trace there
            torch.cuda._sleep(1000 + 1000 * len(order) * 2 + 100 * stage)
            for i in range(n_launch):
                wb.stage(i, qm.STAGE_1 if stage == 1 else qm.STAGE_2)
            torch.cuda.synchronize()
            log(f"counter probe: {n_launch} stage-{stage} calls of {name}")
        del wb
        torch.cuda.empty_cache()


def counter_summarize(fetch_dir, write_dir, mfma_dir):
    """Counter figures per kernel launch from the passes over the probe (FETCH_SIZE, WRITE_SIZE
    in KiB per dispatch, each scaled by what the same counter reads for the copy probe of known
    size; MfmaUtil, the MFMA-busy share of all SIMD cycles).  Writes profiles/counters.json and
    returns a markdown table."""
    import csv
    import glob

    def rows_of(d):
        out = []
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            out.extend(csv.DictReader(open(f)))
        return out

    def per_dispatch(rows):
        """{dispatch id: (kernel name, {counter: value})} in dispatch order."""
        disp = {}
        for r in rows:
            did = int(r.get("Dispatch_Id", r.get("Correlation_Id", 0)))
            k, c = r["Kernel_Name"], r["Counter_Name"]
            disp.setdefault(did, [k, {}])[1][c] = disp.get(did, [k, {}])[1].get(c, 0.0) + float(r["Counter_Value"])
        return [disp[d] for d in sorted(disp)]

    def attribute(seq):
        """Tag each dispatch with (workload, stage) from the marker sleeps between probe blocks."""
        order = []
        for name, _ in PROBES:
            if name not in order:
                order.append(name)
        tagged, blocks = [], [(n, s) for n in order for s in (1, 2) if (n, s) in PROBES]
        bi = -1
        for k, cs in seq:
            if "sleep" in k.lower() or "spin" in k.lower():
                bi += 1
                continue
            if bi >= 0 and bi < len(blocks):
                tagged.append((blocks[bi], k, cs))
            elif "neg" in k.lower():
                tagged.append((("copy", 0), k, cs))
        return tagged

    def kernel_key(k):
        for kk in KERNEL_KEYS:
            if kk in k:
                return kk
        return None

    res = {}
    factors = {}
    for d, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        tagged = attribute(per_dispatch(rows_of(d)))
        copy = [cs[counter] for (b, k, cs) in tagged if b[0] == "copy"]
        factor = (COPY_PROBE_BYTES / 1024.0) / float(np.median(copy))
        factors[counter] = (float(np.median(copy)), factor)
        for (b, k, cs) in tagged:
            kk = kernel_key(k)
            if b[0] == "copy" or kk is None:
                continue
            res.setdefault(f"{kk}:{b[0]}", {}).setdefault(counter, []).append(cs[counter] * 1024.0 * factor)
    for (b, k, cs) in attribute(per_dispatch(rows_of(mfma_dir))):
        kk = kernel_key(k)
        if b[0] == "copy" or kk is None or "MfmaUtil" not in cs:
            continue
        # MfmaUtil: summed SQ_VALU_MFMA_BUSY_CYCLES over (GRBM_GUI_ACTIVE x SIMDs), in percent
        res.setdefault(f"{kk}:{b[0]}", {}).setdefault("mfma_util", []).append(cs["MfmaUtil"] / 100.0)
    kernels = {}
    lines = [f"copy probe ({COPY_PROBE_BYTES >> 20} MiB read + written): FETCH_SIZE {factors['FETCH_SIZE'][0]:.0f} KiB "
             f"-> factor {factors['FETCH_SIZE'][1]:.4f}; WRITE_SIZE {factors['WRITE_SIZE'][0]:.0f} KiB -> factor "
             f"{factors['WRITE_SIZE'][1]:.4f}", "",
             "| kernel:workload | launches | fetch bytes/launch | write bytes/launch | HBM bytes/launch | MFMA busy (of SIMD cycles) |",
             "|---|---|---|---|---|---|"]
    for key in sorted(res):
        v = res[key]
        f = float(np.mean(v["FETCH_SIZE"])) if "FETCH_SIZE" in v else None
        w = float(np.mean(v["WRITE_SIZE"])) if "WRITE_SIZE" in v else None
        m = float(np.mean(v["mfma_util"])) if "mfma_util" in v else None
        kernels[key] = {"fetch_bytes_per_launch": None if f is None else round(f),
                        "write_bytes_per_launch": None if w is None else round(w),
                        "hbm_bytes_per_launch": None if f is None or w is None else round(f + w),
                        "mfma_util": None if m is None else round(m, 4),
                        "launches": max(len(x) for x in v.values())}
        fmt = lambda x: "—" if x is None else f"{x:,.0f}"
        lines.append(f"| {key} | {kernels[key]['launches']} | {fmt(f)} | {fmt(w)} | "
                     f"{fmt(None if f is None or w is None else f + w)} | {'—' if m is None else f'{m:.3f}'} |")
    rec = {"source_hash": kernel_source_hash(),
           "copy_factor_fetch": round(factors["FETCH_SIZE"][1], 5),
           "copy_factor_write": round(factors["WRITE_SIZE"][1], 5), "kernels": kernels}
    with open(COUNTERS, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return "\n".join(lines)


def gpu_info():
    """The device's power cap, model and clocks from rocm-smi, run as a child process right after
    the headline's timed passes (the clocks are those of a loaded GPU); None where rocm-smi is
    missing or prints something else.  The power cap matters: the pages saw 15-19% swings from
    it."""
    card = None
    for exe in ("rocm-smi", "/opt/rocm/bin/rocm-smi"):
        try:
            out = subprocess.run([exe, "--showmaxpower", "--showclocks", "--showproductname", "--json"],
                                 capture_output=True, text=True, timeout=30).stdout
            card = next(iter(json.loads(out).values()))
            break
        except Exception:
            continue
    if not isinstance(card, dict):
        return None
    keys = {"power_cap_w": "Max Graphics Package Power (W)", "sclk": "sclk clock speed:",
            "mclk": "mclk clock speed:", "gfx": "GFX Version", "model": "Card Model"}
    info = {k: card.get(v) for k, v in keys.items() if v in card}
    try:
        import torch
        info["name"] = torch.cuda.get_device_properties(0).name
    except Exception:
        pass
    return info or None


# ---------------------------------------------------------------------------------- oracle

def cpu_info():
    model = platform.processor() or "unknown"
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except Exception:
        avail = os.cpu_count() or 1
    try:
        import threadpoolctl
        blas = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        blas = 1
    return model, avail, blas


def cpu_oracle_call_us(wl, weights_host, problem, max_experts, budget_s):
    """The oracle (routing sort + fused operator, float64) on one routing, estimated from a
    bounded sample.  The expert-major oracle's work per touched expert is the dequantization of
    its weights (the same for every expert) plus work proportional to its routed rows; both are
    timed on up to max_experts touched experts spread over the touched set (each on the tokens
    routed to it), and the call is estimated as sort (in full) + activation encoding (on up to 512
    token rows, scaled to all tokens) + touched x dequantization + routed rows x per-row time.
    Returns (µs per call, sampled experts, touched experts)."""
    from oracle import moe as om
    from quantized_moe_expert_sort_amd import inputs as gen
    ids, w, x = problem["topk_ids"], problem["topk_w"], problem["x"]
    E, T = wl.experts, wl.tokens
    local = (ids >= 0) & (ids < E)
    touched = np.unique(ids[local])
    pick = np.unique(touched[np.linspace(0, len(touched) - 1, min(max_experts, len(touched))).round().astype(int)])
    w1, w1s, w2, w2s = weights_host
    t0 = time.perf_counter()
    om.sort_layout(ids, 0, E, wl.block_m)
    t_sort = time.perf_counter() - t0
    nx = min(T, 512)
    t0 = time.perf_counter()
    om.activation_values(x[:nx], wl.a_dtype)
    t_act = (time.perf_counter() - t0) * T / nx
    t_deq, t_rows, n_rows, n = 0.0, 0.0, 0, 0
    for e in pick:
        toks = np.nonzero((ids == e).any(axis=1))[0]
        t0 = time.perf_counter()
        om.expert_weights(w1, w1s, w2, w2s, int(e))
        t1 = time.perf_counter()
        om.moe_fused(x[toks], wl.a_dtype, w1[e:e + 1], w1s[e:e + 1], w2[e:e + 1], w2s[e:e + 1], ids[toks], w[toks],
                     int(e), 1, "situv2", gen.BETA, gen.LINEAR_BETA)
        t2 = time.perf_counter()
        t_deq += t1 - t0
        t_rows += max(0.0, (t2 - t1) - (t1 - t0))
        n_rows += int((ids[toks] == e).sum())
        n += 1
        if t2 - t0 + t_deq >= budget_s:
            break
    est = t_sort + t_act + len(touched) * t_deq / n + int(local.sum()) * t_rows / max(n_rows, 1)
    return est * 1e6, n, len(touched)


def cpu_baseline(wl, weights_host, problems, budget_s=12.0):
    """The oracle on the host on whole calls of the headline workload (inputs generated before
    the clock starts), as many calls as fit the budget (at least 3), median per call."""
    from oracle import moe as om
    from quantized_moe_expert_sort_amd import inputs as gen
    model, avail, blas = cpu_info()
    times = []
    t_all = time.perf_counter()
    for i, p in enumerate(problems):
        t0 = time.perf_counter()
        om.sort_layout(p["topk_ids"], 0, wl.experts, wl.block_m)
        om.moe_fused(p["x"], wl.a_dtype, *weights_host, p["topk_ids"], p["topk_w"], 0, wl.experts,
                     "situv2", gen.BETA, gen.LINEAR_BETA)
        times.append(time.perf_counter() - t0)
        if len(times) >= 3 and time.perf_counter() - t_all >= budget_s:
            break
    return {"value": round(float(np.median(times)) * 1e6, 1), "unit": "us/call", "cores": int(blas),
            "kind": "oracle",
            "sample": f"{wl.name}: {len(times)} whole calls (routings 0..{len(times) - 1}; median), routing sort + "
                      f"fused operator in float64 NumPy; matrix products on {blas} BLAS threads, the rest on one "
                      f"thread; host {model}, {avail} cores available"}


# ---------------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dec-1")
    ap.add_argument("--routings", type=int, default=64)
    ap.add_argument("--tiers", default=",".join(TIERS), help="comma-separated tier workloads")
    ap.add_argument("--no-tiers", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counter-probe", action="store_true",
                    help="only the launches for the counter passes (run under rocprofv3 --pmc)")
    ap.add_argument("--counter-summarize", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "MFMA_DIR"),
                    help="turn the three counter passes into profiles/counters.json (no GPU needed)")
    args = ap.parse_args()
    if args.counter_summarize:
        print(counter_summarize(*args.counter_summarize))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "multi-GPU expert/tensor-parallel sharding is not part of this build", file=sys.stderr)
        sys.exit(2)
    if args.counter_probe:
        counter_probe()
        return

    import torch
    import quantized_moe_expert_sort_amd as qm
    from quantized_moe_expert_sort_amd import inputs as gen
    torch.cuda.set_device(0)
    wl = gen.WORKLOADS[args.workload]
    weights = {}

    def weights_for(w):
        key = (w.seed, w.experts, w.model_dim, w.inter_dim)
        if key not in weights:
            weights.clear()
            torch.cuda.empty_cache()
            log(f"generating weights E={w.experts} D={w.model_dim} I={w.inter_dim}")
            host = gen.make_weights(w.seed, w.experts, w.model_dim, w.inter_dim)
            weights[key] = (host, qm.device_weights(*host))
        return weights[key]

    host, dev_w = weights_for(wl)
    log(f"workload {wl.name}: preparing {args.routings} routings")
    wb = Workbench(wl, args.routings, dev_w)
    log(f"timing {args.steps} steps after {args.warmup} warmup")
    r = wb.run(args.steps, args.warmup, graph_calls=200)
    gpu = gpu_info()
    s = summarize(wl, r)
    log(f"{wl.name}: {s}")
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(wl, host, wb.host)
    del wb
    torch.cuda.empty_cache()

    tiers = {}
    if not args.no_tiers:
        names = [n for n in args.tiers.split(",") if n and n != wl.name]
        # workloads sharing a weight set run together (the weights are generated once per set)
        names.sort(key=lambda n: (gen.WORKLOADS[n].inter_dim, gen.WORKLOADS[n].experts) != (wl.inter_dim, wl.experts))
        for name in names:
            t = gen.WORKLOADS[name]
            thost, tw = weights_for(t)
            nr = 64 if t.tokens <= 16 else (16 if t.tokens <= 1024 else 4)
            log(f"tier {name}: {nr} routings")
            tb = Workbench(t, nr, tw)
            tr = tb.run(max(20, args.steps // 4), 5, graph_calls=200 if t.tokens <= 1024 else 20)
            tiers[name] = summarize(t, tr)
            if not args.no_cpu_baseline:
                us, n, u = cpu_oracle_call_us(t, thost, tb.host[0], 4 if t.inter_dim > 1024 else 16, 2.0)
                tiers[name]["cpu_oracle_us_per_call"] = round(us, 1)
                tiers[name]["cpu_oracle_sample"] = (f"routing 0: sort in full, activation encoding on "
                                                    f"{min(t.tokens, 512)} rows scaled to {t.tokens}, per-expert "
                                                    f"dequantization and per-row time from {n} of {u} touched "
                                                    f"experts, scaled to {u} experts and all routed rows")
            log(f"{name}: {tiers[name]}")
            del tb
            torch.cuda.empty_cache()

    model, avail, blas = cpu_info()
    line = {
        "metric": METRIC, "value": s["us_per_step"], "unit": "us/call", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 6),
        "higher_is_better": False, "scaling": "weak",
        # the pages time Stage1 + Stage2 kernels only (no sort): not this metric's scope
        "vs_baseline": None,
        "pages_fused_us_context": PAGES_US.get(wl.name),
        "dtype": wl.a_dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name}: tokens={wl.tokens}, experts={wl.experts}, topk={wl.topk}, "
                               f"model_dim={wl.model_dim}, inter_dim={wl.inter_dim}, a_dtype={wl.a_dtype}, "
                               f"weights=mxfp4, SiTUv2 beta={gen.BETA} linear_beta={gen.LINEAR_BETA}, "
                               f"{args.routings} rotating routings",
                   "tokens": wl.tokens, "experts": wl.experts, "topk": wl.topk, "model_dim": wl.model_dim,
                   "inter_dim": wl.inter_dim, "block_m": wl.block_m, "parallelism": "single GPU"},
        "parts_us": {"moe_sort": s["sort_us"], "moe_quant_act": s["quant_us"], "moe_fused": s["fused_us"],
                     "moe_fused_graph_replay": s["fused_graph_us"]},
        "fused_tflops": s["fused_tflops"], "fused_weight_gbps": s["fused_weight_gbps"],
        "fused_weight_hbm_frac": s["fused_weight_hbm_frac"], "fused_mfma_frac": s["fused_mfma_frac"],
        "stage_calls_us": s["stage_calls_us"], "graph_replays_us": s["graph_replays_us"],
        "eager_host_us_per_step": s["eager_host_us_per_step"], "host_bound": s["host_bound"],
        "touched_experts": s["touched_experts"],
        "roofline": s["roofline"], "cpu_baseline": cpu,
        "host_cpu": {"model": model, "cores_available": avail, "blas_threads": blas},
        "gpu": gpu,
        "tiers": tiers,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
