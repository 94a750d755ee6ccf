#!/usr/bin/env python3
"""Benchmark of the fused MXFP4 MoE hot path on one MI355X.

One step = the whole path over one batch: moe_sort (routing sort) -> moe_quant_act (fp8 / fp4
workloads only) -> moe_fused (Stage1 + Stage2 + combine, one launch per stage).  Inputs
(weights, activations and a set of rotating routings) are resident in HBM before timing starts;
consecutive steps use different routings so the experts they touch change and the weight stream
is not served from the last-level cache.  Each part is also timed alone over the same rotating
routings (moe_fused over pre-sorted layouts, the sort, the quantization), and the per-stage
launches (Stage1 alone, Stage2 + combine alone) for reference.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dec-1] [--no-tiers]
                  [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "fused MoE µs/call, TFLOP/s and weight GB/s (% roofline) at 1/256/8192 tokens"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}   # dense; fp8 x fp4 at the fp8 rate
PAGES_US = {("bf16", 1): 28.3}      # a16w4 us1+us2 at 1 token, 3584x384, E=896, top-16 (gfx950)
# the pages' us1 + us2 (Stage1 + Stage2 kernels, no sort) for the tiers of the same shape and
# routing (3584 x 384, all 896 experts, uniform routing): context, not this metric's scope
PAGES_TIER_US = {"dec-4": 42.7, "dec-16": 107.3, "mid-64": 229.1, "mid-256": 329.8, "mid-1024": 365.7,
                 "pre-a16-8192": 1994.4, "pre-a8-8192": 1249.4}
TIERS = ["dec-4", "dec-16", "mid-64", "mid-256", "mid-1024", "ep-8192", "pre-16384", "pre-a16-8192",
         "pre-a8-8192"]


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


class Workbench:
    """Device-resident inputs and preallocated buffers of one workload."""

    def __init__(self, wl, n_routings, weights_d):
        import torch
        import quantized_moe_expert_sort_amd as qm
        from quantized_moe_expert_sort_amd import inputs as gen
        self.wl, self.qm, self.torch = wl, qm, torch
        self.w = weights_d
        self.routings, self.stats = [], []
        D, I, K, E = wl.model_dim, wl.inter_dim, wl.topk, wl.experts
        w1b, w2b = per_expert_bytes(D, I)
        for r in range(n_routings):
            p = gen.make_problem(wl, routing_seed=r, with_weights=False)
            ids = p["topk_ids"]
            local = (ids >= 0) & (ids < E)
            rows = int(local.sum())
            touched = int(np.unique(ids[local]).size)
            s1 = touched * w1b + wl.tokens * act_bytes(wl.a_dtype, D) + rows * act_bytes(wl.a_dtype, I)
            s2 = touched * w2b + rows * act_bytes(wl.a_dtype, I) + 2 * wl.tokens * D
            fb = touched * (w1b + w2b) + wl.tokens * act_bytes(wl.a_dtype, D) + 2 * wl.tokens * D
            self.stats.append({"rows": rows, "touched": touched, "weight_bytes": touched * (w1b + w2b),
                               "flops": 6.0 * rows * D * I, "stage1_bytes": s1, "stage2_bytes": s2,
                               "fused_bytes": fb})
            x = torch.from_numpy(p["x"].view(np.int16)).cuda()
            self.routings.append((x, torch.from_numpy(ids).cuda(), torch.from_numpy(p["topk_w"]).cuda()))
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

    def step(self, i):
        """One pass of the whole path on routing i: sort, activation quant, fused operator."""
        from quantized_moe_expert_sort_amd import inputs as gen
        qm, wl = self.qm, self.wl
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
        from quantized_moe_expert_sort_amd import inputs as gen
        xa, xs, w, lay, ws = self.per[i % len(self.per)]
        self.qm.moe_fused(xa, xs, self.wl.a_dtype, *self.w, w, lay, self.wl.experts, "situv2", gen.BETA,
                          gen.LINEAR_BETA, out=self.out, ws=ws, stages=stages)

    def device_ms(self, fn, steps, start):
        """Device time per call of fn(i), i = start .. start+steps-1.  The calls are enqueued behind
        a spin kernel so that the GPU runs them back to back (as under graph replay or any launcher
        that stays ahead of the device) rather than waiting on Python between launches; if the spin
        ends before the host has enqueued everything, it is lengthened and the pass repeated."""
        torch = self.torch
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        host = time.perf_counter()
        for i in range(steps):
            fn(start + i)
        torch.cuda.synchronize()
        host_ms = (time.perf_counter() - host) * 1e3
        spin_ms = max(5.0, 3.0 * host_ms)
        for _ in range(4):
            gate = torch.cuda.Event()
            torch.cuda._sleep(int(spin_ms * self.cyc_per_ms))
            gate.record()
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

    def sort_only(self, i):
        wl = self.wl
        _, ids, _ = self.routings[i % len(self.routings)]
        self.qm.moe_sort(ids, None, 0, wl.experts, wl.block_m, with_weights=False, layout=self.layout,
                         ws=self.sort_ws)

    def quant_only(self, i):
        x, _, _ = self.routings[i % len(self.routings)]
        self.qm.moe_quant_act(x, self.wl.a_dtype, self.q, self.qs)

    def run(self, steps, warmup):
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
        idx = [(warmup + i) % len(self.routings) for i in range(steps)]
        st = [self.stats[j] for j in idx]
        mean = lambda k: float(np.mean([s[k] for s in st]))
        return {"ms_per_step": ms, "host_ms_per_step": host_ms,
                "host_bound": bool(starved or stf or st1 or st2 or sts or stq),
                "fused_ms": fz, "stage1_ms": s1, "stage2_ms": s2, "sort_ms": so, "quant_ms": qa,
                "weight_bytes": mean("weight_bytes"), "flops": mean("flops"), "rows": mean("rows"),
                "touched": mean("touched"), "stage1_bytes": mean("stage1_bytes"),
                "stage2_bytes": mean("stage2_bytes"), "fused_bytes": mean("fused_bytes"),
                "stage1_gbps": mean("stage1_bytes") / (s1 * 1e-3) / 1e9,
                "stage2_gbps": mean("stage2_bytes") / (s2 * 1e-3) / 1e9}


def spin_cycles_per_ms():
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    a.record()
    torch.cuda._sleep(2_000_000)
    b.record()
    torch.cuda.synchronize()
    return 2_000_000 / max(a.elapsed_time(b), 1e-3)


def summarize(wl, r):
    us = r["ms_per_step"] * 1e3
    fz = r["fused_ms"]
    tflops = r["flops"] / (fz * 1e-3) / 1e12
    gbps = r["weight_bytes"] / (fz * 1e-3) / 1e9
    peak_t = MFMA_PEAK_TFLOPS[wl.a_dtype]
    return {"us_per_step": round(us, 3), "fused_us": round(fz * 1e3, 3), "sort_us": round(r["sort_ms"] * 1e3, 3),
            "quant_us": round(r["quant_ms"] * 1e3, 3),
            "fused_tflops": round(tflops, 3), "fused_weight_gbps": round(gbps, 1),
            "fused_weight_hbm_frac": round(gbps / HBM_PEAK_GBPS, 4), "fused_mfma_frac": round(tflops / peak_t, 5),
            "per_stage_launches_us": {"stage1": round(r["stage1_ms"] * 1e3, 3),
                                      "stage2_and_combine": round(r["stage2_ms"] * 1e3, 3)},
            "touched_experts": round(r["touched"], 1), "routed_rows": round(r["rows"], 1),
            "eager_host_us_per_step": round(r["host_ms_per_step"] * 1e3, 3), "host_bound": r["host_bound"]}


def traffic_record(kernel):
    """HBM bytes per launch from the committed counter summary, if it matches this source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("kernels", {}).get(kernel)


COPY_PROBE_BYTES = 1 << 30      # elementwise float32 negation of 1 GiB: reads and writes 1 GiB


def traffic_probe(wl, host_w_dev, n_launch=40):
    """Launches for the counter passes: the copy probe (3 launches, known bytes) and n_launch
    Stage1-only launches of workload wl over pre-sorted rotating layouts."""
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    wb = Workbench(wl, 64, host_w_dev)
    wb.prepare_stages()
    for i in range(n_launch):
        wb.stage(i, wb.qm.STAGE_1)
    torch.cuda.synchronize()
    log(f"traffic probe: 3 copy launches, {n_launch} stage1 launches of {wl.name}")


def traffic_summarize(fetch_dir, write_dir, wl_name):
    """HBM bytes per Stage1 launch from the two counter passes (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch), each scaled by what the same counter reads for the copy probe of known size.
    Writes profiles/traffic.json and returns a markdown table."""
    import csv
    import glob

    def per_kernel(d, counter):
        rows = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                n = r["Kernel_Name"]
                key = "copy" if "neg" in n else ("stage1" if "stage1_kernel" in n else None)
                if key:
                    rows.setdefault(key, []).append(float(r["Counter_Value"]))
        return rows

    out = {}
    lines = ["| counter | copy probe (KiB/launch) | expected (KiB) | factor | stage1 (KiB/launch) | stage1 scaled (bytes/launch) |",
             "|---|---|---|---|---|---|"]
    for d, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        k = per_kernel(d, counter)
        copy_kib = float(np.median(k["copy"]))
        factor = (COPY_PROBE_BYTES / 1024.0) / copy_kib
        s1_kib = float(np.mean(k["stage1"]))
        out[counter] = {"copy_kib": copy_kib, "factor": factor, "stage1_kib": s1_kib,
                        "stage1_bytes": s1_kib * 1024.0 * factor, "stage1_launches": len(k["stage1"])}
        lines.append(f"| {counter} | {copy_kib:.0f} | {COPY_PROBE_BYTES // 1024} | {factor:.4f} | {s1_kib:.1f} | "
                     f"{s1_kib * 1024.0 * factor:.0f} |")
    rec = {"source_hash": kernel_source_hash(),
           "kernels": {f"stage1:{wl_name}": {
               "hbm_bytes_per_launch": round(out["FETCH_SIZE"]["stage1_bytes"] + out["WRITE_SIZE"]["stage1_bytes"]),
               "fetch_bytes_per_launch": round(out["FETCH_SIZE"]["stage1_bytes"]),
               "write_bytes_per_launch": round(out["WRITE_SIZE"]["stage1_bytes"]),
               "copy_factor_fetch": round(out["FETCH_SIZE"]["factor"], 5),
               "copy_factor_write": round(out["WRITE_SIZE"]["factor"], 5)}}}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return "\n".join(lines)


def cpu_baseline(wl, weights_host, budget_s=15.0):
    """The oracle (sort layout + fused operator) on the host, on routings 0, 1, ... until the
    time budget is spent (at least one)."""
    from oracle import moe as om
    from quantized_moe_expert_sort_amd import inputs as gen
    try:
        import threadpoolctl
        cores = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        cores = 1
    n, t0 = 0, time.perf_counter()
    while True:
        p = gen.make_problem(wl, routing_seed=n, with_weights=False)
        om.sort_layout(p["topk_ids"], 0, wl.experts, wl.block_m)
        om.moe_fused(p["x"], wl.a_dtype, *weights_host, p["topk_ids"], p["topk_w"], 0, wl.experts,
                     "situv2", gen.BETA, gen.LINEAR_BETA)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(el / n * 1e6, 1), "unit": "us/call", "cores": int(cores), "kind": "oracle",
            "sample": f"{wl.name}: {n} step(s) (routings 0..{n - 1}), routing sort + fused operator, float64"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dec-1")
    ap.add_argument("--routings", type=int, default=64)
    ap.add_argument("--no-tiers", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only the launches for the HBM-traffic counter passes (run under rocprofv3 --pmc)")
    ap.add_argument("--traffic-summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn the two counter passes into profiles/traffic.json (no GPU needed)")
    args = ap.parse_args()
    if args.traffic_summarize:
        print(traffic_summarize(*args.traffic_summarize, args.workload))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "multi-GPU expert/tensor-parallel sharding is not part of this build", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_moe_expert_sort_amd as qm
    from quantized_moe_expert_sort_amd import inputs as gen
    torch.cuda.set_device(0)
    wl = gen.WORKLOADS[args.workload]
    weights = {}

    def weights_for(w):
        key = (w.seed, w.experts, w.model_dim, w.inter_dim)
        if key not in weights:
            log(f"generating weights E={w.experts} D={w.model_dim} I={w.inter_dim}")
            host = gen.make_weights(w.seed, w.experts, w.model_dim, w.inter_dim)
            weights[key] = (host, qm.device_weights(*host))
        return weights[key]

    host, dev_w = weights_for(wl)
    if args.traffic_probe:
        traffic_probe(wl, dev_w)
        return
    log(f"workload {wl.name}: preparing {args.routings} routings")
    wb = Workbench(wl, args.routings, dev_w)
    log(f"timing {args.steps} steps after {args.warmup} warmup")
    r = wb.run(args.steps, args.warmup)
    s = summarize(wl, r)
    log(f"{wl.name}: {s}")

    # dominant kernel: the Stage1 launch (timed alone over the same pre-sorted rotating layouts)
    bound_hbm = r["weight_bytes"] / (HBM_PEAK_GBPS * 1e9) >= r["flops"] / (MFMA_PEAK_TFLOPS[wl.a_dtype] * 1e12)
    k_ms, k_bytes, k_flops = r["stage1_ms"], r["stage1_bytes"], r["flops"] * (2.0 / 3.0)
    if bound_hbm:
        a = k_bytes / (k_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBPS, 4)}
    else:
        a = k_flops / (k_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(a, 2), "peak": MFMA_PEAK_TFLOPS[wl.a_dtype],
                "unit": "TFLOP/s", "frac": round(a / MFMA_PEAK_TFLOPS[wl.a_dtype], 4)}
    kname = "stage1"
    roof["kernel"] = kname
    roof["per_launch_bytes" if bound_hbm else "per_launch_flops"] = round(k_bytes if bound_hbm else k_flops)
    roof["launch_us"] = round(k_ms * 1e3, 3)
    tr = traffic_record(f"{kname}:{wl.name}")
    roof["traffic"] = None if tr is None else tr.get("hbm_bytes_per_launch")

    tiers = {}
    if not args.no_tiers:
        for name in TIERS:
            if name == wl.name:
                continue
            t = gen.WORKLOADS[name]
            _, tw = weights_for(t)
            nr = 64 if t.tokens <= 16 else (16 if t.tokens <= 1024 else 4)
            log(f"tier {name}: {nr} routings")
            tb = Workbench(t, nr, tw)
            tiers[name] = summarize(t, tb.run(max(20, args.steps // 4), 5))
            if name in PAGES_TIER_US:
                tiers[name]["pages_fused_us_context"] = PAGES_TIER_US[name]
            log(f"{name}: {tiers[name]}")
            del tb
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(wl, host)

    pages = PAGES_US.get((wl.a_dtype, wl.tokens), PAGES_TIER_US.get(wl.name))
    line = {
        "metric": METRIC, "value": s["us_per_step"], "unit": "us/call", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 6),
        "higher_is_better": False, "scaling": "weak",
        # the pages time Stage1 + Stage2 kernels only (no sort): not this metric's scope
        "vs_baseline": None,
        "pages_fused_us_context": pages,
        "dtype": wl.a_dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name}: tokens={wl.tokens}, experts={wl.experts}, topk={wl.topk}, "
                               f"model_dim={wl.model_dim}, inter_dim={wl.inter_dim}, a_dtype={wl.a_dtype}, "
                               f"weights=mxfp4, SiTUv2 beta={gen.BETA} linear_beta={gen.LINEAR_BETA}, "
                               f"{args.routings} rotating routings",
                   "tokens": wl.tokens, "experts": wl.experts, "topk": wl.topk, "model_dim": wl.model_dim,
                   "inter_dim": wl.inter_dim, "block_m": wl.block_m, "parallelism": "single GPU"},
        "parts_us": {"moe_sort": s["sort_us"], "moe_quant_act": s["quant_us"], "moe_fused": s["fused_us"]},
        "fused_tflops": s["fused_tflops"], "fused_weight_gbps": s["fused_weight_gbps"],
        "fused_weight_hbm_frac": s["fused_weight_hbm_frac"], "fused_mfma_frac": s["fused_mfma_frac"],
        "per_stage_launches_us": s["per_stage_launches_us"],
        "eager_host_us_per_step": s["eager_host_us_per_step"], "host_bound": s["host_bound"],
        "touched_experts": s["touched_experts"],
        "roofline": roof, "cpu_baseline": cpu, "tiers": tiers,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
