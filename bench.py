"""Benchmark of the Paged Experts hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode-bf16|...]

A step is one pass of the whole decode hot path over one batch: router ->
slot plan (host sees the plan) -> page-in of the misses (pinned host -> slot,
copy stream) -> expert FFN over the slots (compute stream), for every wave.
Inputs (router logits, hidden states) are resident in HBM before the timed
region; the expert store lives in pinned host memory by design of the method.

Prints one JSON line: the metric value is decode tokens/s; `roofline` is the
dominant kernel's achieved HBM bandwidth measured with HIP events on the
stream it runs on; `cpu_baseline` is the float64 CPU oracle timed on a
bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE decode tok/s at batch 1 (Qwen3-30B-A3B shapes) + achieved HBM GB/s"
HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "expert_weight_paging_amd", "csrc"))):
        with open(os.path.join(ROOT, "expert_weight_paging_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_peaks(torch, dev):
    """Stream-copy HBM rate and pinned host->device rate on this machine."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    hbm = 2 * n * 10 / (time.perf_counter() - t0) / 1e9
    del a, b
    h = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        d.copy_(h, non_blocking=True)
    s.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(s):
        for _ in range(8):
            d.copy_(h, non_blocking=True)
    s.synchronize()
    h2d = 8 * (256 << 20) / (time.perf_counter() - t0) / 1e9
    return {"hbm_copy_read_plus_write_GBps": round(hbm, 1), "h2d_pinned_GBps": round(h2d, 2)}


# ---------------------------------------------------------------- decode workloads

def decode_bench(args, torch, dev):
    import expert_weight_paging_amd as ewp
    import workloads as W
    from workloads import gen

    cfg = W.CONFIGS[2 if args.workload == "decode-bf16" else 3]
    B = args.batch
    rec = ewp.record_bytes(cfg.fmt, cfg.H, cfg.I)
    log("building pinned store: %d experts x %d B" % (cfg.E, rec))
    host = ewp.HostStore(cfg.E, rec)
    gen.expert_store(cfg, out=host.array)
    slots, state = ewp.alloc_layer_buffers(cfg.E, cfg.K, rec, dev)
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    layer = ewp.Layer(cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K, cfg.fmt, host, slots, state,
                      compute, copy, compute)
    plan = ewp.Plan(layer, B)
    total = args.warmup + args.steps
    logits, x = gen.decode_inputs(cfg, B, steps=total)
    lg_d = torch.from_numpy(logits).to(dev)
    x_d = torch.from_numpy(x.view(np.int16)).to(dev)
    out = torch.empty(B, cfg.H, dtype=torch.float32, device=dev)

    def run(t0, n):
        for t in range(t0, t0 + n):
            layer.step(plan, lg_d[t], x_d[t], out)

    run(0, args.warmup)
    torch.cuda.synchronize()
    s0 = layer.stats()
    t0 = time.perf_counter()
    run(args.warmup, args.steps)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    s1 = layer.stats()
    log("timed %d steps in %.3f s" % (args.steps, el))

    # roofline pass: same workload replayed from the start with event timing
    layer.reset()
    layer.timing_enable(True)
    nprof = min(total, 128)
    run(0, nprof)
    torch.cuda.synchronize()
    tm = layer.timing_read()
    layer.timing_enable(False)

    misses = s1["misses"] - s0["misses"]
    refs = s1["refs"] - s0["refs"]
    res = {
        "value": args.steps * B / el,
        "ms_per_step": el / args.steps * 1e3,
        "timing": tm,
        "hits": s1["hits"] - s0["hits"], "misses": misses, "refs": refs,
        "waves": s1["waves"] - s0["waves"],
        "cfg": cfg, "B": B, "rec": rec,
        "logits": logits, "x": x, "host": host,
    }
    plan.close()
    layer.close()
    return res


def cpu_baseline_decode(res, budget_s):
    """The float64 oracle, as it stands, on the first steps of the same workload."""
    from oracle.layer import PagedLayer
    from workloads import gen
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = 1
    cfg, B = res["cfg"], res["B"]
    ref = PagedLayer(np.array(res["host"].array), cfg.fmt, cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K)
    logits, x = res["logits"], res["x"]
    n = 0
    t0 = time.perf_counter()
    while n < logits.shape[0] and (time.perf_counter() - t0) < budget_s:
        ref.step(logits[n], gen.bf16_bits_to_f32(x[n]).astype(np.float64))
        n += 1
    el = time.perf_counter() - t0
    return {"value": n * B / el, "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": "first %d decode steps (batch %d) of the same workload from a cold table, "
                      "float64 numpy oracle incl. routing, LRU plan, record copies and SwiGLU "
                      "experts, %.1f s" % (n, B, el)}


def traffic_from_profiles(kernel_name, hash_now):
    """HBM bytes per launch from the committed PMC summary, if taken on this source."""
    p = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    k = d.get("kernels", {}).get(kernel_name)
    if not k or d.get("source_hash") != hash_now:
        return None
    return k.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="decode-bf16", choices=["decode-bf16", "decode-fp8"])
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the Paged Experts path is single-GPU and this "
              "build has no multi-GPU mode (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    peaks = None if args.no_peaks else measured_peaks(torch, dev)
    res = decode_bench(args, torch, dev)
    tm = res["timing"]
    cfg = res["cfg"]
    # dominant kernel by measured time
    kinds = [k for k in ("ffn_up", "ffn_down") if tm[k]["count"]]
    dom = max(kinds, key=lambda k: tm[k]["ms"])
    avg_ms = tm[dom]["ms"] / tm[dom]["count"]
    bytes_per_launch = tm[dom]["bytes"] / tm[dom]["count"]
    achieved = bytes_per_launch / (avg_ms * 1e-3) / 1e9
    ffn_bytes = tm["ffn_up"]["bytes"] + tm["ffn_down"]["bytes"]
    ffn_ms = tm["ffn_up"]["ms"] + tm["ffn_down"]["ms"]
    kname = {"ffn_up": "ffn_up_kernel", "ffn_down": "ffn_down_kernel"}[dom]
    traffic = traffic_from_profiles(kname, kernel_source_hash())
    pin = tm["page_in"]
    line = {
        "metric": METRIC,
        "value": round(res["value"], 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {1: "bf16", 2: "fp8"}.get(cfg.fmt, "bf16"),
        "data": "synthetic (seeded; correlated routing p=0.75, weights N(0,0.02))",
        "config": {
            "workload": "one Qwen3-30B-A3B-shaped MoE layer, %s experts, E=%d top_k=%d hidden=%d "
                        "intermediate=%d, K=%d resident slots, decode at batch %d, cold start"
                        % ({1: "bf16", 2: "block-FP8"}[cfg.fmt], cfg.E, cfg.top_k, cfg.H, cfg.I,
                           cfg.K, res["B"]),
            "batch": res["B"], "num_slots": cfg.K, "experts": cfg.E, "top_k": cfg.top_k,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm", "kernel": kname,
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": bytes_per_launch,
        },
        "ffn": {"achieved_GBps": round(ffn_bytes / (ffn_ms * 1e-3) / 1e9, 1),
                "up_us": round(tm["ffn_up"]["ms"] / max(tm["ffn_up"]["count"], 1) * 1e3, 3),
                "down_us": round(tm["ffn_down"]["ms"] / max(tm["ffn_down"]["count"], 1) * 1e3, 3)},
        "page_in": {"GBps": round(pin["bytes"] / max(pin["ms"], 1e-9) / 1e6, 2),
                    "waves_with_copies": pin["count"]},
        "route_us": round(tm["route"]["ms"] / max(tm["route"]["count"], 1) * 1e3, 3),
        "hit_rate": round(res["hits"] / max(res["refs"], 1), 4),
        "misses_per_step": round(res["misses"] / args.steps, 4),
        "measured_peaks": peaks,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (budget %.0f s)" % args.cpu_budget)
        line["cpu_baseline"] = cpu_baseline_decode(res, args.cpu_budget)
    res["host"].free()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
