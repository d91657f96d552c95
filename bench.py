"""Benchmark of the Paged Experts hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [...]

Workloads (synthetic, seeded, Qwen3-30B-A3B shapes: 128 experts, top-8,
hidden 2048, MoE intermediate 768):
  decode-bf16  (default) one bf16 MoE layer, K=40 slots, batch-1 decode,
               correlated routing p=0.75, cold table. A step is one token:
               router -> slot plan -> page-in of the misses (pinned host ->
               slots) -> expert FFN over the slots, every wave.
  decode-fp8   the same layer with block-FP8 experts, --batch B
  decode-mxfp4 the same layer with MXFP4 experts (E2M1 weights, one E8M0
               scale per 32), --batch B
  stack-int4   48 int4 layers, K=92 each, batch-1 decode; a step is one token
               through all 48 layers, each reading the unit-gain RMSNorm of
               the residual stream and adding its output back (bf16); --routing
               uniform for the control run; --lookahead to route/page-in
               layer l+1 while layer l computes
  prefill-bf16 one 2048-token chunk through 48 bf16 layers, K=92, warm
               tables, uniform routing; a step is one chunk
Modes. By default a decode step whose batch fits one wave (B * top_k <= K)
is device-resolved (the plan stays on the GPU, a copy kernel pages the misses
in through the host store's device mapping, no host synchronisation), and a
stack token is one HIP graph of such steps through the 48 layers, replayed
per token. --host forces host-driven steps (the host reads the plan and
issues DMA copies on a copy stream while the resident experts compute);
--device asks for device-resolved steps without the graph. Batches beyond one
wave: --waves expert (default, host-driven expert-partitioned waves) or
--waves token (groups of K // top_k tokens, each a device-resolved step);
--slots K overrides the decode workloads' slot count (the 4-request cliff).
Inputs (router logits, hidden states) are resident in HBM before the timed
region; expert stores live in pinned host memory by design of the method.

Prints ONE JSON line: `value` is tokens/s of the workload; `roofline` is the
dominant kernel's achieved rate over the timed region, from HIP events
recorded on the stream the kernel runs on, against the MI355X peak;
`cpu_baseline` is the float32 CPU oracle timed on a bounded sample, with the
host's core count, CPU model and BLAS library.
For the decode workloads the headline `roofline` is the expert FFN (up and
down kernels together) measured with the caches cold: --cold-layers
independent layers of the same shape taken in turn, so that a layer's experts
have left the 256 MB last-level cache before it runs again; `roofline_warm` is
the same figure on the one layer of the timed steps.
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
DECODE_CONFIG = {"decode-bf16": 2, "decode-fp8": 3, "decode-mxfp4": 6}
FMT_NAME = {0: "f32", 1: "bf16", 2: "fp8", 3: "int4", 4: "mxfp4"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# source file of each kernel whose counters are stored (plus the shared headers)
KERNEL_SOURCE = {"ffn_up_kernel": "ffn_gemv.hip", "ffn_down_kernel": "ffn_gemv.hip",
                 # the bf16-weight instances (second template argument: the weight format)
                 "grouped_gemm_kernel<true,1>": "ffn_gemm.hip", "grouped_gemm_kernel<false,1>": "ffn_gemm.hip",
                 "combine_kernel": "ffn_gemm.hip", "route_plan_small_kernel": "plan.hip",
                 "route_plan_wave_kernel": "plan.hip", "route_plan_page_in_kernel": "plan.hip",
                 "page_in_kernel": "page_in.hip"}


def kernel_source_hash(kernel_name):
    """Hash of the source that defines a kernel and of every shared header: a
    stored traffic figure is used only while these are unchanged."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "expert_weight_paging_amd", "csrc")
    headers = sorted(f for f in os.listdir(d) if f.endswith(".h"))
    for f in [KERNEL_SOURCE[kernel_name]] + headers:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_name, workload):
    """HBM bytes per launch from the committed PMC summary, only if it was taken
    on the current source of that kernel (else null)."""
    p = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    # a graph replays the device-resolved launches unchanged: same bytes per launch
    for key in (workload, workload.replace(" graph", " device")):
        k = d.get("workloads", {}).get(key, {}).get("kernels", {}).get(kernel_name)
        if k and kernel_name in KERNEL_SOURCE and k.get("source_hash") == kernel_source_hash(kernel_name):
            return k.get("bytes_per_launch")
    return None


KERNEL_KEYS = tuple((k, k) for k in KERNEL_SOURCE)


def ingest_pmc(fetch_csv, write_csv, workload):
    """HBM bytes per launch of each of this library's kernels from two
    rocprofv3 --pmc runs of the same bench command (FETCH_SIZE, then
    WRITE_SIZE; KiB per dispatch). Each counter is scaled by the factor that
    maps its reading for the run's 1 GiB device-to-device copy (the copy in
    measured_peaks) onto 1 GiB. Writes profiles/pmc_traffic.json, keyed by the
    hash of the kernel sources, so bench.py drops the figure once a kernel
    changes (each kernel's entry carries the hash of its own source)."""
    import csv
    def load(path, counter):
        per = {}
        calib = []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"])
                name = r["Kernel_Name"]
                if "copyBuffer" in name and v > 256 * 1024:  # the 1 GiB copy (>= 256 MiB read)
                    calib.append(v)
                    continue
                for pat, key in KERNEL_KEYS:  # the kernel's own name, not a longer one ending in it
                    if "::" + pat in name.replace(" ", ""):
                        per.setdefault(key, []).append(v)
        if not calib:
            raise SystemExit("no 1 GiB copy in %s: run the bench without --no-peaks" % path)
        calib.sort()
        return per, (1 << 20) / calib[len(calib) // 2]
    fetch, ff = load(fetch_csv, "FETCH_SIZE")
    write, wf = load(write_csv, "WRITE_SIZE")
    p = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    d = {}
    if os.path.exists(p):
        with open(p) as f:
            d = json.load(f)
    d = {"workloads": d.get("workloads", {})}
    w = {}
    for key in sorted(set(fetch) & set(write)):
        fk = sum(fetch[key]) / len(fetch[key]) * ff
        wk = sum(write[key]) / len(write[key]) * wf
        w[key] = {"bytes_per_launch": round((fk + wk) * 1024.0, 1), "fetch_bytes": round(fk * 1024.0, 1),
                  "write_bytes": round(wk * 1024.0, 1), "launches": len(fetch[key]),
                  "source_hash": kernel_source_hash(key)}
    d["workloads"][workload] = {"kernels": w, "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)}
    with open(p, "w") as f:
        json.dump(d, f, indent=1, sort_keys=True)
    print(json.dumps(d["workloads"][workload], indent=1))


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


def one_launch_read_reference(torch, dev, roof):
    """The FFN launches against a plain one-launch streaming read of the same
    bytes (moe_read_probe: every load issued up front, nothing computed or
    stored), timed by the same dispatch-stamped events, each launch reading
    memory the previous ones did not (a 2 GiB buffer, eight times the
    last-level cache): what one launch of that many cold bytes takes on this
    box, fixed costs included. ratio = the kernels' time over the reads'."""
    import expert_weight_paging_amd as ewp
    buf = torch.zeros(2 << 30, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    out, k_us, r_us = {}, 0.0, 0.0
    for name, v in roof["kernels"].items():
        nb = int(v["algorithmic_bytes_per_launch"]) // 16 * 16
        us = ewp.read_probe(buf, nb, stream=torch.cuda.current_stream())
        out[name] = {"bytes": nb, "read_us": round(us, 3), "kernel_us": v["avg_launch_us"],
                     "ratio": round(v["avg_launch_us"] / us, 3)}
        k_us += v["avg_launch_us"]
        r_us += us
    pair = sum(v["bytes"] for v in out.values())
    out["pair_as_one_read_us"] = round(ewp.read_probe(buf, pair // 16 * 16, stream=torch.cuda.current_stream()), 3)
    out["pair_ratio"] = round(k_us / r_us, 3)
    del buf
    return out


def oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        return 1


def host_info():
    """The host the CPU baseline ran on: cores visible to this process, the CPU
    model and the BLAS library numpy calls (with its thread count)."""
    info = {"nproc": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        info["blas"] = ["%s %s (%s, %d threads)" % (p.get("internal_api"), p.get("version"),
                                                    p.get("threading_layer"), p.get("num_threads", 0))
                        for p in threadpool_info() if p.get("user_api") == "blas"]
    except Exception:
        info["blas"] = None
    return info


def merge_timing(ts):
    out = {}
    for t in ts:
        for k, v in t.items():
            o = out.setdefault(k, {"count": 0, "ms": 0.0, "bytes": 0.0, "flops": 0.0})
            for f in o:
                o[f] += v[f]
    return out


def sum_stats(layers):
    tot = {}
    for l in layers:
        for k, v in l.stats().items():
            tot[k] = tot.get(k, 0) + v
    return tot


# ---------------------------------------------------------------- decode: one layer

def bench_decode(args, torch, dev):
    import expert_weight_paging_amd as ewp
    import workloads as W
    from workloads import gen

    cfg = W.CONFIGS[DECODE_CONFIG[args.workload]]
    B = args.batch
    rec = ewp.record_bytes(cfg.fmt, cfg.H, cfg.I)
    log("building pinned store: %d experts x %d B" % (cfg.E, rec))
    host = ewp.HostStore(cfg.E, rec)
    gen.expert_store(cfg, out=host.array)
    K = args.slots or cfg.K
    slots, state = ewp.alloc_layer_buffers(cfg.E, K, rec, dev)
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    layer = ewp.Layer(cfg.E, cfg.top_k, cfg.H, cfg.I, K, cfg.fmt, host, slots, state,
                      compute, copy, compute)
    G = min(K // cfg.top_k, B, 64)
    plan = ewp.Plan(layer, B)
    total = args.warmup + args.steps
    logits, x = gen.decode_inputs(cfg, B, steps=total)
    lg_d = torch.from_numpy(logits).to(dev)
    x_d = torch.from_numpy(x.view(np.int16)).to(dev)
    out = torch.empty(B, cfg.H, dtype=torch.float32, device=dev)

    step = step_fn(args)

    def run(t0, n):
        for t in range(t0, t0 + n):
            step(layer, plan, lg_d[t], x_d[t], out)

    run(0, args.warmup)
    torch.cuda.synchronize()
    s0 = layer.stats()
    t0 = time.perf_counter()
    run(args.warmup, args.steps)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    s1 = layer.stats()
    # roofline pass: the timed steps again, same table state, with events
    layer.reset()
    run(0, args.warmup)
    layer.timing_enable(True)
    run(args.warmup, args.steps)
    torch.cuda.synchronize()
    tm = layer.timing_read()
    floor_us = ewp.timing_floor(compute)
    layer.timing_enable(False)
    plan.close()
    layer.close()
    d = {k: s1[k] - s0[k] for k in s1}
    res = {"value": args.steps * B / el, "ms_per_step": el / args.steps * 1e3, "timing": tm,
           "floor_us": floor_us,
           "stats": d, "cfg": cfg, "B": B, "K": K,
           "workload": "one Qwen3-30B-A3B-shaped MoE layer, %s experts, E=%d top_k=%d hidden=%d "
                       "intermediate=%d, K=%d resident slots, decode at batch %d, correlated routing "
                       "p=%.2f, cold table%s" % (FMT_NAME[cfg.fmt], cfg.E, cfg.top_k, cfg.H, cfg.I,
                                                K, B, cfg.p_keep,
                                                ", " + mode_name(args) if (args.device or args.waves == "token") else "")}

    def cpu(budget):
        from oracle.layer import PagedLayer
        ref = PagedLayer(np.array(host.array), cfg.fmt, cfg.E, cfg.top_k, cfg.H, cfg.I, K, dtype=np.float32)
        # a longer decode sequence from the same seeded generator (same recipe),
        # so that the sample holds about `budget` seconds of oracle work
        lg_c, x_c = gen.decode_inputs(cfg, B, steps=max(total, 4096))
        n = 0
        t0 = time.perf_counter()
        while n < len(lg_c) and (time.perf_counter() - t0) < budget:
            xv = gen.bf16_bits_to_f32(x_c[n])
            if args.waves == "token":
                ref.step_token_waves(lg_c[n], xv, G)
            else:
                ref.step(lg_c[n], xv)
            n += 1
        el = time.perf_counter() - t0
        return {"value": n * B / el, "unit": "tok/s", "cores": oracle_threads(), "kind": "oracle",
                "sample": "%d decode steps (batch %d) of the same workload recipe from a cold table: "
                          "float32 numpy oracle incl. routing, LRU plan, record copies (host memcpy, "
                          "no PCIe) and SwiGLU experts, %.1f s" % (n, B, el), **host_info()}
    res["cpu"] = cpu
    res["cleanup"] = host.free
    res["pool"] = host.array
    res["step_fn"] = step_fn(args)
    return res


def step_fn(args):
    """The per-layer decode step of the chosen mode."""
    def step(layer, plan, lg, x, out):
        if args.waves == "token":
            layer.step_token_waves(plan, lg, x, out)
        elif args.device:
            layer.step_device(plan, lg, x, out)
        else:
            layer.step(plan, lg, x, out)
    return step


def bench_decode_cold(args, torch, dev, cfg, K, B, pool, step):
    """The decode layer's FFN with the chip's caches cold: n independent layers
    of the same shape (own pinned store, a permutation of the workload's
    records, own slots and routing chain) taken in turn at every step, so that
    between two steps of one layer the others stream n - 1 steps' experts
    (at batch 1 and bf16, 75.5 MB each: 528 MB for n = 8, twice the 256 MB
    last-level cache). Returns the timing of the expert kernels and the
    layer-steps per second."""
    import expert_weight_paging_amd as ewp
    from workloads import gen
    n = args.cold_layers
    rec = pool.shape[1]
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    hosts, layers, plans = [], [], []
    t0 = time.perf_counter()
    for l in range(n):
        h = ewp.HostStore(cfg.E, rec)
        gen.fill_layer_store(cfg, l, h.array, pool)
        slots, state = ewp.alloc_layer_buffers(cfg.E, K, rec, dev)
        L = ewp.Layer(cfg.E, cfg.top_k, cfg.H, cfg.I, K, cfg.fmt, h, slots, state, compute, copy, compute)
        hosts.append(h)
        layers.append(L)
        plans.append(ewp.Plan(L, B))
    log("cold pass: %d layers built in %.1f s (%.1f GB pinned, %.1f GB of slots)"
        % (n, time.perf_counter() - t0, n * cfg.E * rec / 1e9, n * K * rec / 1e9))
    warm, steps = args.cold_warmup, args.cold_steps
    logits, x = gen.cold_cycle_inputs(cfg, n, B, warm + steps)
    lg_d = torch.from_numpy(logits).to(dev)
    x_d = torch.from_numpy(x.view(np.int16)).to(dev)
    out = torch.empty(B, cfg.H, dtype=torch.float32, device=dev)

    def run(t0, m):
        for t in range(t0, t0 + m):
            for l in range(n):
                step(layers[l], plans[l], lg_d[t, l], x_d[t], out)

    run(0, warm)
    torch.cuda.synchronize()
    s0 = sum_stats(layers)
    t1 = time.perf_counter()
    run(warm, steps)
    torch.cuda.synchronize()
    el = time.perf_counter() - t1
    s1 = sum_stats(layers)
    for L in layers:
        L.reset()
    run(0, warm)
    for L in layers:
        L.timing_enable(True)
    run(warm, steps)
    torch.cuda.synchronize()
    tm = merge_timing([L.timing_read() for L in layers])
    for p in plans:
        p.close()
    for L in layers:
        L.close()
    for h in hosts:
        h.free()
    d = {k: s1[k] - s0[k] for k in s1}
    return {"timing": tm, "layer_steps_per_s": steps * n / el, "ms_per_layer_step": el / (steps * n) * 1e3,
            "layers": n, "steps": steps, "warmup": warm, "stats": d}


# ---------------------------------------------------------------- 48-layer stacks

def build_stack(cfg, dev, torch, max_tokens, initial_fill):
    import expert_weight_paging_amd as ewp
    from workloads import gen
    rec = ewp.record_bytes(cfg.fmt, cfg.H, cfg.I)
    log("generating the %d-record pool (%s)" % (cfg.E, FMT_NAME[cfg.fmt]))
    pool = gen.pool_records(cfg)
    compute, copy, route = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    hosts, layers, plans = [], [], []
    t0 = time.perf_counter()
    for l in range(cfg.layers):
        h = ewp.HostStore(cfg.E, rec)
        gen.fill_layer_store(cfg, l, h.array, pool)
        slots, state = ewp.alloc_layer_buffers(cfg.E, cfg.K, rec, dev)
        L = ewp.Layer(cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K, cfg.fmt, h, slots, state,
                      compute, copy, route, initial_fill=initial_fill)
        hosts.append(h)
        layers.append(L)
        plans.append(ewp.Plan(L, max_tokens))
    log("built %d layers: %.1f GB pinned, %.1f GB of slots, in %.1f s"
        % (cfg.layers, cfg.layers * cfg.E * rec / 1e9, cfg.layers * cfg.K * rec / 1e9,
           time.perf_counter() - t0))
    return hosts, layers, plans, pool, compute


def resolve_default_mode(args):
    """Without a mode flag, a decode step runs device-resolved (one wave when
    B * top_k <= K, else the expert waves it needs, at most 16), the stack as
    one HIP graph per token (the captured single-wave path); --lookahead and
    prefill run host-driven."""
    if args.host or args.device or args.graph or args.waves == "token":
        return
    import workloads as W
    if args.workload.startswith("decode"):
        cfg = W.CONFIGS[DECODE_CONFIG[args.workload]]
        K = args.slots or cfg.K
        if args.batch <= 64 and -(-min(args.batch * cfg.top_k, cfg.E) // K) <= 16:
            args.device = True
    elif args.workload == "stack-int4" and not args.lookahead:
        args.graph = True


def mode_name(args):
    if args.waves == "token":
        return ("token-partitioned waves: groups of K // top_k tokens, each a device-resolved "
                "single-wave step (kernel page-in, no host synchronisation)")
    la = ", routes and copies ahead on the copy stream (lookahead)" if args.lookahead else ""
    if args.graph:
        return "device-resolved steps (kernel page-in) captured in one HIP graph per token" + la
    if args.device:
        return "device-resolved steps (kernel page-in, no host synchronisation; expert waves when B * top_k > K)" + la
    return "one-layer lookahead" if args.lookahead else "strict layer order"


def bench_stack(args, torch, dev):
    import expert_weight_paging_amd as ewp
    import workloads as W
    from workloads import gen

    cfg = W.CONFIGS[4]
    hosts, layers, plans, pool, compute = build_stack(cfg, dev, torch, 1, False)
    total = args.warmup + args.steps
    logits, x0 = gen.stack_inputs(cfg, steps=total, routing=args.routing)
    lg_d = torch.from_numpy(logits).to(dev)             # [steps][L][1][E]
    x0_d = torch.from_numpy(x0.view(np.int16)).to(dev)  # [steps][1][H]
    x = torch.empty(1, cfg.H, dtype=torch.int16, device=dev)
    out = torch.empty(1, cfg.H, dtype=torch.float32, device=dev)
    lg_buf = torch.empty_like(lg_d[0])                  # fixed input of a captured token
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        # one token through the 48 device-resolved layers, captured once and
        # replayed per token (inputs copied into fixed buffers on the stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=compute):
            ewp.stack_forward_device(layers, plans, lg_buf, x, out, lookahead=args.lookahead)
        torch.cuda.synchronize()

    def run(t0, n, eager=False, lookahead=args.lookahead):
        with torch.cuda.stream(compute):  # inputs are written on the stream that reads them
            for t in range(t0, t0 + n):
                x.copy_(x0_d[t])
                if graph is not None and not eager:
                    lg_buf.copy_(lg_d[t])
                    graph.replay()
                elif args.device:
                    ewp.stack_forward_device(layers, plans, lg_d[t], x, out, lookahead=lookahead)
                else:
                    ewp.stack_forward(layers, plans, lg_d[t], x, out, lookahead=lookahead)

    run(0, args.warmup)
    torch.cuda.synchronize()
    s0 = sum_stats(layers)
    t0 = time.perf_counter()
    run(args.warmup, args.steps)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    s1 = sum_stats(layers)
    for L in layers:
        L.reset()
    # timers need eager launches; with device lookahead the up projection shares
    # its launch with the next layer's copies, so the kernels are timed in
    # strict order (the same kernels, each launched on its own)
    timed_la = args.lookahead and not args.device
    run(0, args.warmup, eager=True, lookahead=timed_la)
    for L in layers:
        L.timing_enable(True)
    run(args.warmup, args.steps, eager=True, lookahead=timed_la)
    torch.cuda.synchronize()
    tm = merge_timing([L.timing_read() for L in layers])
    floor_us = ewp.timing_floor()
    d = {k: s1[k] - s0[k] for k in s1}
    res = {"value": args.steps / el, "ms_per_step": el / args.steps * 1e3, "timing": tm, "stats": d,
           "floor_us": floor_us,
           "cfg": cfg, "B": 1,
           "workload": "48-layer Qwen3-30B-A3B-shaped MoE stack (attention omitted; each layer reads the "
                       "unit-gain RMSNorm of the residual stream), int4 asym g128 "
                       "experts, E=128 top_k=8 hidden=2048 intermediate=768, K=92 slots per layer, "
                       "batch-1 decode, %s routing%s, %s, cold tables"
                       % ("correlated p=0.75" if args.routing == "correlated" else "uniform",
                          "", mode_name(args))}

    def cpu(budget):
        from oracle.layer import PagedLayer
        refs = [PagedLayer(pool[gen.layer_permutation(cfg, l)], cfg.fmt, cfg.E, cfg.top_k, cfg.H,
                           cfg.I, cfg.K, dtype=np.float32) for l in range(4)]
        from oracle.layer import bf16_rne, rms_norm
        t0 = time.perf_counter()
        nl = nt = 0
        # tokens in order through the first four layers (tables start cold),
        # until the budget is spent; the rate is scaled to 48 layers
        while nt < len(x0) and time.perf_counter() - t0 < budget:
            xv = gen.bf16_bits_to_f32(x0[nt])
            for l in range(4):
                o, *_ = refs[l].step(logits[nt, l], bf16_rne(rms_norm(xv)))
                xv = bf16_rne(xv + o)
                nl += 1
            nt += 1
        el = time.perf_counter() - t0
        per_token = el / nl * cfg.layers
        return {"value": 1.0 / per_token, "unit": "tok/s", "cores": oracle_threads(), "kind": "oracle",
                "sample": "tokens 0..%d through the first 4 of 48 layers (tables start cold) with the "
                          "float32 numpy oracle, %.1f s, scaled to 48 layers" % (nt - 1, el), **host_info()}
    res["cpu"] = cpu

    def cleanup():
        for p in plans:
            p.close()
        for L in layers:
            L.close()
        for h in hosts:
            h.free()
    res["cleanup"] = cleanup
    return res


def bench_prefill(args, torch, dev):
    import expert_weight_paging_amd as ewp
    import workloads as W
    from workloads import gen

    cfg = W.CONFIGS[5]
    T = cfg.tokens
    hosts, layers, plans, pool, compute = build_stack(cfg, dev, torch, T, True)
    total = args.warmup + args.steps
    chunks = [gen.prefill_inputs(cfg, salt=c) for c in range(total)]
    x_d = torch.empty(T, cfg.H, dtype=torch.int16, device=dev)
    out = torch.empty(T, cfg.H, dtype=torch.float32, device=dev)
    lg_d = [torch.from_numpy(c[0]).to(dev) for c in chunks]
    x0_d = [torch.from_numpy(c[1].view(np.int16)).to(dev) for c in chunks]

    def run(c0, n):
        with torch.cuda.stream(compute):  # inputs are written on the stream that reads them
            for c in range(c0, c0 + n):
                x_d.copy_(x0_d[c])
                ewp.stack_forward(layers, plans, lg_d[c], x_d, out, lookahead=args.lookahead)

    run(0, args.warmup)
    torch.cuda.synchronize()
    s0 = sum_stats(layers)
    t0 = time.perf_counter()
    run(args.warmup, args.steps)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    s1 = sum_stats(layers)
    for L in layers:
        L.reset()
    run(0, args.warmup)
    for L in layers:
        L.timing_enable(True)
    run(args.warmup, args.steps)
    torch.cuda.synchronize()
    tm = merge_timing([L.timing_read() for L in layers])
    floor_us = ewp.timing_floor()
    d = {k: s1[k] - s0[k] for k in s1}
    res = {"value": args.steps * T / el, "ms_per_step": el / args.steps * 1e3, "timing": tm,
           "floor_us": floor_us,
           "stats": d, "cfg": cfg, "B": T,
           "workload": "prefill: one 2048-token chunk through a 48-layer Qwen3-30B-A3B-shaped bf16 "
                       "MoE stack (attention omitted; each layer reads the unit-gain RMSNorm of the "
                       "residual stream), E=128 top_k=8 hidden=2048 intermediate=768, "
                       "K=92 slots per layer warm with experts 0..91, uniform routing"}

    def cpu(budget):
        from oracle.layer import PagedLayer, bf16_rne, rms_norm
        lg, x0 = chunks[0]
        xv = gen.bf16_bits_to_f32(x0)
        t0 = time.perf_counter()
        nl = 0
        for l in range(cfg.layers):
            ref = PagedLayer(pool[gen.layer_permutation(cfg, l)], cfg.fmt, cfg.E, cfg.top_k, cfg.H,
                             cfg.I, cfg.K, initial_fill=True, dtype=np.float32)
            o, *_ = ref.step(lg[l], bf16_rne(rms_norm(xv)))
            xv = bf16_rne(xv + o)
            nl += 1
            if time.perf_counter() - t0 > budget:
                break
        el = time.perf_counter() - t0
        return {"value": T / (el / nl * cfg.layers), "unit": "tok/s", "cores": oracle_threads(),
                "kind": "oracle",
                "sample": "chunk 0 (2048 tokens) through the first %d of 48 layers with the float32 "
                          "numpy oracle, %.1f s, scaled to 48 layers" % (nl, el), **host_info()}
    res["cpu"] = cpu

    def cleanup():
        for p in plans:
            p.close()
        for L in layers:
            L.close()
        for h in hosts:
            h.free()
    res["cleanup"] = cleanup
    return res


# ---------------------------------------------------------------- report

def roofline(res, workload, variant):
    """variant: the workload name plus any non-default option; PMC traffic is
    stored per variant (the committed profiles use the default options)."""
    tm = res["timing"]
    if workload == "prefill-bf16":
        kinds = [k for k in ("gemm_up", "gemm_down") if tm[k]["count"]]
        dom = max(kinds, key=lambda k: tm[k]["ms"])
        sec = tm[dom]["ms"] * 1e-3
        flops = tm[dom]["flops"] / sec / 1e12
        gbps = tm[dom]["bytes"] / sec / 1e9
        kname = "grouped_gemm_kernel<%s,1>" % ("true" if dom == "gemm_up" else "false")
        # both GEMMs of the expert FFN together (the down GEMM's flops count h once)
        both = sum(tm[k]["flops"] for k in kinds) / (sum(tm[k]["ms"] for k in kinds) * 1e-3) / 1e12
        both_gbps = sum(tm[k]["bytes"] for k in kinds) / (sum(tm[k]["ms"] for k in kinds) * 1e-3) / 1e9
        # flops per weight byte = 2 x the routed rows per expert (about 2 x 128 at
        # 2048 tokens, top-8 of 128): below the ridge of bf16 MFMA over HBM
        # (2500 TFLOP/s / 8 TB/s = 312.5 flop/B), so the GEMMs are bound by
        # streaming their weights, and the roofline is the HBM one
        ai = tm[dom]["flops"] / tm[dom]["bytes"]
        ridge = BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
        common = {"kernel": kname, "traffic": traffic_from_profiles(kname, variant),
                  "avg_launch_us": round(tm[dom]["ms"] / tm[dom]["count"] * 1e3, 3),
                  "launches": tm[dom]["count"],
                  "algorithmic_bytes_per_launch": tm[dom]["bytes"] / tm[dom]["count"],
                  "algorithmic_flops_per_launch": tm[dom]["flops"] / tm[dom]["count"],
                  "flop_per_weight_byte": round(ai, 1), "ridge_flop_per_byte": round(ridge, 1),
                  "mfma_TFLOPs": round(flops, 1), "mfma_frac": round(flops / BF16_MFMA_PEAK_TFLOPS, 4),
                  "gemm_up_plus_down_GBps": round(both_gbps, 1),
                  "gemm_up_plus_down_hbm_frac": round(both_gbps / HBM_PEAK_GBPS, 4),
                  "gemm_up_plus_down_TFLOPs": round(both, 1),
                  "gemm_up_plus_down_mfma_frac": round(both / BF16_MFMA_PEAK_TFLOPS, 4),
                  "launch_floor_us": round(res["floor_us"], 3)}
        if ai < ridge:
            return {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(gbps / HBM_PEAK_GBPS, 4), **common}
        return {"bound": "mfma", "achieved": round(flops, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(flops / BF16_MFMA_PEAK_TFLOPS, 4), **common}
    return hbm_roofline(tm, res["floor_us"], variant)


def expert_ffn_bytes(fmt, H, I):
    """Weight bytes one expert's up launch (W13 and its scales / zero points)
    and down launch (W_d and its tables) read, by the record formats."""
    n13, nd = 2 * I * H, H * I
    if fmt == 0:   # f32
        return 4 * n13, 4 * nd
    if fmt == 1:   # bf16
        return 2 * n13, 2 * nd
    if fmt == 2:   # FP8 e4m3, fp32 scales per 128 x 128 block
        return n13 + 4 * (n13 // (128 * 128)), nd + 4 * (nd // (128 * 128))
    if fmt == 3:   # int4, fp16 scale and zero point per 128 weights
        return n13 // 2 + 4 * (n13 // 128), nd // 2 + 4 * (nd // 128)
    if fmt == 4:   # MXFP4, one E8M0 byte per 32 weights
        return n13 // 2 + n13 // 32, nd // 2 + nd // 32
    raise ValueError(fmt)


def exact_ffn_bytes(tm, refs, cfg):
    """The decode FFN timers of device-resolved steps count the most experts a
    step can route (the host does not see the plan); the timed steps' exact
    bytes are their distinct experts (the layer counters' refs, summed over
    the steps, which the event-timed pass replays) times each expert's bytes.
    Host-driven launches count exactly, and this gives the same figure."""
    up, dn = expert_ffn_bytes(cfg.fmt, cfg.H, cfg.I)
    out = {k: dict(v) for k, v in tm.items()}
    if out["ffn_up"]["count"]:
        out["ffn_up"]["bytes"] = float(refs * up)
    if out["ffn_down"]["count"]:
        out["ffn_down"]["bytes"] = float(refs * dn)
    return out


def hbm_roofline(tm, floor_us, variant, cache=None):
    """The decode step's expert FFN, its two kernels (gate/up + SiLU, down +
    weighted combine) together: algorithmic bytes (the weight bytes of the
    experts each launch reads) over the summed event-measured durations of
    both kernels, with each kernel's own figures beside it. `traffic` is the
    counter-measured HBM bytes of one up launch plus one down launch."""
    per, traffic = {}, 0.0
    for k, name in (("ffn_up", "ffn_up_kernel"), ("ffn_down", "ffn_down_kernel")):
        v = tm[k]
        if not v["count"]:
            return None
        gbps = v["bytes"] / (v["ms"] * 1e-3) / 1e9
        t = traffic_from_profiles(name, variant)
        traffic = None if (t is None or traffic is None) else traffic + t
        per[name] = {"avg_launch_us": round(v["ms"] / v["count"] * 1e3, 3),
                     "algorithmic_bytes_per_launch": v["bytes"] / v["count"],
                     "achieved": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": t,
                     "launches": v["count"]}
    up, dn = tm["ffn_up"], tm["ffn_down"]
    achieved = (up["bytes"] + dn["bytes"]) / ((up["ms"] + dn["ms"]) * 1e-3) / 1e9
    r = {"bound": "hbm", "kernel": "ffn_up_kernel + ffn_down_kernel", "achieved": round(achieved, 1),
         "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
         "traffic": traffic,
         "algorithmic_bytes_per_launch_pair": (up["bytes"] + dn["bytes"]) / up["count"],
         "avg_launch_pair_us": round((up["ms"] + dn["ms"]) / up["count"] * 1e3, 3),
         "kernels": per, "launch_floor_us": round(floor_us, 3)}
    if cache:
        r["cache"] = cache
    return r


def cold_only_line(args, torch, dev, variant):
    """Only the cache-cold pass of a decode workload (what its profiles are taken on)."""
    import workloads as W
    from workloads import gen
    cfg = W.CONFIGS[DECODE_CONFIG[args.workload]]
    K = args.slots or cfg.K
    pool = gen.pool_records(cfg)
    cold = bench_decode_cold(args, torch, dev, cfg, K, args.batch, pool, step_fn(args))
    import expert_weight_paging_amd as ewp
    return {"metric": METRIC, "value": round(cold["layer_steps_per_s"] * args.batch, 2), "unit": "tok/s",
            "n_gpus": 1, "steps": cold["steps"], "warmup": cold["warmup"],
            "ms_per_step": round(cold["ms_per_layer_step"], 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": FMT_NAME[cfg.fmt], "data": "synthetic (seeded)",
            "config": {"workload": "%d independent %s MoE layers of the Qwen3-30B-A3B shape taken in turn, "
                                   "K=%d, batch %d; value = tokens/s of one layer (layer-steps/s x batch)"
                                   % (cold["layers"], FMT_NAME[cfg.fmt], K, args.batch)},
            "roofline": hbm_roofline(exact_ffn_bytes(cold["timing"], cold["stats"]["refs"], cfg),
                                     ewp.timing_floor(), variant + " cold", cache="cold")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode-bf16",
                    choices=["decode-bf16", "decode-fp8", "decode-mxfp4", "stack-int4", "prefill-bf16"])
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--routing", default="correlated", choices=["correlated", "uniform"])
    ap.add_argument("--lookahead", action="store_true")
    ap.add_argument("--device", action="store_true",
                    help="device-resolved single-wave steps (kernel page-in, no host sync)")
    ap.add_argument("--host", action="store_true",
                    help="host-driven steps (the host reads each plan and issues DMA page-ins) even "
                         "when the batch fits one wave")
    ap.add_argument("--graph", action="store_true",
                    help="stack-int4 only: device-resolved token captured in a HIP graph")
    ap.add_argument("--waves", default="expert", choices=["expert", "token"],
                    help="decode batches beyond one wave: expert-partitioned waves (host-driven, "
                         "default) or groups of K // top_k tokens as device-resolved steps")
    ap.add_argument("--slots", type=int, default=None, help="decode workloads: K instead of the config's")
    ap.add_argument("--cold-layers", type=int, default=8,
                    help="decode workloads: the headline roofline is measured on this many independent "
                         "layers of the same shape taken in turn (caches cold between a layer's steps); "
                         "0 = measure it on the one layer (caches warm)")
    ap.add_argument("--cold-steps", type=int, default=64)
    ap.add_argument("--cold-warmup", type=int, default=16)
    ap.add_argument("--cold-only", action="store_true",
                    help="decode workloads: run only the cache-cold pass (for profiling it alone)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn two rocprofv3 --pmc counter CSVs of this workload "
                         "(FETCH_SIZE, WRITE_SIZE) into profiles/pmc_traffic.json")
    args = ap.parse_args()
    if args.host and (args.device or args.graph or args.waves == "token"):
        print("--host excludes --device, --graph and --waves token", file=sys.stderr)
        sys.exit(2)
    resolve_default_mode(args)
    variant = args.workload + "".join(
        s for s, on in ((" lookahead", args.lookahead), (" uniform", args.routing != "correlated"),
                        (" batch=%d" % args.batch, args.batch != 1), (" device", args.device and not args.graph),
                        (" graph", args.graph), (" waves=token", args.waves == "token"),
                        (" K=%s" % args.slots, args.slots is not None)) if on)
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], variant + (" cold" if args.cold_only else ""))
        return
    if args.graph:
        args.device = True
        if args.workload != "stack-int4":
            print("--graph applies to --workload stack-int4", file=sys.stderr)
            sys.exit(2)
    if args.device and (args.workload == "prefill-bf16" or
                        (args.lookahead and args.workload != "stack-int4")):
        print("--device runs single-wave decode steps: not with prefill-bf16; --lookahead only "
              "with stack-int4", file=sys.stderr)
        sys.exit(2)
    if (args.waves == "token" or args.slots) and not args.workload.startswith("decode"):
        print("--waves token and --slots apply to the decode workloads", file=sys.stderr)
        sys.exit(2)
    if args.waves == "token" and args.device:
        print("--waves token already runs device-resolved steps", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the Paged Experts path is single-GPU and this "
              "build has no multi-GPU mode (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    defaults = {"decode-bf16": (256, 32), "decode-fp8": (256, 32), "decode-mxfp4": (256, 32),
                "stack-int4": (128, 16),
                "prefill-bf16": (3, 1)}[args.workload]
    args.steps = defaults[0] if args.steps is None else args.steps
    args.warmup = defaults[1] if args.warmup is None else args.warmup
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    peaks = None if args.no_peaks else measured_peaks(torch, dev)
    fn = {"decode-bf16": bench_decode, "decode-fp8": bench_decode, "decode-mxfp4": bench_decode,
          "stack-int4": bench_stack,
          "prefill-bf16": bench_prefill}[args.workload]
    decode = args.workload.startswith("decode")
    if args.cold_only:
        if not decode or args.cold_layers < 2:
            print("--cold-only applies to the decode workloads with --cold-layers >= 2", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(cold_only_line(args, torch, dev, variant)), flush=True)
        return
    res = fn(args, torch, dev)
    log("timed %d steps: %.3f ms/step" % (args.steps, res["ms_per_step"]))
    cold = None
    if decode and args.cold_layers >= 2:
        cold = bench_decode_cold(args, torch, dev, res["cfg"], res["K"], res["B"], res["pool"], res["step_fn"])
        log("cold pass: %d layers x %d steps, %.3f ms per layer-step"
            % (cold["layers"], cold["steps"], cold["ms_per_layer_step"]))
    tm, st, cfg = res["timing"], res["stats"], res["cfg"]
    if args.workload.startswith("decode"):
        tm = exact_ffn_bytes(tm, st["refs"], cfg)
        res["timing"] = tm
        if cold is not None:
            cold["timing"] = exact_ffn_bytes(cold["timing"], cold["stats"]["refs"], cfg)
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
        "dtype": FMT_NAME[cfg.fmt],
        "data": "synthetic (seeded; %s routing, weights N(0,0.02))"
                % ("correlated p=0.75" if cfg.routing == "correlated" and args.routing == "correlated"
                   else "uniform"),
        "config": {"workload": res["workload"], "batch": res["B"], "num_slots": res.get("K", cfg.K),
                   "experts": cfg.E, "top_k": cfg.top_k, "layers": cfg.layers,
                   "lookahead": bool(args.lookahead), "parallelism": "single GPU"},
        "roofline": roofline(res, args.workload, variant) if cold is None else
                    hbm_roofline(cold["timing"], res["floor_us"], variant + " cold",
                                 cache="cold: %d independent layers of this shape taken in turn, %d steps "
                                       "after %d, so each layer's experts are out of the 256 MB "
                                       "last-level cache when it runs again" % (cold["layers"],
                                                                                cold["steps"],
                                                                                cold["warmup"])),
        "kernels_us": {k: round(v["ms"] / v["count"] * 1e3, 3) for k, v in tm.items() if v["count"]},
        "roofline_warm": None if cold is None else
                         hbm_roofline(tm, res["floor_us"], variant,
                                      cache="warm: the one layer of the timed steps, whose step shares "
                                            "most experts with the one before (last-level cache hits)"),
        "cold_pass": None if cold is None else
                     {"layers": cold["layers"], "steps": cold["steps"],
                      "ms_per_layer_step": round(cold["ms_per_layer_step"], 4),
                      "misses_per_layer_step": round(cold["stats"]["misses"] / max(cold["stats"]["steps"], 1), 4),
                      "kernels_us": {k: round(v["ms"] / v["count"] * 1e3, 3)
                                     for k, v in cold["timing"].items() if v["count"]}},
        # device-resolved copies are timed without their byte count (the host does not see
        # the plan); the timed pass pages the same bytes as the counted one
        "page_in": {"GBps": round((pin["bytes"] or st["bytes_paged"]) / max(pin["ms"], 1e-9) / 1e6, 2),
                    "waves_with_copies": pin["count"], "bytes_per_step": st["bytes_paged"] / args.steps},
        "hit_rate": round(st["hits"] / max(st["refs"], 1), 4),
        "miss_rate_per_activation": round(st["misses"] / max(st["activations"], 1), 4),
        "misses_per_step": round(st["misses"] / args.steps, 4),
        "waves_per_layer_step": round(st["waves"] / max(st["steps"], 1), 4),
        "measured_peaks": peaks,
    }
    if peaks is not None and line["roofline"] and "kernels" in line["roofline"]:
        line["roofline"]["one_launch_read"] = one_launch_read_reference(torch, dev, line["roofline"])
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (budget %.0f s)" % args.cpu_budget)
        line["cpu_baseline"] = res["cpu"](args.cpu_budget)
    res["cleanup"]()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
