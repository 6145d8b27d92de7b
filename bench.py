"""Benchmark: one MI355X's share of the SS-HSDP update phase.

    python bench.py [--steps K] [--warmup W] [--config 2] [--layout L] [--ns-tiles P] [--ns-gram O] [--g G]
                    [--no-cpu] [--no-graph]
    python bench.py --part rs [--config N]      (the reduce-scatter tail)

A step is one sshdp_update_step over the whole workload: Muon momentum,
batched bf16 MFMA Newton-Schulz, main-weight update, AdamW, and the MXFP8
requantisation of every runtime weight.  Inputs are seeded synthetic roots,
resident in HBM before timing starts.  The default workload is the dense
transformer block (d=2048, 16 heads of 128, 4 KV heads, MLP 8192, per-head
QKV Muon units), the configuration the metric is quoted on.

Prints one JSON line.  `value` = parameters updated per second (padding
excluded) from HIP events around K steps on the launch stream (`step_ms`:
median/min/max of the single steps).  `roofline` covers the Newton-Schulz
phase, the dominant part: executed MFMA flops of its tile schedule per step
divided by the phase's time (HIP events from the fork on the launch stream to
the join of the concurrent streams, in a second pass of K steps), against the
dense bf16 peak; `traffic` is the phase's HBM-side bytes per step from the
counter runs recorded in profiles/traffic.json (null when the kernel sources
changed since).  `repack_roofline` is G (with AdamW where fused) against HBM
bandwidth.  `graph_ms_per_step` is the same step captured once into a HIP
graph and replayed K times (context only; `value` is the eager figure).
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E
METRIC = "update-step params/sec (Muon+AdamW+MXFP8 repack); NS MFMA %, repack HBM %"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--layout", choices=["rowmajor", "tile32x4", "block32x32"], default=None,
                    help="scale layout (default: the workload's own); block32x32 = one scale per 32x32 block")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--ns-tiles", choices=["auto", "small", "large"], default="auto",
                    help="Newton-Schulz tile policy of the plan (default: the planner's choice)")
    ap.add_argument("--ns-gram", choices=["auto", "nt"], default="auto",
                    help="Gram operand: the planner's choice (X^T for 128-tile Grams) or X row-major everywhere")
    ap.add_argument("--g", choices=["mxfp8", "bf16"], default="mxfp8",
                    help="G on the runtime weights: MXFP8 requant (default) or a bfloat16 cast")
    ap.add_argument("--cpu-budget", type=float, default=25.0, help="seconds of oracle work to aim for")
    ap.add_argument("--part", choices=["step", "rs"], default="step",
                    help="step: the update step (default); rs: the reduce-scatter tail on the workload's "
                         "gradient size (4 BF16 slices -> BF16-SR partial; 2 partials accumulated into FP32)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="before timing, copy a 1 GiB buffer three times (a plain copy kernel of known "
                         "size, the calibration for HBM byte counters)")
    return ap.parse_args()


def source_digest(names):
    """sha256 over the kernel sources a counter figure was taken on."""
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mxfp8_weight_repack_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, part):
    """HBM bytes per step of `part` ("ns_phase" or "repack") on `workload`, from
    the counter runs recorded in profiles/traffic.json, or None when there are
    none or the kernel sources changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload, {}).get(part)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("src_digest") != source_digest(rec.get("sources", [])):
        return None
    return rec["bytes_per_step"]


def cpu_baseline(wl, budget_s):
    """Time the oracle (as it stands) on a bounded sample of the workload's
    units: units are taken in table order until the estimated cost fills the
    budget; params/s = sampled params / oracle time."""
    import oracle
    from oracle.views import resolve_views, unit_indices
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in blas] or [1])
        backend = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip() for i in blas}))
    except Exception:  # pragma: no cover
        threads, backend = 1, "unknown BLAS"
    backend = backend or "unknown BLAS"
    w0, g = wl.arrays()
    res = resolve_views(wl.nodes, wl.root_numel, wl.scale_layout)
    # cost model for picking the sample: ~0.3 us/element elementwise, ~25 GF/s per BLAS thread for NS
    pick, est = [], 0.0
    for i, r in enumerate(res):
        if not r["is_unit"]:
            continue
        n = r["rows"] * r["cols"]
        cost = 3e-7 * n
        if r["optimizer"] == "muon":
            rr, cc = min(r["rows"], r["cols"]), max(r["rows"], r["cols"])
            cost += 5 * (4 * rr * rr * cc + 2 * rr ** 3) / (25e9 * threads)
        if est + cost > budget_s and pick:
            continue
        pick.append(i)
        est += cost
    sub = [dict(wl.nodes[i], parent=-1, offset=res[i]["abs"]) for i in pick]
    w, m, v = w0.copy(), np.zeros_like(w0), np.zeros_like(w0)
    codes = np.zeros(wl.root_numel, np.uint8)
    scales = np.zeros((wl.root_numel + 31) // 32, np.uint8)
    # quantise the sampled units' own elements (their share of G)
    for nd in sub:
        nd["quantize"] = nd["cols"] % 32 == 0 and nd["row_stride"] == nd["cols"] and nd["offset"] % 32 == 0
    params = sum(nd["rows"] * nd["cols"] for nd in sub)
    t0 = time.perf_counter()
    oracle.update_step(sub, wl.root_numel, w, g, m, v, codes, scales, 1, layout="rowmajor")
    dt = time.perf_counter() - t0
    return {"value": params / dt, "unit": "params/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(sub)} of {len(wl.units())} units ({params} params, one full update step "
                      f"incl. their MXFP8 repack) in {dt:.1f} s; NumPy fp64 on {backend}, {threads} BLAS threads",
            "seconds": dt}


def run_env(torch, wl):
    """What the numbers were taken on: device, software versions, host cores
    and the input seeds."""
    p = torch.cuda.get_device_properties(0)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count()
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    return {"device": p.name, "gcn_arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "l2_bytes": getattr(p, "L2_cache_size", None), "hbm_gib": round(p.total_memory / 2 ** 30, 1),
            "torch": torch.__version__, "hip": torch.version.hip,
            "host_cores": cores, "host_cpu": cpu,
            "seeds": f"numpy PCG64(SeedSequence([{wl.config_id}, stream])), stream 0 = w, 1 = g, 2 = structure"}


def bench_rs(args, wl):
    """The reduce-scatter tail at the workload's gradient size: a local
    reducer sums 4 BF16 slices into a BF16 partial with stochastic rounding
    (10 B/element: 4 x 2 read, 2 written), then the final reduction adds 2
    such partials into the persistent FP32 gradient (12 B/element).  A step is
    one of each; inputs are resident before timing."""
    import torch
    import mxfp8_weight_repack_amd as sh
    n = (wl.root_numel + 15) // 16 * 16
    dev = "cuda:0"
    gen = torch.Generator(device=dev).manual_seed(args.config)
    slices = [(torch.randn(n, device=dev, generator=gen) * 1e-3).to(torch.bfloat16) for _ in range(4)]
    parts = [torch.empty(n, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    g = torch.zeros(n, dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream()
    sp = s.cuda_stream

    def step(t):
        for i in range(2):
            sh.rs_reduce(slices, "bf16", parts[i], "bf16_sr", n, seed=1234, ctr=2 * t + i, g0=0, stream=sp)
        sh.rs_accumulate(parts, "bf16", g, n, first=(t == 0), stream=sp)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ms_red = ms_acc = 0.0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for t in range(args.steps):
        ev[0].record(s)
        for i in range(2):
            sh.rs_reduce(slices, "bf16", parts[i], "bf16_sr", n, seed=1234, ctr=2 * t + i, g0=0, stream=sp)
        ev[1].record(s)
        sh.rs_accumulate(parts, "bf16", g, n, first=False, stream=sp)
        ev[2].record(s)
        torch.cuda.synchronize()
        ms_red += ev[0].elapsed_time(ev[1]) / 2
        ms_acc += ev[1].elapsed_time(ev[2])
    e1.record(s)
    torch.cuda.synchronize()
    ms_red /= args.steps
    ms_acc /= args.steps
    red_gbs = 10.0 * n / (ms_red / 1e3) / 1e9
    acc_gbs = 12.0 * n / (ms_acc / 1e3) / 1e9
    out = {"metric": "reduce-scatter tail GB/s (BF16-SR partial + FP32 accumulate)",
           "value": (2 * 10.0 + 12.0) * n / ((2 * ms_red + ms_acc) / 1e3) / 1e9, "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": 2 * ms_red + ms_acc,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"{wl.name}: gradient of {n} elements, 4 BF16 slices per partial, 2 partials"},
           "roofline": {"bound": "hbm", "kernel": "k_rs_reduce (BF16 in, BF16-SR out)", "achieved": red_gbs,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": red_gbs / HBM_PEAK_GBS, "traffic": None},
           "accumulate_roofline": {"bound": "hbm", "kernel": "k_rs_accumulate", "achieved": acc_gbs,
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": acc_gbs / HBM_PEAK_GBS},
           "components": {"rs_reduce": {"ms_per_call": ms_red}, "rs_accumulate": {"ms_per_call": ms_acc}}}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no "
              f"multi-GPU path: run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import mxfp8_weight_repack_amd as sh
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = workloads.config(args.config)
    if args.part == "rs":
        return bench_rs(args, wl)
    w0, g0 = wl.arrays()
    layout = args.layout or wl.scale_layout
    nodes = wl.nodes
    if args.g == "bf16":                      # every G region becomes a bfloat16 cast
        nodes = [dict(nd, quantize="bf16") if nd["quantize"] else nd for nd in nodes]
    plan = sh.Plan(nodes, wl.root_numel, layout=layout, ns_tiles=args.ns_tiles, ns_gram=args.ns_gram)
    st = plan.stats()
    w = torch.from_numpy(w0).to(dev)
    g = torch.from_numpy(g0).to(dev)
    m = torch.zeros_like(w)
    v = torch.zeros_like(w) if st["n_adamw_units"] else None
    codes = torch.zeros(wl.root_numel, dtype=torch.uint8, device=dev)
    scales = torch.zeros(st["scale_bytes"], dtype=torch.uint8, device=dev)
    ws_bytes = max(int(st["workspace_bytes"]), 256)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    w16 = torch.empty(wl.root_numel, dtype=torch.bfloat16, device=dev) if args.g == "bf16" else None
    bufs = sh.buffers(w, g, m, v, codes, scales, w_bf16=w16)
    mhp, ahp = sh.muon_hp(), sh.adamw_hp()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    step = 0
    for _ in range(args.warmup):
        step += 1
        sh.update_step(plan, bufs, mhp, ahp, step, ws, ws_bytes, sp)
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for k in range(args.steps):
        step += 1
        sh.update_step(plan, bufs, mhp, ahp, step, ws, ws_bytes, sp)
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per_step = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps))
    value = wl.params / (ms / 1e3)

    # the same step captured once into a HIP graph (side streams joined inside the
    # capture) and replayed K times: the launch sequence without the host in the loop
    graph_ms = None
    if not args.no_graph:
        gstream = torch.cuda.Stream()
        gstream.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gstream):
            sh.update_step(plan, bufs, mhp, ahp, step + 1, ws, ws_bytes, gstream.cuda_stream)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        gev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        gev[0].record()
        for _ in range(args.steps):
            graph.replay()
        gev[1].record()
        torch.cuda.synchronize()
        graph_ms = gev[0].elapsed_time(gev[1]) / args.steps
        step += 1 + args.warmup + args.steps
        del graph

    # per-kernel-class durations: HIP events bracketing every launch, same K steps
    plan.profile(True)
    for _ in range(args.steps):
        step += 1
        sh.update_step(plan, bufs, mhp, ahp, step, ws, ws_bytes, sp)
    torch.cuda.synchronize()
    prof = plan.profile_read()
    plan.profile(False)
    components = {c: {"ms_per_step": prof[c][0] / args.steps, "launches_per_step": prof[c][1] / args.steps}
                  for c in prof if prof[c][1]}
    # Newton-Schulz: all groups' contraction launches (concurrent streams) over the NS phase,
    # fork to join on the launch stream; executed = the MFMA work of the tile schedule
    roofline = None
    ns_ms = prof["ns_phase"][0] / args.steps if prof["ns_phase"][1] else 0.0
    if ns_ms > 0:
        ns_s = ns_ms / 1e3
        achieved = st["ns_tile_flops"] / ns_s / 1e12
        ns_launches = sum(prof[c][1] for c in ("ns_gram", "ns_poly", "ns_update")) / args.steps
        roofline = {"bound": "mfma",
                    "kernel": "k_ns (Newton-Schulz contraction: every group's launches, NS phase wall time)",
                    "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                    "traffic": measured_traffic(wl.name, "ns_phase"),
                    "executed_tflop_per_step": st["ns_tile_flops"] / 1e12,
                    "dense_tflop_per_step": st["ns_flops"] / 1e12,
                    "effective_dense_tflops": st["ns_flops"] / ns_s / 1e12,
                    "ns_phase_ms": ns_ms, "launches_per_step": ns_launches}
    # repack (G) HBM fraction: algorithmic bytes 4 (read w) + 1 (code) + 1/32 (scale) per element,
    # plus 28 B/element of AdamW where it is fused
    rq_ms = prof["requant"][0] + prof["adamw_requant"][0]
    repack = None
    if rq_ms > 0:
        fused = st["fused_quant_elems"]
        per_scale = 1.0 / 1024 if layout == "block32x32" else 1.0 / 32
        byts = (st["quant_elems"] - fused) * (5.0 + per_scale) + fused * (29.0 + per_scale)
        gbs = byts * args.steps / (rq_ms / 1e3) / 1e9
        repack = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": gbs / HBM_PEAK_GBS, "bytes_per_step": byts,
                  "traffic": measured_traffic(wl.name, "repack")}
    cast = None
    if prof["cast_bf16"][0] > 0:          # G as a bfloat16 cast: 4 (read w) + 2 (write) bytes per element
        byts = 6.0 * st["cast_elems"]
        gbs = byts * args.steps / (prof["cast_bf16"][0] / 1e3) / 1e9
        cast = {"bound": "hbm", "kernel": "k_cast_bf16", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "bytes_per_step": byts}
    out = {
        "metric": METRIC, "value": value, "unit": "params/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms,
        "step_ms": {"median": per_step[len(per_step) // 2], "min": per_step[0], "max": per_step[-1]},
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "params": wl.params, "root_numel": wl.root_numel,
                   "muon_units": st["n_muon_units"], "adamw_units": st["n_adamw_units"],
                   "ns_groups": [[gi["r"], gi["c"], gi["n_units"]] for gi in plan.groups()],
                   "scale_layout": layout, "g": args.g, "ns_tiles": args.ns_tiles, "ns_gram": args.ns_gram,
                   "ns_tflop_per_step": st["ns_flops"] / 1e12},
        "roofline": roofline, "repack_roofline": repack, "cast_roofline": cast, "components": components,
        "graph_ms_per_step": graph_ms,
    }
    out["env"] = run_env(torch, wl)
    if not args.no_cpu:
        cb = cpu_baseline(wl, args.cpu_budget)
        cb.pop("seconds", None)
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
