"""Benchmark: one MI355X's share of the SS-HSDP update phase.

    python bench.py [--steps K] [--warmup W] [--config 5] [--repack-config 4] [--layout L] [--ns-tiles P]
                    [--ns-gram O] [--g G] [--no-cpu] [--no-graph]
    python bench.py --part rs [--config N]      (the reduce-scatter tail)

A step is one sshdp_update_step over the whole workload: Muon momentum,
batched bf16 MFMA Newton-Schulz, main-weight update, AdamW, and the MXFP8
requantisation of every runtime weight.  Inputs are seeded synthetic roots,
resident in HBM before timing starts.  The default workload is the largest
one a single GPU holds: the d=8192 dense block (64 heads of 128, 8 KV heads,
MLP 28672; per-head QKV Muon units, 855.6 M parameters, 148.7 TFLOP of
Newton-Schulz per step).

Prints one JSON line.  `value` = parameters updated per second (padding
excluded) from HIP events around K steps on the launch stream (`step_ms`:
median/min/max of the single steps).

`roofline` is the dominant kernel's: the Newton-Schulz update product
X' = aX + BX of the groups on the launch stream (for the d=8192 block, the
three 8192 x 28672 MLP units in 256-tiles), its executed MFMA flops per launch
(zero-momentum units excluded) over its average launch time from HIP events
bracketing each launch on that stream, against the dense bf16 peak; `traffic`
is its HBM-side bytes per launch from the FETCH_SIZE / WRITE_SIZE counter runs
recorded in profiles/traffic.json (null when the kernel sources changed
since).  `ns_phase` is the whole Newton-Schulz phase (every group, concurrent
streams) over its wall time.

`repack_roofline` is the other half of the metric, AdamW + MXFP8 repack, timed
in the same run on the flat ragged shard of 5e8 elements (--repack-config):
the fused AdamW+G pass at 29.03125 algorithmic bytes per element against HBM
bandwidth.  `g_roofline` is the main workload's own G.  `graph_ms_per_step` is
the same step captured once into a HIP graph and replayed K times (context
only; `value` is the eager figure).  `cpu_baseline` times the CPU oracle on a
bounded sample of the main workload and extrapolates to one whole step.
"""

import argparse
import ctypes
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
    ap.add_argument("--config", type=int, default=5,
                    help="workload (1-5; default 5, the d=8192 dense block, the largest one GPU holds)")
    ap.add_argument("--repack-config", type=int, default=4,
                    help="workload whose fused AdamW + MXFP8 pass gives repack_roofline, timed in the same run "
                         "(default 4, the flat 5e8-element shard; 0 = none)")
    ap.add_argument("--layout", choices=["rowmajor", "tile32x4", "block32x32"], default=None,
                    help="scale layout (default: the workload's own); block32x32 = one scale per 32x32 block")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--ns-tiles", choices=["auto", "small", "large"], default="auto",
                    help="Newton-Schulz tile policy of the plan (default: the planner's choice)")
    ap.add_argument("--ns-gram", choices=["auto", "nt"], default="auto",
                    help="Gram operand: the planner's choice (X^T for 128-tile Grams) or X row-major everywhere")
    ap.add_argument("--ns-streams", choices=["auto", "one"], default="auto",
                    help="Newton-Schulz groups on the planner's streams, or every group on the launch stream")
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
    """sha256 over the code of the kernel sources a counter figure was taken on:
    comments and blank space are left out, so an edited comment keeps the
    figure while any change to the code drops it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mxfp8_weight_repack_amd", "csrc", n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)          # block comments
        text = re.sub(r"//[^\n]*", " ", text)                        # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, part):
    """HBM-side bytes per launch of `part` ("dominant": the kernel `roofline`
    covers; "repack": the fused AdamW + G pass) on `workload`, from the counter
    runs recorded in profiles/traffic.json, or None when there are none or the
    kernel sources changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload, {}).get(part)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("src_digest") != source_digest(rec.get("sources", [])):
        return None
    return rec["bytes_per_launch"]


def cpu_baseline(wl, budget_s):
    """The oracle (as it stands) on a bounded sample of the workload, extrapolated
    to one whole update step.

    Per distinct Muon unit shape, one unit runs the oracle's Muon update in full
    (momentum, normalisation, Newton-Schulz, weight update) when its five
    float64 Newton-Schulz steps fit the budget's share; larger units run it with
    0 and with 1 Newton-Schulz step, and the step count scales the difference
    (each step is the same three products).  AdamW is timed on up to 4 M
    elements of its units, G on up to 1 M elements of a quantised region; both
    scale by element count.  params/s = the workload's parameters / the
    extrapolated step time."""
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
    hp = oracle.OracleHyper()
    # a quick BLAS rate for choosing what runs in full
    a = np.random.default_rng(0).standard_normal((1024, 1024))
    t0 = time.perf_counter()
    _ = a @ a
    rate = 2 * 1024 ** 3 / max(time.perf_counter() - t0, 1e-6)
    shapes = {}
    for i, r in enumerate(res):
        if r["is_unit"] and r["optimizer"] == "muon":
            shapes.setdefault((r["rows"], r["cols"]), []).append(i)
    total, parts, measured = 0.0, [], 0.0
    for (rows, cols), units in shapes.items():
        r = res[units[0]]
        idx = unit_indices(r)
        rr, cc = min(rows, cols), max(rows, cols)
        ns_est = hp.ns_steps * (4 * rr * rr * cc + 2 * rr ** 3) / rate
        z = np.zeros(idx.shape, np.float32)
        if ns_est <= budget_s / max(len(shapes), 1):
            t0 = time.perf_counter()
            oracle.muon_update_unit(w0[idx], g[idx], z, hp)
            t_unit = time.perf_counter() - t0
            measured += t_unit
            how = "full"
        else:
            # the unit's update without Newton-Schulz steps (momentum, normalisation, weight
            # update), then one step's cost as NS(u, 1 step) - NS(u, 0 steps) on the same u
            t0 = time.perf_counter()
            oracle.muon_update_unit(w0[idx], g[idx], z, oracle.OracleHyper(ns_steps=0))
            t_elem = time.perf_counter() - t0
            u = oracle.momentum_step(z, g[idx], hp.momentum)[1]
            t = []
            for k in (0, 1):
                t0 = time.perf_counter()
                oracle.newton_schulz(u, k, hp.a, hp.b, hp.c, hp.ns_eps)
                t.append(time.perf_counter() - t0)
            measured += t_elem + sum(t)
            t_unit = t_elem + hp.ns_steps * max(t[1] - t[0], 0.0)
            how = "no NS step + one NS step"
        total += len(units) * t_unit
        parts.append(f"{len(units)} x {rows}x{cols} ({how}: {t_unit:.2f} s/unit)")
    adam = [r for r in res if r["is_unit"] and r["optimizer"] == "adamw"]
    if adam:
        n_all = sum(r["rows"] * r["cols"] for r in adam)
        done, t_adam = 0, 0.0
        for r in adam:
            if done >= 4_000_000:
                break
            idx = unit_indices(r)
            if idx.size > 4_000_000:
                idx = idx.ravel()[:4_000_000]
            z = np.zeros(idx.shape, np.float32)
            t0 = time.perf_counter()
            oracle.adamw_step(w0[idx], g[idx], z, z, 1, hp.adam_lr, hp.beta1, hp.beta2, hp.adam_eps, hp.adam_wd)
            t_adam += time.perf_counter() - t0
            done += idx.size
        measured += t_adam
        total += t_adam * n_all / done
        parts.append(f"AdamW {n_all} elements (timed on {done})")
    quant = [r for r in res if r["quantize"]]
    if quant:
        n_all = sum(r["rows"] * r["cols"] for r in quant)
        r = max(quant, key=lambda x: x["rows"] * x["cols"])
        rows = max(1, min(r["rows"], 1_000_000 // r["cols"]))
        sub = dict(r, rows=rows, extent=rows * r["cols"])
        n_s = (rows * r["cols"]) // 32 * 32
        codes = np.zeros(wl.root_numel, np.uint8)
        scales = np.zeros((wl.root_numel + 31) // 32 + 1, np.uint8)
        t0 = time.perf_counter()
        oracle.requant_root(w0, [sub], "rowmajor", codes, scales)
        t_q = time.perf_counter() - t0
        measured += t_q
        total += t_q * n_all / max(n_s, 1)
        parts.append(f"G {n_all} elements (timed on {n_s})")
    return {"value": wl.params / total, "unit": "params/s", "cores": int(threads), "kind": "oracle",
            "sample": f"extrapolated to one whole step ({total:.1f} s) from {measured:.1f} s of oracle work: "
                      + "; ".join(parts) + f"; NumPy fp64 on {backend}, {threads} BLAS threads",
            "seconds": measured}


def peak_clock_mhz():
    """The device's peak engine clock as the HIP runtime reports it (the clock
    it sustains under the large contractions is lower: see the MFMA counter
    summaries, which derive it from GRBM_GUI_ACTIVE)."""
    try:
        # by its soname, so the runtime torch has already loaded is the one asked
        hip = ctypes.CDLL("libamdhip64.so.7")
        v = ctypes.c_int(0)
        # hipDeviceAttributeClockRate (= 5 in hip_runtime_api.h), in kHz
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0:
            return v.value // 1000
    except OSError:  # pragma: no cover
        pass
    return None


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
            "peak_sclk_mhz": peak_clock_mhz(),
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


class Setup:
    """Device roots, plan and workspace of one workload (torch for memory only)."""

    def __init__(self, torch, sh, wl, args, layout=None, g_mode="mxfp8"):
        dev = "cuda:0"
        self.wl = wl
        w0, g0 = wl.arrays()
        self.layout = layout or wl.scale_layout
        nodes = wl.nodes
        if g_mode == "bf16":                      # every G region becomes a bfloat16 cast
            nodes = [dict(nd, quantize="bf16") if nd["quantize"] else nd for nd in nodes]
        self.plan = sh.Plan(nodes, wl.root_numel, layout=self.layout, ns_tiles=args.ns_tiles, ns_gram=args.ns_gram,
                            ns_streams=getattr(args, "ns_streams", "auto"))
        self.st = self.plan.stats()
        self.w = torch.from_numpy(w0).to(dev)
        self.g = torch.from_numpy(g0).to(dev)
        self.m = torch.zeros_like(self.w)
        self.v = torch.zeros_like(self.w) if self.st["n_adamw_units"] else None
        self.codes = torch.zeros(wl.root_numel, dtype=torch.uint8, device=dev)
        self.scales = torch.zeros(self.st["scale_bytes"], dtype=torch.uint8, device=dev)
        self.ws_bytes = max(int(self.st["workspace_bytes"]), 256)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.w16 = torch.empty(wl.root_numel, dtype=torch.bfloat16, device=dev) if g_mode == "bf16" else None
        self.bufs = sh.buffers(self.w, self.g, self.m, self.v, self.codes, self.scales, w_bf16=self.w16)
        self.mhp, self.ahp = sh.muon_hp(), sh.adamw_hp()
        self.sh = sh
        self.step_no = 0

    def step(self, sp):
        self.step_no += 1
        self.sh.update_step(self.plan, self.bufs, self.mhp, self.ahp, self.step_no, self.ws, self.ws_bytes, sp)

    def profiled(self, torch, sp, steps):
        """K steps with every kernel class bracketed by HIP events on its stream."""
        self.plan.profile(True)
        for _ in range(steps):
            self.step(sp)
        torch.cuda.synchronize()
        prof = self.plan.profile_read()
        self.plan.profile(False)
        return prof


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
    torch.cuda.set_device(0)
    wl = workloads.config(args.config)
    if args.part == "rs":
        return bench_rs(args, wl)
    S = Setup(torch, sh, wl, args, layout=args.layout, g_mode=args.g)
    st, layout = S.st, S.layout
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    for _ in range(args.warmup):
        S.step(sp)
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for k in range(args.steps):
        S.step(sp)
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
            S.sh.update_step(S.plan, S.bufs, S.mhp, S.ahp, S.step_no + 1, S.ws, S.ws_bytes, gstream.cuda_stream)
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
        S.step_no += 1 + args.warmup + args.steps
        del graph

    # per-kernel-class durations: HIP events bracketing every launch, same K steps
    prof = S.profiled(torch, sp, args.steps)
    components = {c: {"ms_per_step": prof[c][0] / args.steps, "launches_per_step": prof[c][1] / args.steps}
                  for c in prof if prof[c][1]}
    groups = S.plan.groups()
    roofline = ns_phase = None
    if st["n_muon_units"]:
        units_nz, exec_flops = S.plan.ns_executed(S.ws, S.ws_bytes, sp)
        # the dominant kernel: the 256-tile launch of the update product on the launch stream (steps
        # before the last); executed MFMA flops per launch = 2 r_pad per output element of the groups'
        # 256-tile regions, for every unit whose momentum is not all zero
        lane0 = [i for i, gi in enumerate(groups) if gi["lane"] == 0]
        upd_flops = sum(units_nz[i] * 2.0 * groups[i]["upd256_rows"] * groups[i]["upd256_cols"] * groups[i]["r_pad"]
                        for i in lane0)
        ms_upd, n_upd = prof["lane0_update"]
        if n_upd and upd_flops > 0:
            ms_launch = ms_upd / n_upd
            achieved = upd_flops / (ms_launch / 1e3) / 1e12
            names = ", ".join(f"{groups[i]['r']}x{groups[i]['c']} x{groups[i]['n_units']}" for i in lane0
                              if groups[i]["upd256_rows"])
            roofline = {"bound": "mfma",
                        "kernel": f"k_ns<2, 256-tile> update X' = aX + BX (groups {names}; launch stream)",
                        "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                        "traffic": measured_traffic(wl.name, "dominant"),
                        "tflop_per_launch": upd_flops / 1e12, "ms_per_launch": ms_launch,
                        "launches_per_step": n_upd / args.steps,
                        "timing": "HIP events bracketing each launch on its stream, profiled pass of K steps"}
        ns_ms = prof["ns_phase"][0] / args.steps if prof["ns_phase"][1] else 0.0
        if ns_ms > 0:
            ns_s = ns_ms / 1e3
            dense = sum(units_nz[i] * 5 * (4.0 * gi["r"] ** 2 * gi["c"] + 2.0 * gi["r"] ** 3)
                        for i, gi in enumerate(groups))
            ns_phase = {"bound": "mfma", "achieved": exec_flops / ns_s / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": exec_flops / ns_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                        "executed_tflop_per_step": exec_flops / 1e12,
                        "dense_tflop_per_step": dense / 1e12,
                        "effective_dense_tflops": dense / ns_s / 1e12, "ms": ns_ms,
                        "nonzero_units": int(sum(units_nz)), "units": st["n_muon_units"]}
    # G (and fused AdamW + G) against HBM: 4 (read w) + 1 (code) + 1/32 (scale) bytes per element,
    # plus 28 B/element of AdamW where it is fused
    per_scale = 1.0 / 1024 if layout == "block32x32" else 1.0 / 32

    def hbm_obj(prof_, st_, steps, kernel):
        rq_ms = prof_["requant"][0] + prof_["adamw_requant"][0]
        if rq_ms <= 0:
            return None
        fused = st_["fused_quant_elems"]
        byts = (st_["quant_elems"] - fused) * (5.0 + per_scale) + fused * (29.0 + per_scale)
        gbs = byts * steps / (rq_ms / 1e3) / 1e9
        return {"bound": "hbm", "kernel": kernel, "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "bytes_per_step": byts, "ms_per_launch": rq_ms / steps}

    g_roof = hbm_obj(prof, st, args.steps, "k_quant (G on the main workload)")
    repack = None
    repack_wl = None
    if args.config == args.repack_config:
        repack = hbm_obj(prof, st, args.steps, "k_quant<true> (AdamW + MXFP8 G fused)")
        repack_wl = wl
    elif args.repack_config:
        # the AdamW + MXFP8 half of the metric, on its own workload, in the same run
        del S
        torch.cuda.empty_cache()
        repack_wl = workloads.config(args.repack_config)
        R = Setup(torch, sh, repack_wl, argparse.Namespace(ns_tiles="auto", ns_gram="auto"))
        for _ in range(args.warmup):
            R.step(sp)
        torch.cuda.synchronize()
        rprof = R.profiled(torch, sp, args.steps)
        repack = hbm_obj(rprof, R.st, args.steps, "k_quant<true> (AdamW + MXFP8 G fused)")
        del R
    if repack is not None:
        repack["workload"] = repack_wl.name
        repack["traffic"] = measured_traffic(repack_wl.name, "repack")
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
                   "ns_groups": [[gi["r"], gi["c"], gi["n_units"]] for gi in groups],
                   "scale_layout": layout, "g": args.g, "ns_tiles": args.ns_tiles, "ns_gram": args.ns_gram,
                   "ns_streams": args.ns_streams,
                   "ns_tflop_per_step": st["ns_flops"] / 1e12,
                   "repack_workload": repack_wl.name if repack_wl is not None else None},
        "roofline": roofline, "ns_phase": ns_phase, "repack_roofline": repack, "g_roofline": g_roof,
        "cast_roofline": cast, "components": components, "graph_ms_per_step": graph_ms,
    }
    if roofline is None and ns_phase is not None:      # no 256-tile update launch (small workloads)
        roofline = dict(ns_phase, kernel="k_ns (every Newton-Schulz launch, NS phase wall time)",
                        traffic=measured_traffic(wl.name, "dominant"))
    out["roofline"] = roofline
    out["env"] = run_env(torch, wl)
    if not args.no_cpu:
        cb = cpu_baseline(wl, args.cpu_budget)
        cb.pop("seconds", None)
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
