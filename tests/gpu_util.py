"""Helpers for the GPU parity tests: upload a workload's seeded roots, run the
HIP library through its C ABI, and run the oracle on the same host arrays."""

import sys

import numpy as np

import oracle
import mxfp8_weight_repack_amd as sh

MUON = dict(lr=0.02, momentum=0.95, weight_decay=0.0)
ADAM = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class DeviceState:
    """Device roots for one workload (torch is used for memory and streams only)."""

    def __init__(self, wl, w=None, g=None, m=None, v=None, layout=None, plan_kw=None):
        import torch
        self.torch = torch
        self.wl = wl
        self.layout = layout or wl.scale_layout
        w0, g0 = wl.arrays()
        w = w0 if w is None else w
        g = g0 if g is None else g
        dev = "cuda"
        self.plan = sh.Plan(wl.nodes, wl.root_numel, layout=self.layout, **(plan_kw or {}))
        self.stats = self.plan.stats()
        self.w = torch.from_numpy(np.ascontiguousarray(w)).to(dev)
        self.g = torch.from_numpy(np.ascontiguousarray(g)).to(dev)
        self.m = torch.zeros_like(self.w) if m is None else torch.from_numpy(m).to(dev)
        self.v = torch.zeros_like(self.w) if v is None else torch.from_numpy(v).to(dev)
        self.codes = torch.zeros(wl.root_numel, dtype=torch.uint8, device=dev)
        self.scales = torch.zeros(self.stats["scale_bytes"], dtype=torch.uint8, device=dev)
        self.ws_bytes = max(int(self.stats["workspace_bytes"]), 256)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        assert self.ws.data_ptr() % 256 == 0

    def bufs(self):
        return sh.buffers(self.w, self.g, self.m, self.v, self.codes, self.scales)

    def stream(self):
        return self.torch.cuda.current_stream().cuda_stream

    def step(self, t=1, muon=None, adam=None):
        sh.update_step(self.plan, self.bufs(), sh.muon_hp(**(muon or MUON)), sh.adamw_hp(**(adam or ADAM)), t,
                       self.ws, self.ws_bytes, self.stream())

    def host(self):
        self.torch.cuda.synchronize()
        return {k: getattr(self, k).cpu().numpy() for k in ("w", "m", "v", "codes", "scales")}


def oracle_step(wl, layout, w, g, m, v, step=1, hp=None, **kw):
    """Run the oracle on copies of the host arrays; returns the new state and
    the per-unit float64 Newton-Schulz directions."""
    w = w.copy(); m = m.copy(); v = v.copy()
    codes = np.zeros(wl.root_numel, np.uint8)
    scales = np.zeros((wl.root_numel + 1023) // 1024 if layout == "block32x32" else (wl.root_numel + 31) // 32,
                      np.uint8)
    dirs = oracle.update_step(wl.nodes, wl.root_numel, w, g, m, v, codes, scales, step, hp=hp,
                              layout=layout, keep_v=True, **kw)
    return dict(w=w, m=m, v=v, codes=codes, scales=scales), dirs


def adam_elementwise_ok(w_gpu, w_ref, lr=ADAM["lr"]):
    """The elementwise AdamW bound beside the normwise one: every element within
    1e-6 of its own magnitude plus 4 float32 units of the step size,
    |w_gpu - w_ref| <= 1e-6 |w_ref| + 4 lr 2^-24 (the additive term covers
    elements near zero, where a relative bound alone is ill-posed).  Returns
    the worst ratio of error to bound (<= 1 passes)."""
    w_gpu = np.asarray(w_gpu, np.float64)
    w_ref = np.asarray(w_ref, np.float64)
    bound = 1e-6 * np.abs(w_ref) + 4.0 * np.float64(np.float32(lr)) * 2.0 ** -24
    return float(np.max(np.abs(w_gpu - w_ref) / bound)) if w_ref.size else 0.0


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
