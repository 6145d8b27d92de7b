"""Seeded synthetic workloads for the update phase: view tables and root arrays.

Shared by the tests (which feed the same arrays to the oracle and to the HIP
library) and by bench.py.  It holds none of the method's arithmetic: only
shapes, offsets and seeded random draws.

Shapes follow the workloads of the SS-HSDP page (per-head QKV views inside one
packed projection, [SS-HSDP §3.1 EG1]; dense blocks and MoE expert banks,
[SS-HSDP Appendix B.1, Table 5], whose inputs are synthetic too) and, for the
flat ragged shard, the veScale page's rule of padding only between tensors to
block boundaries [veScale §5].

Random numbers: numpy Generator(PCG64(SeedSequence([config_id, stream]))),
stream 0 = main weights, 1 = gradients, 2 = structure (expert choice, ragged
sizes), 16 + t = the fresh gradient of step t > 1 in multi-step tests.  w ~ N(0, 0.02^2), g ~ N(0, 1e-3^2), momentum and second moment zero,
padding zero in every field.
"""

from dataclasses import dataclass, field
import math

import numpy as np

W_STD = 0.02
G_STD = 1e-3


def rng(config_id, stream):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config_id, stream])))


@dataclass
class Workload:
    name: str
    config_id: int
    nodes: list
    root_numel: int
    scale_layout: str
    params: int                      # elements owned by units (padding excluded)
    zero_grad_units: list = field(default_factory=list)   # node indices with g == 0
    padding: list = field(default_factory=list)           # (start, length) of padding runs
    _arrays: dict = field(default_factory=dict, repr=False)

    def units(self, opt=None):
        return [i for i, n in enumerate(self.nodes)
                if n["is_unit"] and (opt is None or n["optimizer"] == opt)]

    def arrays(self):
        """(w, g) float32 roots, generated once from the config's seeds."""
        if not self._arrays:
            w = rng(self.config_id, 0).standard_normal(self.root_numel, dtype=np.float32)
            w *= np.float32(W_STD)
            for s, n in self.padding:
                w[s:s + n] = 0
            self._arrays = {"w": w, "g": self._draw_gradient(rng(self.config_id, 1))}
        return self._arrays["w"], self._arrays["g"]

    def gradient(self, t):
        """The gradient root of step t (t >= 1): step 1 is arrays()'s, every later
        step a fresh draw from stream 16 + t, with the same zero padding and
        zero-gradient units."""
        if t == 1:
            return self.arrays()[1]
        return self._draw_gradient(rng(self.config_id, 16 + t))

    def _draw_gradient(self, gen):
        g = gen.standard_normal(self.root_numel, dtype=np.float32)
        g *= np.float32(G_STD)
        for s, n in self.padding:
            g[s:s + n] = 0
        for i in self.zero_grad_units:
            nd = self.nodes[i]
            a = _abs_offset(self.nodes, i)
            for r in range(nd["rows"]):
                s = a + r * nd["row_stride"]
                g[s:s + nd["cols"]] = 0
        return g


def _abs_offset(nodes, i):
    a = 0
    while i >= 0:
        a += nodes[i]["offset"]
        i = nodes[i]["parent"]
    return a


class _Tree:
    """Appends nodes to a packed root; every top-level region starts 32-aligned."""

    def __init__(self):
        self.nodes = []
        self.top = 0            # next free element of the root
        self.padding = []

    def node(self, parent, offset, rows, cols, unit=False, opt=None, quant=False, row_stride=None):
        self.nodes.append(dict(parent=parent, offset=int(offset), rows=int(rows), cols=int(cols),
                               row_stride=int(row_stride if row_stride is not None else cols),
                               is_unit=bool(unit), optimizer=opt if unit else None,
                               quantize=bool(quant)))
        return len(self.nodes) - 1

    def region(self, rows, cols, unit=False, opt=None, quant=False, pad_to=32):
        start = self.top
        i = self.node(-1, start, rows, cols, unit, opt, quant)
        end = start + rows * cols
        padded = -(-end // pad_to) * pad_to
        if padded > end:
            self.padding.append((end, padded - end))
        self.top = padded
        return i


def dense_block(cid, name, d, n_heads, head_dim, n_kv, ffn, n_norms, quant_all, layout):
    """Attention (+ optional MLP) block: packed QKV split into per-head Muon
    units, O projection and MLP matrices as whole-matrix Muon units, norm
    vectors under AdamW."""
    t = _Tree()
    nq = n_heads + 2 * n_kv
    qkv = t.region(nq * head_dim, d, quant=True)
    for h in range(nq):
        t.node(qkv, h * head_dim * d, head_dim, d, unit=True, opt="muon")
    t.region(n_heads * head_dim, d, unit=True, opt="muon", quant=quant_all)   # O: [d, H*hd] as rows x K
    if ffn:
        t.region(ffn, d, unit=True, opt="muon", quant=quant_all)    # gate  (tall)
        t.region(ffn, d, unit=True, opt="muon", quant=quant_all)    # up    (tall)
        t.region(d, ffn, unit=True, opt="muon", quant=quant_all)    # down  (wide)
    for _ in range(n_norms):
        t.region(1, d, unit=True, opt="adamw")
    return _finish(cid, name, t, layout)


def moe_layer(cid, name, n_exp, d, ffn, n_zero, layout):
    """Expert bank: gate/up [E, ffn, d] and down [E, d, ffn] packed per expert,
    each expert matrix a Muon unit; router [E, d] under AdamW; n_zero experts
    (chosen on the structure stream) get an exactly zero gradient."""
    t = _Tree()
    zero = sorted(rng(cid, 2).choice(n_exp, n_zero, replace=False).tolist()) if n_zero else []
    zunits = []
    for rows, cols in ((ffn, d), (ffn, d), (d, ffn)):
        bank = t.region(n_exp * rows, cols, quant=True)
        for e in range(n_exp):
            u = t.node(bank, e * rows * cols, rows, cols, unit=True, opt="muon")
            if e in zero:
                zunits.append(u)
    t.region(n_exp, d, unit=True, opt="adamw")
    wl = _finish(cid, name, t, layout)
    wl.zero_grad_units = zunits
    return wl


def flat_shard(cid, name, total, lo=4096, hi=50_000_000, frac2d=0.9,
               ks=(256, 512, 1024, 2048, 4096, 8192)):
    """Flat AdamW shard of exactly ``total`` elements built from ragged tensors,
    sizes log-uniform in [lo, hi]; 2-D tensors [max(1, s//K), K], 1-D tensors
    padded to the next multiple of 32; the last 1-D tensor fills the rest.
    Every tensor is requantised (1 x 32 blocks along its contiguous dim)."""
    assert total % 32 == 0
    r = rng(cid, 2)
    t = _Tree()
    while True:
        s = int(round(math.exp(r.uniform(math.log(lo), math.log(hi)))))
        if r.uniform() < frac2d:
            K = int(ks[r.integers(len(ks))])
            rows, cols, padded = max(1, s // K), K, max(1, s // K) * K
        else:
            rows, cols, padded = 1, s, -(-s // 32) * 32
        if t.top + padded > total:
            break
        if rows > 1 or cols % 32 == 0:
            t.region(rows, cols, unit=True, opt="adamw", quant=True)
        else:
            q = t.region(1, padded, quant=True)
            t.node(q, 0, 1, cols, unit=True, opt="adamw")
            t.padding.append((t.top - padded + cols, padded - cols))
    rest = total - t.top
    if rest:
        t.region(1, rest, unit=True, opt="adamw", quant=True)
    assert t.top == total
    return _finish(cid, name, t, "rowmajor")


def ragged_mix(cid=100, name="ragged mix (odd shapes, strided views)"):
    """Small mixed tree whose shapes span several tiles with ragged tails:
    wide and tall Muon units not multiple of any tile, strided column views
    (per-head slices of an output projection), odd-length AdamW vectors, and a
    Muon and an AdamW unit whose gradient is exactly zero."""
    t = _Tree()
    qkv = t.region(6 * 48, 160, quant=True)                      # 6 heads of 48 x 160
    for h in range(6):
        t.node(qkv, h * 48 * 160, 48, 160, unit=True, opt="muon")
    t.region(201, 72, unit=True, opt="muon", quant=False)        # tall, ragged
    t.region(135, 328, unit=True, opt="muon", quant=False)       # wide, ragged
    o = t.region(96, 128, quant=True)                            # O proj, two column-half views
    t.node(o, 0, 96, 64, unit=True, opt="muon", row_stride=128)
    t.node(o, 64, 96, 64, unit=True, opt="muon", row_stride=128)
    t.region(1, 37, unit=True, opt="adamw")                      # odd 1-D, padded to 64
    t.region(3, 224, unit=True, opt="adamw", quant=True)
    s = t.region(5, 48)                                          # strided AdamW column view
    t.node(s, 8, 5, 20, unit=True, opt="adamw", row_stride=48)
    t.region(40, 64, unit=True, opt="muon", quant=True)          # 40 x 64 zero-grad unit
    zmuon = len(t.nodes) - 1
    t.region(2, 96, unit=True, opt="adamw", quant=True)          # zero-grad AdamW unit (decay only, G fused)
    wl = _finish(cid, name, t, "rowmajor")
    wl.zero_grad_units = [zmuon, len(t.nodes) - 1]
    return wl


def mixed_tiles(cid=101, name="odd multiples of 128 (256-tile blocks with 128-tile strips)"):
    """Muon units whose padded edges are odd multiples of 128, so a plan with
    256-tiles covers each product's 256-aligned leading block and leaves a
    128-wide strip: wide 320 x 500 (x2), tall 700 x 384, and 130 x 260."""
    t = _Tree()
    t.region(320, 500, unit=True, opt="muon")
    t.region(320, 500, unit=True, opt="muon")
    t.region(700, 384, unit=True, opt="muon", quant=True)
    t.region(130, 260, unit=True, opt="muon")
    t.region(1, 96, unit=True, opt="adamw", quant=True)
    return _finish(cid, name, t, "rowmajor")


def long_k_units(cid=105, name="4096 x 4224 wide and 4224 x 4096 tall Muon units"):
    """Two Muon units of one oriented shape, r = 4096, c = 4224: large enough
    that the default plan runs the Gram and polynomial in 256-tiles (with a
    128 strip, c_pad = 4224) and the update with K = 4096, the long-K update's
    tile order; small enough for the float64 oracle (about 2 TFLOP each)."""
    t = _Tree()
    t.region(4096, 4224, unit=True, opt="muon", quant=True)
    t.region(4224, 4096, unit=True, opt="muon", quant=True)
    t.region(1, 4096, unit=True, opt="adamw")
    return _finish(cid, name, t, "tile32x4")


def longest_edge_units(cid=106, name="2 x 4194176 wide and 4194176 x 4 tall Muon units"):
    """Muon units at the longest edge the library takes (4194176, the largest
    multiple of 128 whose 256-row operand panels stay within 32-bit byte
    offsets), wide (quantised) and tall, beside an AdamW vector: the Gram then
    runs one 128-tile per unit over K = 4194176 and the update 32767 tiles."""
    t = _Tree()
    t.region(2, 4194176, unit=True, opt="muon", quant=True)
    t.region(4194176, 4, unit=True, opt="muon")
    t.region(1, 4096, unit=True, opt="adamw")
    return _finish(cid, name, t, "rowmajor")


def random_units(cid=102, n=6, name="random Muon shapes"):
    """n Muon units of random shapes (rows, cols in [2, 640], cols a multiple
    of 4, drawn on the structure stream), wide and tall, each its own region,
    plus one AdamW vector: shapes that land anywhere relative to the 128- and
    256-tile grids."""
    r = rng(cid, 2)
    t = _Tree()
    for _ in range(n):
        rows = int(r.integers(2, 641))
        cols = int(r.integers(1, 161)) * 4
        t.region(rows, cols, unit=True, opt="muon")
    t.region(1, 100, unit=True, opt="adamw")
    return _finish(cid, name, t, "rowmajor")


def degenerate(kind):
    """Plans with a whole optimizer or G missing.  "g_only": quantised regions
    that hold no unit (G alone); "muon_only": Muon units, nothing quantised, no
    AdamW; "adamw_g": an AdamW unit inside a quantised region (G fused into the
    AdamW pass) beside a quantised region with no unit (plain G)."""
    t = _Tree()
    if kind == "g_only":
        t.region(64, 256, quant=True)
        t.region(3, 96, quant=True)
        return _finish(110, "G only (quantised regions, no units)", t, "rowmajor")
    if kind == "muon_only":
        t.region(48, 160, unit=True, opt="muon")
        t.region(201, 72, unit=True, opt="muon")
        return _finish(111, "Muon only (no AdamW, nothing quantised)", t, "rowmajor")
    if kind == "adamw_g":
        t.region(4, 224, unit=True, opt="adamw", quant=True)
        t.region(32, 128, quant=True)
        return _finish(112, "AdamW + G beside a unit-less quantised region", t, "rowmajor")
    raise ValueError(kind)


def _finish(cid, name, t, layout):
    params = 0
    for n in t.nodes:
        if n["is_unit"]:
            params += n["rows"] * n["cols"]
    return Workload(name=name, config_id=cid, nodes=t.nodes, root_numel=t.top,
                    scale_layout=layout, params=params, padding=t.padding)


def config(cid, small=False):
    """The five workloads (c1..c5) at full size, or a downsized twin (small=True)
    with the same structure for oracle-speed parity tests."""
    if cid == 1:
        return dense_block(1, "tiny attention block d=256, 4 heads x 64", 256, 4, 64, 4, 0, 1,
                           False, "tile32x4")
    if cid == 2:
        if small:
            return dense_block(12, "dense block d=256, 4 heads x 64, 2 KV, ffn 640", 256, 4, 64, 2,
                               640, 2, True, "tile32x4")
        return dense_block(2, "dense block d=2048, 16 heads x 128, 4 KV, ffn 8192", 2048, 16, 128, 4,
                           8192, 2, True, "tile32x4")
    if cid == 3:
        if small:
            return moe_layer(13, "MoE 8 experts d=256 ffn 384", 8, 256, 384, 2, "tile32x4")
        return moe_layer(3, "MoE 64 experts d=2048 ffn 1408", 64, 2048, 1408, 16, "tile32x4")
    if cid == 4:
        if small:
            return flat_shard(14, "flat ragged shard 4e6", 4_000_000, lo=256, hi=400_000)
        return flat_shard(4, "flat ragged shard 5e8", 500_000_000)
    if cid == 5:
        if small:
            return dense_block(15, "dense block d=512, 4 heads x 128, 1 KV, ffn 1536", 512, 4, 128, 1,
                               1536, 0, True, "tile32x4")
        return dense_block(5, "dense block d=8192, 64 heads x 128, 8 KV, ffn 28672", 8192, 64, 128, 8,
                           28672, 0, True, "tile32x4")
    raise ValueError(cid)
