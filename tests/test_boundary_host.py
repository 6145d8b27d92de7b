"""The C-ABI library on the host (no GPU): it loads, exports every function
include/sshdp.h declares, and its planner (run host-only) resolves offsets,
rejects bad trees with the error class of the oracle's rule list
[SS-HSDP Appendix A, Table 4] plus the library's own access rules
(tests/boundary_rules.py), and groups Muon units by oriented shape
[SS-HSDP §4.1].  No compute call is made."""

import os
import re

import numpy as np
import pytest

import mxfp8_weight_repack_amd as sh
from mxfp8_weight_repack_amd import _lib
import oracle
from oracle.views import ViewError
import workloads
from boundary_rules import expected_code

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "sshdp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(sshdp_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    decl = _declared()
    assert len(decl) >= 14
    L = sh.lib()
    for name in decl:
        assert hasattr(L, name), name
        assert name in _lib.SIGNATURES, name
    assert set(_lib.SIGNATURES) == set(decl)
    assert L.sshdp_abi_version() == 6
    assert L.sshdp_status_string(-5) == b"geometry or metadata the kernels cannot take"


def _plan(nodes, n, layout="rowmajor"):
    return sh.Plan(nodes, n, layout=layout, host_only=True)


def _random_tree(rng, N, blocks32=False):
    nodes = []
    for i in range(int(rng.integers(1, 7))):
        p = int(rng.integers(-1, i)) if i else -1
        if rng.uniform() < 0.05:
            p = int(rng.integers(-3, i + 2))
        rows = int(rng.integers(0 if rng.uniform() < 0.03 else 1, 6))
        if blocks32 and rng.uniform() < 0.5:
            rows = int(rng.choice([32, 64, 48]))
        cols = int(rng.choice([4, 8, 12, 32, 64, 96, 128, 5, 37]))
        rs = cols + int(rng.choice([0, 0, 0, 4, 32, -2]))
        off = int(rng.choice([0, 4, 8, 32, 64, 3, 128, 256] + ([1024, 2048, 3072] if blocks32 else [])))
        unit = rng.uniform() < 0.6
        opt = rng.choice(["muon", "adamw"]) if unit else None
        if unit and rng.uniform() < 0.03:
            opt = "sgd"
        q = rng.uniform() < 0.3
        nodes.append(dict(parent=p, offset=off, rows=rows, cols=cols, row_stride=rs, is_unit=unit,
                          optimizer=opt, quantize=q))
    return nodes


@pytest.mark.parametrize("layout", ["rowmajor", "tile32x4", "block32x32"])
def test_planner_agrees_with_oracle_rules_on_random_trees(layout):
    rng = np.random.default_rng({"rowmajor": 42, "tile32x4": 43, "block32x32": 44}[layout])
    n_ok = n_err = 0
    root = 16384 if layout == "block32x32" else 2048
    for _ in range(3000):
        nodes = _random_tree(rng, root, blocks32=layout == "block32x32")
        exp = expected_code(nodes, root, layout)
        if exp is None:
            res = oracle.resolve_views(nodes, root, layout)
        try:
            p = _plan(nodes, root, layout)
            got = None
        except sh.SshdpError as e:
            got = e.name
        assert got == exp, (nodes, got, exp)
        if exp is None:
            n_ok += 1
            for i, r in enumerate(res):
                assert p.node(i)[0] == r["abs"]
            st = p.stats()
            assert st["muon_elems"] == sum(r["rows"] * r["cols"] for r in res if r["optimizer"] == "muon")
            assert st["adamw_elems"] == sum(r["rows"] * r["cols"] for r in res if r["optimizer"] == "adamw")
            assert st["quant_elems"] == sum(r["rows"] * r["cols"] for r in res if r["quantize"])
        else:
            n_err += 1
    assert n_ok > 100 and n_err > 100


def test_planner_groups_and_stats_on_workloads():
    for cid in (1, 2, 3, 4, 5):
        wl = workloads.config(cid)
        p = _plan(wl.nodes, wl.root_numel, wl.scale_layout)
        st = p.stats()
        assert st["muon_elems"] + st["adamw_elems"] == wl.params
        assert st["scale_bytes"] == (wl.root_numel + 31) // 32
        shapes = {}
        for i, n in enumerate(wl.nodes):
            if n["is_unit"] and n["optimizer"] == "muon":
                key = (min(n["rows"], n["cols"]), max(n["rows"], n["cols"]))
                shapes[key] = shapes.get(key, 0) + 1
        got = {(g["r"], g["c"]): g["n_units"] for g in p.groups()}
        assert got == shapes
        flops = sum(cnt * 5 * (4 * r * r * c + 2 * r ** 3) for (r, c), cnt in shapes.items())
        assert abs(st["ns_flops"] - flops) <= 1e-9 * max(flops, 1)
        for g in p.groups():
            # padding to 128 only; 256-tiles cover the largest 256-aligned leading block or nothing
            assert g["r_pad"] % 128 == 0 and g["c_pad"] % 128 == 0
            assert 0 <= g["r_pad"] - g["r"] < 128 and 0 <= g["c_pad"] - g["c"] < 128
            assert g["gram256"] in (0, g["r_pad"] // 256 * 256)
            assert (g["upd256_rows"], g["upd256_cols"]) in ((0, 0), (g["r_pad"] // 256 * 256, g["c_pad"] // 256 * 256))
            assert g["tile"] == (256 if g["upd256_rows"] else 128)
            assert g["tile_gram"] == (256 if g["gram256"] else 128)
    # the MoE bank (r = 1408): update in 256-tiles over the leading 1280 rows plus a 128-tile
    # strip, Gram/poly in 128-tiles, no padding
    wl = workloads.config(3)
    (g,) = _plan(wl.nodes, wl.root_numel, "tile32x4").groups()
    assert (g["r_pad"], g["c_pad"], g["gram256"], g["upd256_rows"], g["upd256_cols"]) == (1408, 2048, 0, 1280, 2048)
    for pol, want in (("small", (0, 0, 0)), ("large", (1280, 1280, 2048))):
        (g,) = sh.Plan(wl.nodes, wl.root_numel, layout="tile32x4", host_only=True, ns_tiles=pol).groups()
        assert (g["gram256"], g["upd256_rows"], g["upd256_cols"]) == want
    # the flat shard's requant is fused with AdamW everywhere; the dense block's is not
    wl = workloads.config(4, small=True)
    st = _plan(wl.nodes, wl.root_numel).stats()
    assert st["fused_quant_elems"] == st["quant_elems"] == wl.root_numel
    wl = workloads.config(2, small=True)
    st = _plan(wl.nodes, wl.root_numel, "tile32x4").stats()
    assert st["fused_quant_elems"] == 0
    # one scale per 32x32 block: 1/1024 of the root, never fused with AdamW
    for cid in (1, 2, 3, 5):
        wl = workloads.config(cid)
        st = _plan(wl.nodes, wl.root_numel, "block32x32").stats()
        assert st["scale_bytes"] == (wl.root_numel + 1023) // 1024 and st["fused_quant_elems"] == 0
    wl = workloads.config(4, small=True)
    with pytest.raises(sh.SshdpError) as e:
        _plan(wl.nodes, wl.root_numel, "block32x32")
    assert e.value.name == "SCHEMA"


def test_planner_fuses_g_only_beside_adamw_units():
    """A quantised region is fused into the AdamW pass only when AdamW units lie
    in it; a region holding no unit gets plain G."""
    st = _plan(workloads.degenerate("g_only").nodes, workloads.degenerate("g_only").root_numel, "rowmajor").stats()
    assert st["n_quant_regions"] == 2 and st["quant_elems"] == 64 * 256 + 3 * 96 and st["fused_quant_elems"] == 0
    wl = workloads.degenerate("adamw_g")
    st = _plan(wl.nodes, wl.root_numel, "rowmajor").stats()
    assert st["n_adamw_units"] == 1 and st["quant_elems"] == 4 * 224 + 32 * 128 and st["fused_quant_elems"] == 4 * 224
    wl = workloads.degenerate("muon_only")
    st = _plan(wl.nodes, wl.root_numel, "rowmajor").stats()
    assert st["n_muon_units"] == 2 and st["n_adamw_units"] == 0 and st["quant_elems"] == 0


def _one_unit(rows, cols):
    return [dict(parent=-1, offset=0, rows=rows, cols=cols, row_stride=cols, is_unit=True, optimizer="muon",
                 quantize=False)]


def test_planner_ns_size_limits_and_gram_operand():
    """A Muon unit's edges stop where a 256-row bf16 operand panel reaches 2^31
    bytes; a 128-tile Gram reads X^T only while all of X^T (c_pad x r_pad) is
    addressable with 32-bit byte offsets, else X; ns_gram="nt" reads X always."""
    edge = 4194176                                   # largest multiple of 128 with 256 * edge * 2 < 2^31
    assert 256 * edge * 2 < 2 ** 31 <= 256 * (edge + 128) * 2
    for rows, cols in ((128, edge + 4), (edge + 4, 128)):
        with pytest.raises(sh.SshdpError) as e:
            _plan(_one_unit(rows, cols), rows * cols)
        assert e.value.name == "SCHEMA"
    assert _plan(_one_unit(128, edge), 128 * edge).group(0)["gram_kmajor"] == 1
    # X^T of 1024 x 1048576 ends below byte 2^31; of 1024 x 1048704 it does not
    for cols, km in ((1048576, 1), (1048704, 0)):
        g = _plan(_one_unit(1024, cols), 1024 * cols).group(0)
        assert (g["r_pad"], g["c_pad"], g["gram256"], g["gram_kmajor"]) == (1024, cols, 0, km)
        assert ((cols - 1) * 1024 * 2 + 512 < 2 ** 31) == bool(km)
    wl = workloads.config(2)
    assert [g["gram_kmajor"] for g in _plan(wl.nodes, wl.root_numel).groups()] == [1, 1, 1]
    nt = sh.Plan(wl.nodes, wl.root_numel, host_only=True, ns_gram="nt")
    assert [g["gram_kmajor"] for g in nt.groups()] == [0, 0, 0]
    assert nt.stats()["workspace_bytes"] > _plan(wl.nodes, wl.root_numel).stats()["workspace_bytes"]
    wl = workloads.config(5)
    assert [(g["gram256"] > 0, g["gram_kmajor"]) for g in _plan(wl.nodes, wl.root_numel).groups()] == \
        [(False, 1), (True, 0), (True, 0)]
    with pytest.raises(sh.SshdpError) as e:
        sh.Plan(wl.nodes, wl.root_numel, host_only=True, ns_gram="bogus")
    assert e.value.name == "ARG"


def test_raw_contraction_size_limits():
    """The raw contraction refuses operand panels that one buffer resource
    cannot address, before touching any pointer (the pointers here are fake)."""
    fake = 1 << 12
    cases = [(256, 256, 1 << 23, 256), (128, 128, 1 << 24, 128),      # tile * K * 2 = 2^32
             (2048, 2048, 1 << 20, 1281), (2048, 2048, 1 << 20, 2561)]   # ((K - 1) * M + tile) * 2 > 2^31
    for M, N, K, tile in cases:
        # every case must be refused: a case the library accepted would launch on the fake pointers
        span = tile * K * 2 if tile in (128, 256) else ((K - 1) * M + tile // 10) * 2
        assert span >= 2 ** 31, (M, N, K, tile)
        with pytest.raises(sh.SshdpError) as e:
            sh.gemm_bf16_nt(fake, fake, None, fake, None, M, N, K, 1, 1.0, 0.0, tile)
        assert e.value.name == "SCHEMA", (M, N, K, tile)


def test_planner_argument_errors():
    wl = workloads.config(1)
    with pytest.raises(sh.SshdpError) as e:
        sh.Plan(wl.nodes, wl.root_numel, ns_steps=0, host_only=True)
    assert e.value.name == "ARG"
    with pytest.raises(sh.SshdpError) as e:
        sh.Plan([], 10, host_only=True)
    assert e.value.name == "ARG"
    for bad in ("bogus", None):                      # unknown policy; both tile flags set
        with pytest.raises(sh.SshdpError) as e:
            sh.Plan(wl.nodes, wl.root_numel, host_only=True, ns_tiles=bad)
        assert e.value.name == "ARG"
    p = _plan(wl.nodes, wl.root_numel, "tile32x4")
    # a host-only plan refuses to launch, before touching any pointer
    b = sh.buffers(8, 16, 32, 48, 64, 80)
    with pytest.raises(sh.SshdpError) as e:
        sh.update_step(p, b, sh.muon_hp(), sh.adamw_hp(), 1, 0, 0)
    assert e.value.name == "STATE"
    with pytest.raises(sh.SshdpError) as e:
        sh.requant_mxfp8(p, 16, 32, 48)
    assert e.value.name == "STATE"
    p.destroy()
    p.destroy()


def test_planner_stream_rule_and_split_pairs():
    """Newton-Schulz groups and the streams they run on.  The largest group is on
    the caller's stream (lane 0).  While it leaves workgroup slots idle (the d=2048
    block's MLP Gram), the other groups share one side stream; when it fills the
    GPU at least twice over in every stage (the d=8192 block), only the per-head
    groups (r_pad = 128) leave lane 0.  A one-stream plan keeps every group on
    lane 0.  Exactly the groups of one 128-row tile hold B as a bf16 pair."""
    def lanes(cid, streams="auto", small=False):
        wl = workloads.config(cid, small=small)
        p = sh.Plan(wl.nodes, wl.root_numel, layout=wl.scale_layout, host_only=True, ns_streams=streams)
        gs = p.groups()
        for g in gs:
            assert g["split_b"] == (g["r_pad"] == 128), g
        return {(g["r"], g["c"]): g["lane"] for g in gs}

    assert lanes(2) == {(128, 2048): 1, (2048, 2048): 1, (2048, 8192): 0}
    assert lanes(5) == {(128, 8192): 1, (8192, 8192): 0, (8192, 28672): 0}
    assert lanes(3) == {(1408, 2048): 0}
    assert lanes(5, small=True) == {(128, 512): 1, (512, 512): 1, (512, 1536): 0}
    for cid in (1, 2, 3, 5):
        assert set(lanes(cid, "one").values()) == {0}
