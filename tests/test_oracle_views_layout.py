"""Pins for the oracle's data-tree views, scale layouts and the zero-copy
identity of the packed runtime weight (CPU only).

* offsets: numpy's own strided views of an arange root (a library routine that
  resolves chained views independently of resolve_views);
* planner rules [SS-HSDP Appendix A, Table 4]: every error class is triggered;
* zero-copy [SS-HSDP §3.2, §4.2]: the packed QKV view's bytes are exactly the
  concatenation of its head views' bytes, and requantising per head equals
  requantising the packed projection, byte for byte, in both scale layouts;
* the tile32x4 layout is a bijection onto its region (inverse map round trip).
"""

import numpy as np
import pytest

import oracle
from oracle.views import resolve_views, unit_indices, ViewError
from oracle.mxfp8 import quantize_blocks_fast, scale_index, requant_root
import workloads


def _node(parent, offset, rows, cols, row_stride=None, unit=False, opt=None, quant=False):
    return dict(parent=parent, offset=offset, rows=rows, cols=cols,
                row_stride=cols if row_stride is None else row_stride,
                is_unit=unit, optimizer=opt if unit else None, quantize=quant)


def test_offsets_match_numpy_chained_views():
    rng = np.random.default_rng(0)
    N = 5000
    root = np.arange(N, dtype=np.int64)
    for trial in range(200):
        nodes, views = [], []
        for i in range(6):
            p = int(rng.integers(-1, i)) if i else -1
            pv = root if p < 0 else views[p].ravel() if views[p].flags.c_contiguous else None
            if pv is None:
                p, pv = -1, root
            L = pv.size
            rows = int(rng.integers(1, 5))
            cols = int(rng.integers(1, 8))
            rs = cols + int(rng.integers(0, 4))
            ext = (rows - 1) * rs + cols
            if ext > L:
                rows, rs, ext = 1, cols, cols
                if cols > L:
                    cols = ext = rs = L
            off = int(rng.integers(0, L - ext + 1))
            base = pv[off:off + ext]
            v = np.lib.stride_tricks.as_strided(base, (rows, cols), (rs * 8, 8))
            nodes.append(_node(p, off, rows, cols, rs))
            views.append(v if rows > 1 else v.reshape(1, cols))
        res = resolve_views(nodes, N)
        for r, v in zip(res, views):
            assert np.array_equal(unit_indices(r), v)


@pytest.mark.parametrize("nodes,code", [
    ([], "ARG"),
    ([_node(1, 0, 2, 2), _node(-1, 0, 2, 2)], "TREE"),
    ([_node(-1, 0, 2, 2), _node(1, 0, 2, 2)], "TREE"),
    ([_node(-1, 0, 0, 4)], "SCHEMA"),
    ([_node(-1, 0, 3, 8, row_stride=4)], "SCHEMA"),
    ([_node(-1, 90, 2, 8)], "BOUNDS"),
    ([_node(-1, 0, 4, 8), _node(0, 8, 4, 8)], "BOUNDS"),
    ([_node(-1, 0, 1, 64, unit=True, opt="muon")], "SCHEMA"),
    ([_node(-1, 0, 2, 16, unit=True, opt="sgd")], "SCHEMA"),
    ([_node(-1, 0, 1, 48, quant=True)], "SCHEMA"),
    ([_node(-1, 16, 1, 32, quant=True)], "SCHEMA"),
    ([_node(-1, 0, 2, 32, row_stride=40, quant=True)], "SCHEMA"),
    ([_node(-1, 0, 4, 8, unit=True, opt="adamw"), _node(-1, 24, 2, 8, unit=True, opt="adamw")],
     "OVERLAP"),
    ([_node(-1, 0, 2, 32, quant=True), _node(-1, 32, 1, 32, quant=True)], "OVERLAP"),
])
def test_planner_rejections(nodes, code):
    with pytest.raises(ViewError) as e:
        resolve_views(nodes, 100 if nodes else 0)
    assert e.value.code == code


def test_vector_alignment_is_a_library_rule_not_the_methods():
    """A Muon unit at an odd offset or with cols not a multiple of 4 is a valid
    view for the method (the oracle takes it); only the library, whose rows
    move in 16-byte vectors, refuses it (tests/boundary_rules.py)."""
    from boundary_rules import expected_code
    for nd in (_node(-1, 2, 4, 8, unit=True, opt="muon"), _node(-1, 0, 4, 6, unit=True, opt="muon")):
        res = resolve_views([nd], 100)
        assert res[0]["optimizer"] == "muon"
        assert expected_code([nd], 100) == "SCHEMA"


def test_tile32x4_requires_tile_shape():
    with pytest.raises(ViewError) as e:
        resolve_views([_node(-1, 0, 32, 64, quant=True)], 4096, "tile32x4")
    assert e.value.code == "SCHEMA"
    resolve_views([_node(-1, 0, 32, 128, quant=True)], 4096, "tile32x4")


def test_strided_units_do_not_overlap_when_interleaved():
    nodes = [_node(-1, 0, 4, 64),
             _node(0, 0, 4, 32, row_stride=64, unit=True, opt="muon"),
             _node(0, 32, 4, 32, row_stride=64, unit=True, opt="muon")]
    res = resolve_views(nodes, 256)
    idx = np.concatenate([unit_indices(res[1]).ravel(), unit_indices(res[2]).ravel()])
    assert np.array_equal(np.sort(idx), np.arange(256))


@pytest.mark.parametrize("layout", ["rowmajor", "tile32x4"])
def test_tile_layouts_are_bijections(layout):
    for N, K in [(32, 128), (64, 256), (96, 1408), (128, 2048)]:
        idx = scale_index(layout, 4096, N, K)
        assert np.array_equal(np.sort(idx.ravel()), 128 + np.arange(N * K // 32))
        # inverse map: block index -> (n, kb)
        inv = np.empty(N * K // 32, dtype=np.int64)
        inv[idx.ravel() - 128] = np.arange(N * K // 32)
        assert np.array_equal(inv[idx.ravel() - 128], np.arange(N * K // 32))


@pytest.mark.parametrize("layout", ["rowmajor", "tile32x4"])
def test_zero_copy_packed_qkv_equals_head_views(layout):
    wl = workloads.config(2, small=True)
    w, _ = wl.arrays()
    res = resolve_views(wl.nodes, wl.root_numel, layout)
    qkv = res[0]
    heads = [r for r in res if r["parent"] == 0]
    # packed weight bytes == concatenation of head views
    packed = w[unit_indices(qkv)]
    cat = np.concatenate([w[unit_indices(h)] for h in heads], axis=0)
    assert np.shares_memory(w[qkv["abs"]:qkv["abs"] + qkv["extent"]], w)
    assert np.array_equal(packed, cat)
    # requant of the packed projection == per-head requant into the same roots
    c1 = np.zeros(wl.root_numel, np.uint8)
    s1 = np.zeros(wl.root_numel // 32, np.uint8)
    requant_root(w, [qkv], layout, c1, s1)
    c2 = np.zeros_like(c1)
    s2 = np.zeros_like(s1)
    for h in heads:
        hc, hs = quantize_blocks_fast(w[unit_indices(h)])
        c2[unit_indices(h)] = hc
        s2[scale_index(layout, qkv["abs"], qkv["rows"], qkv["cols"])[
            (h["abs"] - qkv["abs"]) // qkv["cols"]:(h["abs"] - qkv["abs"]) // qkv["cols"] + h["rows"]]] = hs
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    if layout == "tile32x4":
        # a head of 64 rows owns a contiguous run of the scale root
        h = heads[1]
        r0 = (h["abs"] - qkv["abs"]) // qkv["cols"]
        idx = scale_index(layout, qkv["abs"], qkv["rows"], qkv["cols"])[r0:r0 + h["rows"]]
        assert idx.max() - idx.min() + 1 == idx.size


def test_workloads_resolve():
    for cid in (1, 2, 3, 4, 5):
        wl = workloads.config(cid, small=True)
        res = resolve_views(wl.nodes, wl.root_numel, wl.scale_layout)
        assert sum(r["rows"] * r["cols"] for r in res if r["is_unit"]) == wl.params
    wl = workloads.ragged_mix()
    resolve_views(wl.nodes, wl.root_numel, wl.scale_layout)
