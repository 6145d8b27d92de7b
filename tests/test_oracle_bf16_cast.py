"""G as a bfloat16 cast for runtime weights that are not MX-quantised
([SS-HSDP §2.1]: G casts or quantises the main weight), oracle side (CPU).

Pinned by torch's float32 -> bfloat16 conversion (a library routine) of the
same region, and by the planning rules: a bf16 region may not overlap another G
region (the method's rule); the library also wants it contiguous with its first
element and cols multiples of 8 (its 16-byte stores; tests/boundary_rules.py),
which the oracle does not require.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.views import ViewError, resolve_views
from boundary_rules import expected_code

import mxfp8_weight_repack_amd as sh


def bf16_variant(wl):
    """The small dense block with the O projection (a Muon unit) and both norms
    (AdamW units) cast to bf16 instead of MXFP8."""
    nodes = [dict(n) for n in wl.nodes]
    for i, n in enumerate(nodes):
        if n["parent"] == -1 and n["is_unit"] and n["rows"] == n["cols"]:
            n["quantize"] = "bf16"               # O projection
        if n["is_unit"] and n["optimizer"] == "adamw":
            n["quantize"] = "bf16"               # norms
    return nodes


def test_cast_equals_torch_bf16_and_leaves_the_rest():
    wl = workloads.config(2, small=True)
    nodes = bf16_variant(wl)
    w, _ = wl.arrays()
    w = w.copy()
    w[:8] = [np.nan, np.inf, -np.inf, -0.0, 1e-41, 3.4e38, 1.00390625, -1.01171875]
    res = resolve_views(nodes, wl.root_numel)
    out = np.full(wl.root_numel, 0xBEEF, np.uint16)
    oracle.cast_root_bf16(w, res, out)
    mask = np.zeros(wl.root_numel, bool)
    for r in res:
        if r["cast"]:
            mask[r["abs"]:r["abs"] + r["rows"] * r["cols"]] = True
    assert mask.sum() == 256 * 256 + 2 * 256
    ref = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out[mask], ref[mask])
    assert np.all(out[~mask] == 0xBEEF)


def test_bf16_planning_rules_agree():
    base = dict(parent=-1, offset=0, rows=4, cols=64, row_stride=64, is_unit=False, optimizer=None, quantize="bf16")
    # (nodes, oracle's answer, library's answer)
    cases = [
        ([base], None, None),
        ([dict(base, cols=60, row_stride=60)], None, "SCHEMA"),      # cols not a multiple of 8
        ([dict(base, offset=4)], None, "SCHEMA"),                   # start not 8-aligned
        ([dict(base, row_stride=72)], None, "SCHEMA"),              # not contiguous
        ([base, dict(base, offset=128, quantize=True, rows=1)], "OVERLAP", "OVERLAP"),   # overlaps an MXFP8 region
        ([base, dict(base, offset=256, quantize=True, rows=1)], None, None),
        ([dict(base, quantize="fp4")], "SCHEMA", "SCHEMA"),
    ]
    for nodes, exp_o, exp_c in cases:
        try:
            resolve_views(nodes, 1024)
            got_o = None
        except ViewError as e:
            got_o = e.code
        try:
            sh.Plan(nodes, 1024, host_only=True)
            got_c = None
        except sh.SshdpError as e:
            got_c = e.name
        assert got_o == exp_o and got_c == exp_c == expected_code(nodes, 1024), (nodes, got_o, got_c)
    st = sh.Plan(bf16_variant(workloads.config(2, small=True)), workloads.config(2, small=True).root_numel,
                 host_only=True).stats()
    assert st["cast_elems"] == 256 * 256 + 512 and st["n_cast_regions"] == 3
