"""The oracle's whole update step on a mixed tree (CPU only): it touches only
unit elements (padding and non-unit gaps keep their bytes), writes codes and
scales only inside quantised regions, and equals the per-unit functions."""

import numpy as np

import oracle
from oracle.views import resolve_views, unit_indices
import workloads


def test_update_step_touches_only_units_and_quantised_regions():
    wl = workloads.ragged_mix()
    w0, g = wl.arrays()
    w = w0.copy()
    m = np.zeros_like(w)
    v = np.zeros_like(w)
    codes = np.full(wl.root_numel, 0xAB, np.uint8)
    scales = np.full(wl.root_numel // 32 + 1, 0xCD, np.uint8)
    oracle.update_step(wl.nodes, wl.root_numel, w, g, m, v, codes, scales, step=1)
    res = resolve_views(wl.nodes, wl.root_numel)
    unit_mask = np.zeros(wl.root_numel, bool)
    q_mask = np.zeros(wl.root_numel, bool)
    for r in res:
        if r["is_unit"]:
            unit_mask[unit_indices(r).ravel()] = True
        if r["quantize"]:
            q_mask[unit_indices(r).ravel()] = True
    assert np.array_equal(w[~unit_mask], w0[~unit_mask])
    assert np.all(m[~unit_mask] == 0) and np.all(v[~unit_mask] == 0)
    assert np.all(codes[~q_mask] == 0xAB)
    smask = np.zeros(scales.size, bool)
    smask[np.nonzero(q_mask)[0] // 32] = True
    assert np.all(scales[~smask] == 0xCD)
    # zero-gradient Muon unit is bit-identical; AdamW units changed
    z = res[wl.zero_grad_units[0]]
    assert np.array_equal(w[unit_indices(z)], w0[unit_indices(z)])
    # per-unit functions give the same values
    hp = oracle.OracleHyper()
    for r in res:
        if not r["is_unit"]:
            continue
        idx = unit_indices(r)
        if r["optimizer"] == "muon":
            wn, mn, _ = oracle.muon_update_unit(w0[idx], g[idx], np.zeros_like(w0[idx]), hp)
        else:
            z0 = np.zeros_like(w0[idx])
            wn, mn, _ = oracle.adamw_step(w0[idx], g[idx], z0, z0, 1, 1e-3, 0.9, 0.95, 1e-8, 0.1)
        assert np.array_equal(w[idx], wn) and np.array_equal(m[idx], mn)
