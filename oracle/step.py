"""One update step over a packed root: Muon units, AdamW units, then G.

[SS-HSDP §3.4, "Update"]: once the microbatches are done every unit runs its
F (for Muon: f0, f1, f2), and G, run on the new main weights, produces the
runtime weights the next iteration uses.  [SS-HSDP §4.1]: compatible operations are batched; batching changes
launch count, not the result, so the oracle simply loops over units.  Muon and
AdamW units own disjoint elements (checked by resolve_views), so their order
does not matter; G reads every updated weight, so it runs last.
"""

from dataclasses import dataclass

import numpy as np

from .views import resolve_views, unit_indices
from .muon import muon_update_unit
from .adamw import adamw_step
from .mxfp8 import cast_root_bf16, requant_root


@dataclass
class OracleHyper:
    # Muon (f0..f2)
    lr: float = 0.02
    momentum: float = 0.95
    weight_decay: float = 0.0
    nesterov: bool = False
    ns_steps: int = 5
    a: float = 3.4445
    b: float = -4.7750
    c: float = 2.0315
    ns_eps: float = 1e-7
    scale_mode: int = 0
    # AdamW
    adam_lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.95
    adam_eps: float = 1e-8
    adam_wd: float = 0.1


def update_step(nodes, root_numel, w, g, m, v, codes, scales, step, hp=None,
                layout="rowmajor", do_muon=True, do_adamw=True, do_requant=True,
                keep_v=False, bf16_root=None):
    """Apply one step in place to float32 roots w, m, v, uint8 roots codes,
    scales and (when given) the uint16 root of bf16-cast regions.  Returns a
    dict {unit index: float64 NS direction} if keep_v."""
    hp = hp or OracleHyper()
    res = resolve_views(nodes, root_numel, layout)
    dirs = {}
    for i, r in enumerate(res):
        if not r["is_unit"]:
            continue
        idx = unit_indices(r)
        if r["optimizer"] == "muon" and do_muon:
            w_new, m_new, vdir = muon_update_unit(w[idx], g[idx], m[idx], hp)
            w[idx] = w_new
            m[idx] = m_new
            if keep_v:
                dirs[i] = vdir
        elif r["optimizer"] == "adamw" and do_adamw:
            w_new, m_new, v_new = adamw_step(w[idx], g[idx], m[idx], v[idx], step,
                                             hp.adam_lr, hp.beta1, hp.beta2,
                                             hp.adam_eps, hp.adam_wd)
            w[idx], m[idx], v[idx] = w_new, m_new, v_new
    if do_requant:
        requant_root(w, res, layout, codes, scales)
        if bf16_root is not None:
            cast_root_bf16(w, res, bf16_root)
    return dirs
