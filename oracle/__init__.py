"""CPU oracle for one GPU's share of the SS-HSDP update phase.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It is a plain, slow,
obviously-correct statement of what the update phase computes, written in
NumPy with float64 arithmetic, and it shares no code, tables or constants with
the HIP implementation in ``mxfp8_weight_repack_amd``.

Sources (cited by title and section throughout):

* [SS-HSDP] "SS-HSDP: Efficient and Flexible Sharded Data Parallelism via
  Runtime-Update Decoupling" (arXiv:2611.16467v1): the F/G model (§2.1),
  update/runtime parameters and the EG1 example (§3.1), data trees (§3.2),
  execution flow (§3.4), batched update (§4.1), zero-copy weights (§4.2),
  Appendix A and its Table 4 (planning rules).
* [veScale] the veScale-FSDP summary page: block-aligned ragged shards and the
  rule of padding between tensors to block boundaries (§4, §5).
* [OCP-MX] the OCP Microscaling Formats specification v1.0, cited by [SS-HSDP]
  as its MXFP reference: the E4M3 element format and the E8M0 shared scale.

Where the pages leave a step open the oracle takes one plain reading, named in
each function's docstring.  Parity status of each part:

* views, momentum, bf16 rounding, Newton-Schulz (the iteration as stated),
  AdamW, MXFP8 block quantisation, both scale layouts: pinned by the
  ``-m "not gpu"`` tests (closed forms, library routines, brute force).
* The Muon conventions (heavy-ball momentum form, NS epsilon, update scale,
  zero weight decay): parity with the pages' own Muon is UNPINNED -- the pages
  print no Muon update values, so only the convention chosen here is pinned.
"""

from .views import ViewError, resolve_views, unit_indices
from .numerics import bf16_rne, e4m3_decode_table, e4m3_encode, e4m3_decode, e8m0_exponent
from .mxfp8 import quantize_blocks, quantize_blocks_32x32, scale_index, requant_root, cast_root_bf16
from .muon import momentum_step, newton_schulz, muon_scale, muon_update_unit
from .adamw import adamw_step
from .step import update_step, OracleHyper

__all__ = [
    "ViewError", "resolve_views", "unit_indices",
    "bf16_rne", "e4m3_decode_table", "e4m3_encode", "e4m3_decode", "e8m0_exponent",
    "quantize_blocks", "quantize_blocks_32x32", "scale_index", "requant_root", "cast_root_bf16",
    "momentum_step", "newton_schulz", "muon_scale", "muon_update_unit",
    "adamw_step", "update_step", "OracleHyper",
]
