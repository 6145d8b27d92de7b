"""One MI355X's share of the SS-HSDP update phase: Muon (momentum, batched bf16
MFMA Newton-Schulz, weight update), AdamW and in-place MXFP8 requantisation
of packed fp32 roots, as hand-written HIP for gfx950 behind the C ABI in
include/sshdp.h.  This package is the thin ctypes binding of that library.
"""

from ._lib import (  # noqa: F401
    LIB_PATH, SshdpError, Plan, buffers, muon_hp, adamw_hp, update_muon, update_adamw, requant_mxfp8,
    cast_bf16, rs_reduce, rs_accumulate,
    update_step, update_step_noalloc, gemm_bf16_nt, lib, PROF_CLASSES, ERROR_NAMES, NOALLOC_SCRATCH_BYTES,
)
