"""The reduce-scatter tail of [SS-HSDP §4.3 "Reduce-Scatter", Figure 5(e)]
(oracle; test infrastructure only).

Within a node, the slices of one output partition arrive from several ranks;
a local reducer sums them in FP32.  The partial stays FP32, or -- when the
gradients are BF16 -- is stored as BF16 with stochastic rounding (SR).  The
final FP32 reduction adds the arriving partials straight into the persistent
accumulation buffer (G'z2): on the first microbatch it initialises the buffer,
afterwards it accumulates, with no separate result buffer or addition pass.

Readings taken where the pages are silent:
* summation order: inputs in the order given, left to right, each addition
  rounded to FP32 ("sum them in FP32");
* the first microbatch initialises the buffer with the sum of the partials
  (acc = in_0, then + in_1 ...); later microbatches compute ((g + in_0) + in_1) ...;
* SR of a finite FP32 value x to BF16: with lo the BF16 value next to x toward
  zero, hi = lo + one BF16 ulp away from zero and k = (|x| - |lo|) / ulp * 2^16
  (an integer in [0, 2^16)), the result is hi when r >= 2^16 - k for a random
  16-bit integer r, else lo -- so P(hi) = k / 2^16 and E[SR(x)] = x; values
  representable in BF16 are kept; NaN stays NaN; +-Inf stay;
* random bits: Philox4x64-10 (Salmon et al., "Parallel random numbers: as easy
  as 1, 2, 3", SC'11), key (seed, 0); element g (its index in the whole
  tensor) takes block b = g // 16 with counter (b + 1, ctr, 0, 0), word
  (g // 4) % 4 and bits 16*(g % 4) .. +15 of it.  numpy's Philox bit generator
  is this generator (it advances the counter before each block, hence b + 1).
"""

import numpy as np


def philox_bits16(seed, ctr, g0, n):
    """16-bit random integers for elements g0 .. g0+n-1."""
    b0, b1 = g0 // 16, (g0 + n + 15) // 16
    bg = np.random.Philox(key=int(seed), counter=(int(ctr) << 64) + b0)
    words = bg.random_raw(4 * (b1 - b0)).astype(np.uint64)   # 4 words per block
    parts = (words[:, None] >> (np.arange(4, dtype=np.uint64) * np.uint64(16))[None, :]) & np.uint64(0xFFFF)
    return parts.reshape(-1).astype(np.int64)[g0 - 16 * b0:g0 - 16 * b0 + n]


def _bf16_neighbours(ax):
    """For finite |x| (float64 of float32 values): |lo| (BF16 toward zero) and the BF16 ulp there."""
    _, e = np.frexp(ax)                                      # ax = m * 2**e, m in [0.5, 1)
    ulp = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)        # 2**(E-7), subnormal quantum 2**-133
    lo = np.floor(ax / ulp) * ulp
    return lo, ulp


def sr_bf16(x, r):
    """Stochastic rounding of float32 values to BF16 with 16-bit randoms r;
    returns the BF16 bit patterns (uint16)."""
    x = np.asarray(x, dtype=np.float32)
    r = np.asarray(r, dtype=np.int64)
    ax = np.abs(x.astype(np.float64))
    fin = np.isfinite(ax)
    lo, ulp = _bf16_neighbours(np.where(fin, ax, 1.0))
    k = np.where(fin, np.round((ax - lo) / ulp * 65536.0), 0).astype(np.int64)
    up = fin & (k > 0) & (r >= 65536 - k)
    mag = np.where(up, lo + ulp, lo)
    mag = np.where(fin, mag, ax)                              # Inf stays (NaN handled below)
    # mag is a BF16 value (or 2**128 = Inf after rounding up from the top binade)
    with np.errstate(over="ignore"):
        val = np.where(np.signbit(x), -mag, mag).astype(np.float32)
    bits = (val.view(np.uint32) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    bits[nan] = ((x[nan].view(np.uint32) >> 16) | 0x40).astype(np.uint16)
    return bits


def _as_f32(a, dtype):
    a = np.asarray(a)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def fp32_sum(inputs, dtype, start=None):
    """((start + in_0) + in_1) + ... in float32 (start None: in_0 + in_1 + ...)."""
    acc = None if start is None else np.asarray(start, np.float32).copy()
    for a in inputs:
        v = _as_f32(a, dtype)
        acc = v.copy() if acc is None else (acc + v).astype(np.float32)
    return acc


def rs_reduce(inputs, dtype, out_mode, seed=0, ctr=0, g0=0):
    """Local reducer: the FP32 sum of the slices; returned as float32
    (out_mode 'fp32') or as BF16 bit patterns with SR ('bf16_sr')."""
    s = fp32_sum(inputs, dtype)
    if out_mode == "fp32":
        return s
    return sr_bf16(s, philox_bits16(seed, ctr, g0, s.size))


def rs_accumulate(inputs, dtype, g, first):
    """Final reduction into the persistent FP32 buffer g (returned)."""
    return fp32_sum(inputs, dtype, start=None if first else g)
