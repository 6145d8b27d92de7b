"""Number formats used by the update phase (oracle; test infrastructure only).

* bf16: the update temporary ``u`` is BF16 [SS-HSDP §3.1, EG1: the first Muon
  stage writes a BF16 intermediate].  Rounding is round-to-nearest-even
  (reading: the pages name no rounding mode; RNE is IEEE's default).
* E4M3 (FP8) elements and the E8M0 shared scale of an MX block [OCP-MX, cited
  by SS-HSDP §1 and §2.3 as the MXFP format; EG1 names the scale "UE8M0"].
  E4M3 here is the OCP "FN" variant: exponent bias 7, three mantissa bits,
  subnormals m * 2**-9, largest finite 448, no infinities, S.1111.111 = NaN.

Everything is computed on VALUES in float64 (frexp, rint, a sorted table of
decoded codes), deliberately not by manipulating float32 bit fields.
"""

import math
import numpy as np


# --------------------------------------------------------------------------- bf16
def bf16_rne(x):
    """Round float32 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps float32's exponent range and 8 significant bits.  For a
    finite x with 2**E <= |x| < 2**(E+1) the spacing of bf16 values is
    2**(E-7) (for E >= -126; below that the spacing is the subnormal quantum
    2**-133).  Rounding is x/spacing -> nearest integer, ties to even
    (numpy.rint), times spacing; a result of 2**128 or more is infinite.
    Returns float32 holding the bf16 values.  NaN stays NaN, +-Inf stays.
    """
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(invalid="ignore"):
        xd = x.astype(np.float64)
    out = np.empty_like(xd)
    fin = np.isfinite(xd)
    out[~fin] = xd[~fin]
    v = xd[fin]
    a = np.abs(v)
    _, e = np.frexp(a)                     # a = f * 2**e, f in [0.5, 1)  ->  E = e - 1
    E = np.maximum(e - 1, -126)
    spacing = np.ldexp(1.0, E - 7)
    q = np.rint(v / spacing) * spacing     # exact: v/spacing is an exact float64
    q[np.abs(q) >= 2.0 ** 128] = np.copysign(np.inf, v[np.abs(q) >= 2.0 ** 128])
    q[(q == 0)] = np.copysign(0.0, v[(q == 0)])
    out[fin] = q
    return out.astype(np.float32)


# --------------------------------------------------------------------------- E4M3
def e4m3_decode_table():
    """Values of the 127 non-negative finite E4M3FN codes 0x00..0x7E, float64.

    Code bits 0EEEEMMM: E == 0 -> M * 2**-9 (subnormal), else
    (1 + M/8) * 2**(E - 7).  0x7F is NaN and is not in the table.
    """
    vals = []
    for code in range(0x7F):
        E, M = code >> 3, code & 7
        vals.append(M * 2.0 ** -9 if E == 0 else (1 + M / 8.0) * 2.0 ** (E - 7))
    t = np.array(vals, dtype=np.float64)
    assert np.all(np.diff(t) > 0)
    return t


_E4M3 = e4m3_decode_table()


def e4m3_decode(codes):
    """Decode uint8 E4M3FN codes to float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    out = np.where(mag == 0x7F, np.nan, _E4M3[np.minimum(mag, 0x7E)])
    return np.where(c & 0x80, -out, out)


def e4m3_encode(y):
    """Nearest E4M3FN code to each finite float64 ``y`` with |y| <= 448.

    Nearest by value over the full code table (binary search for the
    neighbours, then the closer one); an exact tie goes to the code whose
    mantissa LSB is 0, i.e. the even code.  The sign bit is the sign of y
    (so -0 and negatives that round to zero encode as 0x80).
    """
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.abs(y) <= 448.0):
        raise ValueError("e4m3_encode: |y| > 448 or non-finite (no saturation in this path)")
    a = np.abs(y)
    hi = np.searchsorted(_E4M3, a, side="left")            # first table value >= a
    hi = np.minimum(hi, len(_E4M3) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3[lo]
    dhi = _E4M3[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(a == _E4M3[hi], hi, mag)                 # exact hit
    sign = np.signbit(y).astype(np.int64) << 7
    return (mag | sign).astype(np.uint8)


# --------------------------------------------------------------------------- E8M0
def e8m0_exponent(amax):
    """Shared-scale exponent of one MX block from its largest magnitude.

    Reading (the pages give no scale rule): e is the LEAST integer with
    amax <= 448 * 2**e, so every scaled element fits E4M3's range without
    saturation and the scale is as fine as possible; clamped to E8M0's range
    [-127, 127].  amax == 0 gives -127.  Found by direct search on exact
    float64 comparisons.
    """
    amax = float(amax)
    if amax == 0.0:
        return -127
    _, e2 = math.frexp(amax)              # amax < 2**e2
    e = e2 - 11                           # 448 * 2**(e2-11) < 2**e2 / 4 < amax: too small
    while amax > math.ldexp(448.0, e):
        e += 1
    return max(-127, min(127, e))
