"""G: MXFP8 requantisation of main weights, plus the scale relayout of Tw.

[SS-HSDP §2.1]: G casts or quantises the main weight into the low-precision
weight w and optional scale metadata s.  [SS-HSDP §3.1, EG1]: G produces FP8
weights with UE8M0 scales; Tw packs the per-head weights into the runtime
weight -- a pure view of the same root, no copy [SS-HSDP §3.2, §4.2] -- and
relays the scales out into the layout the GEMM kernel needs.  [OCP-MX]: one
E8M0 scale shared by a block of 32 elements.

Readings taken (the pages are silent or conflicting on these):
* block shape 1 x 32 along K (the contiguous dimension);
* scale exponent: the least e with amax <= 448 * 2**e (numerics.e8m0_exponent);
* element rounding: nearest E4M3FN value, ties to even, sign kept;
* all-zero block -> scale byte 0x00 (e = -127);
* a block holding NaN or +-Inf -> scale byte 0xFF and every code 0x7F;
* scale byte = e + 127.

Codes live at the SAME element offsets as the fp32 main weight (a uint8 root
of root_numel bytes), so a head's codes are a sub-range of the packed
projection's codes.  Scale layouts (per quantised region at absolute element
offset o, rows N, cols K, KB = K/32 blocks per row):
* 'rowmajor': block (n, kb) -> o/32 + n*KB + kb (= its first element / 32);
* 'tile32x4': block (n, kb) -> o/32 + ((n//32)*(KB//4) + kb//4)*128
                                    + (n%32)*4 + kb%4,
  one 128-byte chunk per 32-row x 128-column tile, one 4-byte word per row.

32 x 32 blocks ('block32x32'; [SS-HSDP §3.1 EG1] and [veScale §6] describe G
with 32 x 32 blocks in a k-major layout): one scale per 32-row x 32-column
block of a region (rows and cols multiples of 32, first element a multiple of
1024), chosen by the same least-e rule over the block's 1024 elements; the
block (bn, bk) -> o/1024 + bn*(K/32) + bk.  The same codes serve the
transposed operand: the blocks of X^T are the transposes of X's.
"""

import numpy as np

from .numerics import bf16_rne, e4m3_encode, e8m0_exponent
from .views import unit_indices


def quantize_blocks(x):
    """Quantise a float32 array of shape (N, K), K % 32 == 0, block 1x32 along K.

    Returns (codes uint8 (N, K), scale_bytes uint8 (N, K/32)).
    """
    x = np.asarray(x, dtype=np.float32)
    N, K = x.shape
    assert K % 32 == 0
    blocks = x.reshape(N, K // 32, 32).astype(np.float64)
    codes = np.empty((N, K // 32, 32), dtype=np.uint8)
    sbytes = np.empty((N, K // 32), dtype=np.uint8)
    finite = np.all(np.isfinite(blocks), axis=2)
    amax = np.max(np.abs(np.where(np.isfinite(blocks), blocks, 0.0)), axis=2)
    for n in range(N):
        for kb in range(K // 32):
            if not finite[n, kb]:
                sbytes[n, kb] = 0xFF
                codes[n, kb, :] = 0x7F
                continue
            e = e8m0_exponent(amax[n, kb])
            sbytes[n, kb] = e + 127
            codes[n, kb, :] = e4m3_encode(np.ldexp(blocks[n, kb], -e))   # exact scaling
    return codes.reshape(N, K), sbytes


def quantize_blocks_fast(x):
    """Same result as quantize_blocks, with the per-block exponent search
    vectorised (used for big regions; pinned equal to quantize_blocks)."""
    x = np.asarray(x, dtype=np.float32)
    N, K = x.shape
    blocks = x.reshape(N, K // 32, 32).astype(np.float64)
    finite = np.all(np.isfinite(blocks), axis=2)
    amax = np.max(np.abs(np.where(np.isfinite(blocks), blocks, 0.0)), axis=2)
    # least e with amax <= 448*2**e: start below, step up while the bound fails
    _, e2 = np.frexp(amax)
    e = e2 - 11
    for _ in range(4):
        e = np.where(amax > np.ldexp(448.0, e), e + 1, e)
    assert np.all(amax <= np.ldexp(448.0, e))
    e = np.where(amax == 0, -127, np.clip(e, -127, 127))
    y = np.ldexp(np.where(np.isfinite(blocks), blocks, 0.0), -e[:, :, None])
    codes = e4m3_encode(y)
    codes[~finite] = 0x7F
    sbytes = np.where(finite, e + 127, 0xFF).astype(np.uint8)
    return codes.reshape(N, K), sbytes


def quantize_blocks_32x32(x):
    """Quantise a float32 array of shape (N, K), N and K multiples of 32, with
    one scale per 32 x 32 block: amax over the block's 1024 elements, the
    least-e scale, then every element's nearest E4M3FN code of x * 2**-e.

    Returns (codes uint8 (N, K), scale_bytes uint8 (N/32, K/32)).
    """
    x = np.asarray(x, dtype=np.float32)
    N, K = x.shape
    assert N % 32 == 0 and K % 32 == 0
    codes = np.empty((N, K), dtype=np.uint8)
    sbytes = np.empty((N // 32, K // 32), dtype=np.uint8)
    for bn in range(N // 32):
        for bk in range(K // 32):
            blk = x[32 * bn:32 * bn + 32, 32 * bk:32 * bk + 32].astype(np.float64)
            if not np.all(np.isfinite(blk)):
                sbytes[bn, bk] = 0xFF
                codes[32 * bn:32 * bn + 32, 32 * bk:32 * bk + 32] = 0x7F
                continue
            e = e8m0_exponent(np.max(np.abs(blk)))
            sbytes[bn, bk] = e + 127
            codes[32 * bn:32 * bn + 32, 32 * bk:32 * bk + 32] = e4m3_encode(np.ldexp(blk, -e))
    return codes, sbytes


def scale_index(layout, o, N, K):
    """Index into the scale root of each scale of a region: shape (N, K/32)
    for the 1 x 32 layouts, (N/32, K/32) for 'block32x32'."""
    if layout == "block32x32":
        bn = np.arange(N // 32, dtype=np.int64)[:, None]
        bk = np.arange(K // 32, dtype=np.int64)[None, :]
        return o // 1024 + bn * (K // 32) + bk
    KB = K // 32
    n = np.arange(N, dtype=np.int64)[:, None]
    kb = np.arange(KB, dtype=np.int64)[None, :]
    base = o // 32
    if layout == "rowmajor":
        return base + n * KB + kb
    if layout == "tile32x4":
        return base + ((n // 32) * (KB // 4) + kb // 4) * 128 + (n % 32) * 4 + kb % 4
    raise ValueError(layout)


def requant_root(w_root, resolved, layout, codes_root, scales_root, fast=True):
    """G + Tw over every quantised region of a resolved view table.

    Writes in place into ``codes_root`` (uint8, one per element) and
    ``scales_root`` (uint8, one per 32 elements; one per 1024 for
    'block32x32'); bytes outside quantised
    regions are left untouched.
    """
    q = quantize_blocks_fast if fast else quantize_blocks
    if layout == "block32x32":
        q = quantize_blocks_32x32
    for r in resolved:
        if not r["quantize"]:
            continue
        idx = unit_indices(r)
        c, s = q(w_root[idx])
        codes_root[idx] = c
        scales_root[scale_index(layout, r["abs"], r["rows"], r["cols"])] = s
    return codes_root, scales_root


def cast_root_bf16(w_root, resolved, out_root):
    """G as a bfloat16 cast [SS-HSDP §2.1] over every 'bf16' region of a
    resolved view table: out_root (uint16, one per element of the fp32 root)
    receives the bit pattern of bf16_rne(w) at the elements' own offsets;
    other elements are left untouched."""
    for r in resolved:
        if not r.get("cast"):
            continue
        idx = unit_indices(r)
        b = bf16_rne(np.asarray(w_root[idx], dtype=np.float32))
        out_root[idx] = (b.view(np.uint32) >> 16).astype(np.uint16)
    return out_root
