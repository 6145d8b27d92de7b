"""Pins for the oracle's 32 x 32-block MXFP8 quantiser (CPU only).

[SS-HSDP §3.1 EG1] and [veScale §6] describe G with 32 x 32 blocks in a
k-major layout: one E8M0 scale per 32-row x 32-column block.  Pinned by:
* a block worked by hand (tests/golden/formats.txt, line `block32`);
* reduction to the 1 x 32 quantiser (pinned on its own): the least-e scale
  is monotone in amax, so a 32 x 32 block's scale byte is the largest of its
  32 rows' 1 x 32 scale bytes -- including 0xFF for a non-finite block;
* codes against torch's float32 -> float8_e4m3fn conversion of the exactly
  scaled values (a library routine);
* the transpose property (the same codes serve X^T) and the half-ulp error
  bound; the block scale index is a bijection and per-head views are
  sub-ranges of the packed projection's.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.mxfp8 import quantize_blocks, quantize_blocks_32x32, scale_index
from oracle.views import ViewError, resolve_views

from test_oracle_formats import _golden


def _parse_grid(spec, conv):
    base, *over = spec.split(";")
    g = np.full((32, 32), conv(base))
    for o in over:
        pos, v = o.split("=")
        r, c = (int(t) for t in pos.split(","))
        g[r, c] = conv(v)
    return g


def test_golden_block32():
    (vals, scale, codes), = [g[:3] for g in _golden("block32")]
    x = _parse_grid(vals, float).astype(np.float32)
    exp = _parse_grid(codes.split("=", 1)[1], lambda t: int(t, 16)).astype(np.uint8)
    c, s = quantize_blocks_32x32(x)
    assert s.shape == (1, 1) and s[0, 0] == int(scale.split("=")[1], 16)
    assert np.array_equal(c, exp)


def _region(rng, n, k):
    x = rng.standard_normal((n, k))
    # per-block magnitudes spread over many binades
    mag = np.exp2(rng.integers(-30, 30, (n // 32, k // 32)))
    x = (x * np.kron(mag, np.ones((32, 32)))).astype(np.float32)
    x[:32, :32] = 0                              # zero block
    x[:32, 32:64] = -0.0                         # negative zeros
    x[40, 70] = np.nan                           # NaN block
    x[70, 100] = -np.inf                         # Inf block
    x[96:128, :32] = np.float32(1e-42)           # fp32 subnormals
    x[96:128, 32:64] = np.float32(448.0)
    x[97, 40] = np.float32(3e38)                 # near the fp32 top
    return x


def test_block32_scale_is_max_of_row_scales():
    rng = np.random.default_rng(31)
    x = _region(rng, 128, 192)
    _, s32 = quantize_blocks_32x32(x)
    _, s1 = quantize_blocks(x)                   # (128, 6), one per row and 32 columns
    exp = s1.reshape(4, 32, 6).max(axis=1)
    assert np.array_equal(s32, exp)
    assert s32[1, 2] == 0xFF and s32[2, 3] == 0xFF and s32[0, 0] == 0 and s32[0, 1] == 0


def test_block32_codes_equal_torch_of_exactly_scaled_values():
    rng = np.random.default_rng(32)
    x = _region(rng, 128, 192)
    c, s = quantize_blocks_32x32(x)
    e = np.kron(s.astype(np.int64) - 127, np.ones((32, 32), np.int64))
    finite = np.kron(s != 0xFF, np.ones((32, 32), bool))
    y = np.ldexp(np.where(finite, x, 0).astype(np.float64), -e).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(c[finite], ref[finite])
    assert np.all(c[~finite] == 0x7F)


def test_block32_transpose_serves_the_transposed_operand():
    rng = np.random.default_rng(33)
    x = _region(rng, 128, 160)
    c, s = quantize_blocks_32x32(x)
    ct, st = quantize_blocks_32x32(np.ascontiguousarray(x.T))
    assert np.array_equal(ct, c.T) and np.array_equal(st, s.T)


def test_block32_invariants_and_half_ulp_bound():
    rng = np.random.default_rng(34)
    x = (rng.standard_normal((256, 256)) * np.kron(np.exp2(rng.integers(-40, 40, (8, 8))),
                                                   np.ones((32, 32)))).astype(np.float32)
    c, s = quantize_blocks_32x32(x)
    e = s.astype(np.int64) - 127
    blocks = x.reshape(8, 32, 8, 32).transpose(0, 2, 1, 3).astype(np.float64)
    amax = np.abs(blocks).max(axis=(2, 3))
    scale = np.ldexp(1.0, e)
    assert np.all(amax / scale <= 448) and np.all((amax / scale > 224) | (e == -127))
    y = x.astype(np.float64) / np.kron(scale, np.ones((32, 32)))
    dq = oracle.e4m3_decode(c)
    ay = np.abs(y)
    _, ee = np.frexp(ay)
    ulp = np.where(ay >= 2.0 ** -6, np.ldexp(1.0, ee - 1 - 3), 2.0 ** -9)
    assert np.all(np.abs(y - dq) <= ulp / 2)


def test_block32_scale_index_bijection_and_head_subranges():
    o, N, K = 4096 * 3, 256, 384
    idx = scale_index("block32x32", o, N, K)
    assert idx.shape == (N // 32, K // 32)
    assert np.array_equal(np.sort(idx.ravel()), np.arange(o // 1024, o // 1024 + N * K // 1024))
    # a head of 64 rows at row 128 of the projection: its own region starts at o + 128*K
    head = scale_index("block32x32", o + 128 * K, 64, K)
    assert np.array_equal(head, idx[4:6])


def test_block32_planning_rules():
    base = dict(parent=-1, offset=0, rows=64, cols=64, row_stride=64, is_unit=False, optimizer=None, quantize=True)
    resolve_views([base], 8192, "block32x32")
    with pytest.raises(ViewError) as e:
        resolve_views([dict(base, rows=48)], 8192, "block32x32")
    assert e.value.code == "SCHEMA"
    with pytest.raises(ViewError) as e:
        resolve_views([dict(base, offset=512)], 8192, "block32x32")
    assert e.value.code == "SCHEMA"


def test_requant_root_block32_equals_per_region():
    rng = np.random.default_rng(35)
    root = rng.standard_normal(3 * 4096).astype(np.float32)
    nodes = [dict(parent=-1, offset=0, rows=64, cols=64, row_stride=64, is_unit=False, optimizer=None, quantize=True),
             dict(parent=-1, offset=8192, rows=32, cols=128, row_stride=128, is_unit=False, optimizer=None,
                  quantize=True)]
    res = resolve_views(nodes, root.size, "block32x32")
    codes = np.full(root.size, 0xAB, np.uint8)
    scales = np.full(root.size // 1024, 0xCD, np.uint8)
    oracle.requant_root(root, res, "block32x32", codes, scales)
    c0, s0 = quantize_blocks_32x32(root[:4096].reshape(64, 64))
    c1, s1 = quantize_blocks_32x32(root[8192:].reshape(32, 128))
    assert np.array_equal(codes[:4096], c0.ravel()) and np.array_equal(codes[8192:], c1.ravel())
    assert np.all(codes[4096:8192] == 0xAB)
    assert scales.tolist() == s0.ravel().tolist() + [0xCD] * 4 + s1.ravel().tolist()
