"""Pins for the oracle's number formats (CPU only).

What fixes these values independently of the oracle's code:
* hand-derived values of the OCP MX E4M3 / E8M0 formats and of bf16 RNE
  (tests/golden/formats.txt, each line with its derivation);
* torch's own float32 -> bfloat16 and float32 -> float8_e4m3fn conversions
  (library routines, round-to-nearest-even), compared exhaustively over
  stratified bit patterns;
* brute force over every admissible scale exponent.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import numerics
from oracle.mxfp8 import quantize_blocks, quantize_blocks_fast

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "formats.txt")


def _golden(kind):
    out = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        if parts[0] == kind:
            out.append(parts[1:])
    assert out, kind
    return out


def _bits32(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


# ----------------------------------------------------------------- golden values
def test_golden_e4m3():
    for val, exp, *_ in _golden("e4m3"):
        code = oracle.e4m3_encode(np.array([float(val)]))[0]
        assert code == int(exp, 16), (val, hex(code), exp)


def test_golden_e8m0():
    for val, exp, *_ in _golden("e8m0"):
        e = oracle.e8m0_exponent(np.float32(float(val)))
        assert e + 127 == int(exp, 16), (val, e, exp)


def test_golden_bf16():
    for val, exp, *_ in _golden("bf16"):
        b = oracle.bf16_rne(np.array([float(val)], dtype=np.float32))
        assert (_bits32(b)[0] >> 16) == int(exp, 16), (val, hex(_bits32(b)[0]), exp)


def test_golden_block():
    (vals, scale, codes), = [g[:3] for g in _golden("block")]
    x = []
    for tok in vals.split(","):
        if "*" in tok:
            v, n = tok.split("*")
            x += [float(v)] * int(n)
        else:
            x.append(float(tok))
    exp_codes = []
    for tok in codes.split("=")[1].split(","):
        if "*" in tok:
            v, n = tok.split("*")
            exp_codes += [int(v, 16)] * int(n)
        else:
            exp_codes.append(int(tok, 16))
    c, s = quantize_blocks(np.array([x], dtype=np.float32))
    assert s[0, 0] == int(scale.split("=")[1], 16)
    assert c[0].tolist() == exp_codes


# ----------------------------------------------------------------- bf16 vs torch
def test_bf16_matches_torch_stratified():
    """Every low-16-bit pattern (which decides the rounding) under both signs
    and the exponents where something changes (zero/subnormal, around 1, the
    top finite binades and Inf/NaN) plus 16 seeded others, with upper-mantissa
    patterns that exercise an even LSB and an odd LSB with the carry into the
    exponent: 2**16 patterns per (sign, exponent, upper) triple."""
    low = np.arange(1 << 16, dtype=np.uint32)
    exps = {0, 1, 2, 3, 125, 126, 127, 128, 129, 252, 253, 254, 255}
    exps |= set(np.random.default_rng(7).integers(4, 252, 16).tolist())
    se = np.array(sorted({(sg << 8) | e for e in exps for sg in (0, 1)}), dtype=np.uint32) << 23
    for hi7 in (0x7E, 0x7F):
        bits = (se[:, None] | (np.uint32(hi7) << 16) | low[None, :]).ravel()
        f = bits.view(np.float32)
        ours = oracle.bf16_rne(f)
        ref = torch.from_numpy(f.copy()).to(torch.bfloat16).float().numpy()
        same = (_bits32(ours) == _bits32(ref)) | (np.isnan(ours) & np.isnan(ref))
        assert same.all(), hex(int(bits[~same][0]))


# ----------------------------------------------------------------- E4M3 vs torch
def _torch_e4m3(y32):
    return torch.from_numpy(np.ascontiguousarray(y32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_matches_torch_every_float_in_key_binades():
    """Every float32 in [1, 2), in the subnormal binades [2**-12, 2**-6), and
    in the top binade [256, 448], both signs."""
    m = np.arange(1 << 23, dtype=np.uint32)
    for e in [0, -7, -8, -9, -10, -11, -12, 8]:
        bits = (np.uint32(e + 127) << 23) | m
        y = bits.view(np.float32)
        if e == 8:
            y = y[y <= 448]
        for sgn in (1, -1):
            yy = (sgn * y).astype(np.float32)
            assert np.array_equal(oracle.e4m3_encode(yy.astype(np.float64)), _torch_e4m3(yy)), (e, sgn)


def test_e4m3_matches_torch_at_every_midpoint():
    t = numerics.e4m3_decode_table()
    mids = (t[1:] + t[:-1]) / 2
    pts = np.concatenate([t, mids]).astype(np.float32)
    near = [pts]
    cur = pts.copy()
    for _ in range(4):
        cur = np.nextafter(cur, np.float32(np.inf))
        near.append(cur.copy())
    cur = pts.copy()
    for _ in range(4):
        cur = np.nextafter(cur, np.float32(-np.inf))
        near.append(cur.copy())
    y = np.concatenate(near)
    y = y[np.abs(y) <= 448]
    y = np.concatenate([y, -y])
    assert np.array_equal(oracle.e4m3_encode(y.astype(np.float64)), _torch_e4m3(y))


def test_e4m3_matches_torch_random():
    r = np.random.default_rng(7)
    y = (r.standard_normal(4_000_000) * np.exp2(r.integers(-14, 9, 4_000_000))).astype(np.float32)
    y = np.clip(y, -448, 448).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(y.astype(np.float64)), _torch_e4m3(y))


def test_e4m3_roundtrip_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    back = oracle.e4m3_encode(vals)
    # +0 / -0 are distinct codes and both round-trip through signed zeros
    assert np.array_equal(back, codes)


# ----------------------------------------------------------------- E8M0
def _least_e_brute(amax):
    for e in range(-127, 128):
        if amax <= math.ldexp(448.0, e):
            return e
    return 127


def test_e8m0_brute_force():
    r = np.random.default_rng(3)
    vals = list((r.standard_normal(3000) * np.exp2(r.integers(-150, 120, 3000))).astype(np.float32))
    for k in range(-140, 120, 3):
        b = np.float32(math.ldexp(448.0, k)) if -149 <= k + 8 < 127 else None
        if b is not None and np.isfinite(b) and b > 0:
            vals += [b, np.nextafter(b, np.float32(np.inf)), np.nextafter(b, np.float32(0))]
    vals += [np.float32(1e-45), np.float32(3.4e38), np.float32(0.0)]
    for v in vals:
        a = abs(float(v))
        exp = -127 if a == 0 else _least_e_brute(a)
        assert oracle.e8m0_exponent(a) == exp, (v, oracle.e8m0_exponent(a), exp)


# ----------------------------------------------------------------- block quantiser
def _blocks_with_specials(rng, n):
    x = (rng.standard_normal((n, 32)) * np.exp2(rng.integers(-30, 30, (n, 1)))).astype(np.float32)
    x[0] = 0
    x[1] = -0.0
    x[2, 5] = np.nan
    x[3, 0] = np.inf
    x[4, 31] = -np.inf
    x[5] = np.float32(1e-42)                     # fp32 subnormals
    x[6, :16] = 0
    x[7] = np.float32(448.0)
    x[8] = np.float32(3e38)
    return x


def test_fast_block_quantiser_equals_plain():
    rng = np.random.default_rng(11)
    x = _blocks_with_specials(rng, 400).reshape(100, 128)
    c1, s1 = quantize_blocks(x)
    c2, s2 = quantize_blocks_fast(x)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_block_invariants_and_half_ulp_bound():
    """Scale is a power of two; amax/scale <= 448 and > 224 unless e = -127
    (together these fix e); dequantisation error <= half an E4M3 ulp."""
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((2000, 64)) * np.exp2(rng.integers(-40, 40, (2000, 1)))).astype(np.float32)
    x[:50] *= np.float32(0.02)
    codes, sb = quantize_blocks_fast(x)
    e = sb.astype(np.int64) - 127
    blocks = x.reshape(2000, 2, 32).astype(np.float64)
    amax = np.abs(blocks).max(axis=2)
    scale = np.ldexp(1.0, e)
    assert np.all(amax / scale <= 448)
    assert np.all((amax / scale > 224) | (e == -127) | (amax == 0))
    y = blocks / scale[:, :, None]
    dq = oracle.e4m3_decode(codes).reshape(2000, 2, 32)
    ay = np.abs(y)
    _, ee = np.frexp(ay)
    ulp = np.where(ay >= 2.0 ** -6, np.ldexp(1.0, ee - 1 - 3), 2.0 ** -9)
    assert np.all(np.abs(y - dq) <= ulp / 2)


def test_special_blocks():
    x = np.zeros((4, 32), dtype=np.float32)
    x[1] = -0.0
    x[2, 3] = np.nan
    x[3, 9] = -np.inf
    c, s = quantize_blocks(x.reshape(1, 128))
    assert s.tolist() == [[0x00, 0x00, 0xFF, 0xFF]]
    c = c.reshape(4, 32)
    assert (c[0] == 0).all() and (c[1] == 0x80).all()
    assert (c[2] == 0x7F).all() and (c[3] == 0x7F).all()
