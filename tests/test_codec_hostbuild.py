"""The GPU kernels' MXFP8/bf16 bit logic (csrc/mx_codec.h), compiled for the
host with gcc and checked on the CPU against torch's own float32 -> bfloat16
and float32 -> float8_e4m3fn conversions (library routines) and against
brute force over the scale exponent.  This is host logic of the HIP path,
tested before any GPU run; the oracle is not involved."""

import ctypes
import math
import os
import subprocess

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp8_weight_repack_amd", "csrc")

SHIM = r"""
#include <stdint.h>
#include "mx_codec.h"
void blocks(const uint32_t *x, int64_t nblk, uint8_t *codes, uint8_t *scales) {
  for (int64_t b = 0; b < nblk; ++b) {
    uint32_t a = 0;
    for (int i = 0; i < 32; ++i) { uint32_t v = x[b * 32 + i] & 0x7fffffffu; if (v > a) a = v; }
    uint32_t s = mx_scale_byte(a);
    scales[b] = (uint8_t)s;
    for (int i = 0; i < 32; ++i)
      codes[b * 32 + i] = (uint8_t)(s == 0xFFu ? 0x7Fu : mx_e4m3_code(x[b * 32 + i], (int)s - 127));
  }
}
void codes_at(const uint32_t *x, int64_t n, int e, uint8_t *codes) {
  for (int64_t i = 0; i < n; ++i) codes[i] = (uint8_t)mx_e4m3_code(x[i], e);
}
void bf16(const uint32_t *x, int64_t n, uint16_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint16_t)mx_bf16_bits(x[i]);
}
"""


@pytest.fixture(scope="module")
def codec(tmp_path_factory):
    d = tmp_path_factory.mktemp("codec")
    src = d / "shim.c"
    src.write_text(SHIM)
    so = d / "codec.so"
    subprocess.run(["gcc", "-O2", "-shared", "-fPIC", "-I", CSRC, str(src), "-o", str(so)], check=True)
    L = ctypes.CDLL(str(so))
    P = ctypes.c_void_p
    L.blocks.argtypes = [P, ctypes.c_int64, P, P]
    L.codes_at.argtypes = [P, ctypes.c_int64, ctypes.c_int, P]
    L.bf16.argtypes = [P, ctypes.c_int64, P]
    return L


def _torch_e4m3(y32):
    return torch.from_numpy(np.ascontiguousarray(y32, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_e4m3_code_equals_torch_every_float_in_range(codec):
    """With e = 0 the kernel code of x must equal torch's E4M3FN conversion of x:
    every float32 in the binades [2**-12, 2) and [256, 448], and a dense random
    sample elsewhere in [-448, 448]."""
    m = np.arange(1 << 23, dtype=np.uint32)
    for ex in list(range(-12, 1)) + [8]:
        bits = (np.uint32(ex + 127) << 23) | m
        y = bits.view(np.float32)
        if ex == 8:
            y = y[y <= 448]
        for sgn in (1.0, -1.0):
            yy = (np.float32(sgn) * y).astype(np.float32)
            out = np.empty(yy.size, np.uint8)
            codec.codes_at(yy.ctypes.data, yy.size, 0, out.ctypes.data)
            assert np.array_equal(out, _torch_e4m3(yy)), (ex, sgn)
    r = np.random.default_rng(1)
    y = (r.standard_normal(2_000_000) * np.exp2(r.integers(-20, 9, 2_000_000))).astype(np.float32)
    y = np.clip(y, -448, 448).astype(np.float32)
    y[:1000] = 0
    y[1000:2000] = -0.0
    y[2000:3000] = np.float32(1e-42) * np.arange(1000, dtype=np.float32)
    out = np.empty(y.size, np.uint8)
    codec.codes_at(y.ctypes.data, y.size, 0, out.ctypes.data)
    assert np.array_equal(out, _torch_e4m3(y))


def test_scaled_codes_equal_torch_of_exactly_scaled_values(codec):
    r = np.random.default_rng(2)
    x = (r.standard_normal((20000, 32)) * np.exp2(r.integers(-126, 120, (20000, 1)))).astype(np.float32)
    x[:100] = (r.standard_normal((100, 32)) * 1e-40).astype(np.float32)     # subnormal blocks
    x[100:200] *= np.float32(0.02)
    codes = np.empty(x.size, np.uint8)
    sc = np.empty(20000, np.uint8)
    codec.blocks(x.ctypes.data, 20000, codes.ctypes.data, sc.ctypes.data)
    amax = np.abs(x.astype(np.float64)).max(axis=1)
    for b in range(0, 20000, 7):
        # brute force the least e with amax <= 448*2^e
        e = next(k for k in range(-127, 128) if amax[b] <= math.ldexp(448.0, k)) if amax[b] > 0 else -127
        assert sc[b] == e + 127, (b, amax[b], sc[b], e)
    e = sc.astype(np.int64) - 127
    y = np.ldexp(x.astype(np.float64), -e[:, None]).astype(np.float32)   # exact unless it underflows
    assert np.array_equal(codes.reshape(20000, 32), _torch_e4m3(y).reshape(20000, 32))


def test_bf16_bits_equal_torch(codec):
    low = np.arange(1 << 16, dtype=np.uint32)
    se = np.arange(512, dtype=np.uint32) << 23
    for hi7 in (0x00, 0x7E, 0x7F):
        bits = (se[:, None] | (np.uint32(hi7) << 16) | low[None, :]).ravel()
        out = np.empty(bits.size, np.uint16)
        codec.bf16(bits.ctypes.data, bits.size, out.ctypes.data)
        ref = torch.from_numpy(bits.view(np.float32).copy()).to(torch.bfloat16).view(torch.int16).numpy() \
            .view(np.uint16)
        nan = np.isnan(bits.view(np.float32))
        assert np.array_equal(out[~nan], ref[~nan])
        assert np.all(((out[nan] & 0x7F80) == 0x7F80) & ((out[nan] & 0x7F) != 0))


TILEMAP_SHIM = r"""
#include "tile_map.h"
int check(int tm_n, int tn_n, int *seen) {
  for (int p = 0; p < tm_n * tn_n; ++p) {
    int tm, tn;
    xcd_tile(p, tm_n, tn_n, &tm, &tn);
    if (tm < 0 || tm >= tm_n || tn < 0 || tn >= tn_n) return -1;
    if (seen[tm * tn_n + tn]++) return -2;
  }
  return 0;
}
"""


def test_xcd_tile_map_is_an_in_bounds_bijection(tmp_path):
    """The raw contraction's workgroup -> tile map (csrc/tile_map.h), compiled
    for the host: every grid it can be launched with maps onto its tiles
    exactly once and never outside them."""
    src = tmp_path / "tm.c"
    src.write_text(TILEMAP_SHIM)
    so = tmp_path / "tm.so"
    subprocess.run(["gcc", "-O1", "-shared", "-fPIC", "-I", CSRC, str(src), "-o", str(so)], check=True)
    L = ctypes.CDLL(str(so))
    L.check.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    dims = sorted(set([1, 2, 3, 4, 7, 8, 12, 16, 24, 32, 40, 56, 64, 72, 88, 96, 128, 224]))
    for m in dims:
        for n in dims:
            seen = np.zeros(m * n, np.int32)
            assert L.check(m, n, seen.ctypes.data) == 0, (m, n)
            assert np.all(seen == 1), (m, n)


SWZ_SHIM = r"""
#include "lds_swizzle.h"
int swz64(int r) { return lds_swz<64>(r); }
int swz32(int r) { return lds_swz<32>(r); }
"""


def test_lds_swizzle_conflict_free_and_load_consistent(tmp_path):
    """The contraction's LDS chunk swizzle (csrc/lds_swizzle.h), compiled for the
    host: (1) a fragment read -- lanes 0..31 on 32 consecutive rows, lanes 32..63
    on the next logical chunk -- puts every aligned group of 8 and of 16 lanes on
    distinct 16-byte bank groups (256- and 128-byte-per-cycle LDS models);
    (2) the swizzle repeats with the rows one buffer load spans, so a load's
    per-lane chunk pattern is the same for every row block it fills."""
    src = tmp_path / "swz.cpp"
    src.write_text(SWZ_SHIM.replace("int swz", 'extern "C" int swz'))
    so = tmp_path / "swz.so"
    subprocess.run(["g++", "-O1", "-shared", "-fPIC", "-I", CSRC, str(src), "-o", str(so)], check=True)
    L = ctypes.CDLL(str(so))
    for bk, fn in ((64, L.swz64), (32, L.swz32)):
        cpr, rb = bk // 8, bk * 2
        for base in range(0, 256, 32):
            for c in range(0, cpr, 2):
                addr = []
                for lane in range(64):
                    r = base + (lane & 31)
                    logical = c + (lane >> 5)
                    addr.append(r * rb + (logical ^ fn(r)) * 16)
                for g, mod in ((16, 16), (8, 8)):
                    for s0 in range(0, 64, g):
                        banks = [(a // 16) % mod for a in addr[s0:s0 + g]]
                        assert len(set(banks)) == g, (bk, base, c, s0, banks)
        rpi = 1024 // rb
        for nw in (4, 8):
            for r in range(rpi * nw):
                for i in range(1, 8):
                    assert fn(r) == fn(r + rpi * nw * i), (bk, nw, r, i)
        for r in range(64):                          # each row's chunks stay a permutation
            assert sorted(c ^ fn(r) for c in range(cpr)) == list(range(cpr))
