"""Pins for the oracle's reduce-scatter tail (oracle/reduce.py; CPU only).

* stochastic rounding: averaged over all 2^16 random values it returns x
  exactly (E[SR(x)] = x, a closed form); every result is one of the two BF16
  neighbours of x, and the larger-magnitude one for exactly k of the 2^16
  random values; representable values, +-0, +-Inf and NaN are kept;
* random bits: the documented element -> (block, word, 16-bit part) mapping on
  numpy's Philox4x64-10 stream (a library generator), and offset consistency;
* FP32 summation order: ((1e8 + 1) - 1e8) is 0 in left-to-right FP32 (an FP64
  or reordered sum gives 1); first-microbatch initialisation vs accumulation.
"""

import numpy as np

from oracle import reduce as R


def _vals(bits16):
    return (bits16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_sr_mean_over_all_randoms_is_exact_and_results_are_neighbours():
    rng = np.random.default_rng(41)
    x = (rng.standard_normal(300) * np.exp2(rng.integers(-140, 120, 300))).astype(np.float32)
    x[:5] = [1e-41, -3e-42, 2.5e-39, 3.3e38, -1.7e-38]
    r = np.arange(65536)
    for xi in x:
        b = R.sr_bf16(np.full(65536, xi, np.float32), r)
        v = _vals(b)
        assert np.sum(v) / 65536.0 == float(xi), xi
        u = np.unique(v)
        assert len(u) <= 2
        if len(u) == 2:                                   # adjacent BF16 values bracketing x
            lo, hi = sorted(u, key=abs)
            nb = int(np.sum(v == hi))
            assert abs(lo) < abs(float(xi)) < abs(hi)
            assert abs(np.float32(hi).view(np.uint32) - np.float32(lo).view(np.uint32)) == 1 << 16
            assert 0 < nb < 65536
            assert np.all(v[65536 - nb:] == hi) and np.all(v[:65536 - nb] == lo)   # monotone in r


def test_sr_keeps_representable_and_special_values():
    x = np.array([1.0, -2.5, 0.0, -0.0, np.inf, -np.inf, 3.3895313892515355e38, 2.0 ** -133], np.float32)
    for r in (0, 1, 40000, 65535):
        b = R.sr_bf16(x, np.full(x.size, r))
        assert b.tolist() == [0x3F80, 0xC020, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x7F7F, 0x0001]
    b = R.sr_bf16(np.array([np.nan], np.float32), [123])
    assert (b[0] & 0x7F80) == 0x7F80 and (b[0] & 0x7F) != 0
    # just below FLT_MAX rounds up to +Inf for large r (Inf is the next value up)
    assert R.sr_bf16(np.array([3.4e38], np.float32), [65535])[0] == 0x7F80


def test_philox_bits_follow_the_documented_mapping():
    seed, ctr = 0x1234_5678_9ABC, 7
    bits = R.philox_bits16(seed, ctr, 0, 64)
    raw = np.random.Philox(key=seed, counter=ctr << 64).random_raw(16).astype(np.uint64)
    for g in range(64):
        word = raw[(g // 16) * 4 + (g // 4) % 4]
        assert bits[g] == (int(word) >> (16 * (g % 4))) & 0xFFFF
    assert np.array_equal(R.philox_bits16(seed, ctr, 32, 32), bits[32:])
    assert not np.array_equal(R.philox_bits16(seed, ctr + 1, 0, 64), bits)
    assert not np.array_equal(R.philox_bits16(seed + 1, ctr, 0, 64), bits)


def test_fp32_sum_order_and_accumulation():
    a = [np.array([1e8], np.float32), np.array([1.0], np.float32), np.array([-1e8], np.float32)]
    assert R.fp32_sum(a, "fp32")[0] == 0.0                 # 1e8 + 1 rounds to 1e8 in FP32
    assert R.fp32_sum([a[0], a[2], a[1]], "fp32")[0] == 1.0
    g = np.array([0.5], np.float32)
    assert R.rs_accumulate(a[:2], "fp32", g, first=True)[0] == np.float32(1e8)
    assert R.rs_accumulate([np.array([0.25], np.float32)], "fp32", g, first=False)[0] == 0.75
    bf = np.array([0x3F80, 0xC000], np.uint16)            # 1.0, -2.0
    assert R.rs_accumulate([bf, bf], "bf16", np.zeros(2, np.float32), first=True).tolist() == [2.0, -4.0]
    assert R.rs_reduce([bf, bf], "bf16", "fp32").tolist() == [2.0, -4.0]
    assert R.rs_reduce([bf, bf], "bf16", "bf16_sr", 1, 2, 0).tolist() == [0x4000, 0xC080]
