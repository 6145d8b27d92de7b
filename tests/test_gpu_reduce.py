"""GPU parity for the reduce-scatter tail (sshdp_rs_reduce / sshdp_rs_accumulate)
against the oracle (oracle/reduce.py), bit for bit: FP32 sums in the same
left-to-right order, and the same Philox4x64-10 randoms for the stochastic
rounding -- the oracle draws them from numpy's generator, the kernel computes
the published block function itself."""

import numpy as np
import pytest

from oracle import reduce as R
import mxfp8_weight_repack_amd as sh
from gpu_util import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sh.lib()


def _inputs(rng, k, n, dtype):
    xs = []
    for i in range(k):
        x = (rng.standard_normal(n) * 1e-3 * (1 + i)).astype(np.float32)
        if i == 0 and n >= 64:
            x[:8] = [np.nan, np.inf, -np.inf, -0.0, 1e-41, 3.3e38, 1e-45, -2.5]
        xs.append(x if dtype == "fp32" else (x.view(np.uint32) >> 16).astype(np.uint16))
    return xs


def _dev(a):
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def _eq_bits(got, exp):
    g = np.asarray(got).view(np.uint32 if np.asarray(got).dtype == np.float32 else np.uint16)
    e = np.asarray(exp).view(g.dtype)
    if g.dtype == np.uint32:
        nan = np.isnan(np.asarray(exp))
    else:
        nan = ((e & 0x7F80) == 0x7F80) & ((e & 0x7F) != 0)
    assert np.array_equal(g[~nan], e[~nan])
    if g.dtype == np.uint32:
        assert np.all(np.isnan(np.asarray(got)[nan]))
    else:
        assert np.all(((g[nan] & 0x7F80) == 0x7F80) & ((g[nan] & 0x7F) != 0))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("k", [1, 3, 8])
@pytest.mark.parametrize("n", [16, 4096 * 5 + 16 * 37])
def test_rs_reduce_matches_oracle(dtype, k, n):
    say(f"rs_reduce {dtype} k={k} n={n}")
    rng = np.random.default_rng(k * 1000 + n)
    xs = _inputs(rng, k, n, dtype)
    dev = [_dev(x) for x in xs]
    s = torch.cuda.current_stream().cuda_stream
    out32 = torch.empty(n, dtype=torch.float32, device="cuda")
    sh.rs_reduce(dev, dtype, out32, "fp32", n, stream=s)
    out16 = torch.empty(n, dtype=torch.int16, device="cuda")
    seed, ctr, g0 = 0xC0FFEE + k, 3, 4096 * 7
    sh.rs_reduce(dev, dtype, out16, "bf16_sr", n, seed, ctr, g0, stream=s)
    torch.cuda.synchronize()
    _eq_bits(out32.cpu().numpy(), R.rs_reduce(xs, dtype, "fp32"))
    _eq_bits(out16.cpu().numpy().view(np.uint16), R.rs_reduce(xs, dtype, "bf16_sr", seed, ctr, g0))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rs_accumulate_matches_oracle_over_microbatches(dtype):
    say(f"rs_accumulate {dtype}")
    rng = np.random.default_rng(7)
    n = 4096 * 3 + 48
    g_ref = np.zeros(n, np.float32)
    g = torch.full((n,), 123.0, dtype=torch.float32, device="cuda")   # stale contents: first must overwrite
    s = torch.cuda.current_stream().cuda_stream
    for mb in range(4):
        xs = _inputs(rng, 2, n, dtype)
        if mb:
            for x in xs:
                x[:8] = 0                                              # keep NaN/Inf out after the first
        sh.rs_accumulate([_dev(x) for x in xs], dtype, g, n, first=(mb == 0), stream=s)
        g_ref = R.rs_accumulate(xs, dtype, g_ref, first=(mb == 0))
        torch.cuda.synchronize()
        _eq_bits(g.cpu().numpy(), g_ref)


def test_rs_full_size_sampled():
    """The dense block d=2048's gradient (60,821,504 elements, padded to 16)
    from 4 bf16 slices: SR partial and its accumulation, checked against the
    oracle on sampled ranges spread over the whole tensor."""
    n = (60821504 + 15) // 16 * 16
    say(f"rs full size n={n}")
    rng = np.random.default_rng(9)
    xs = [(rng.standard_normal(n, dtype=np.float32) * np.float32(1e-3)).view(np.uint32) >> 16 for _ in range(4)]
    xs = [x.astype(np.uint16) for x in xs]
    dev = [_dev(x) for x in xs]
    s = torch.cuda.current_stream().cuda_stream
    part = torch.empty(n, dtype=torch.int16, device="cuda")
    sh.rs_reduce(dev, "bf16", part, "bf16_sr", n, 99, 1, 0, stream=s)
    g = torch.zeros(n, dtype=torch.float32, device="cuda")
    sh.rs_accumulate([part, part], "bf16", g, n, first=True, stream=s)
    torch.cuda.synchronize()
    for start in list(range(0, n, n // 7)) + [n - 4096]:
        lo = start // 16 * 16
        hi = min(lo + 4096, n)
        sl = [x[lo:hi] for x in xs]
        exp = R.sr_bf16(R.fp32_sum(sl, "bf16"), R.philox_bits16(99, 1, lo, hi - lo))
        got = part[lo:hi].cpu().numpy().view(np.uint16)
        assert np.array_equal(got, exp), lo
        assert np.array_equal(g[lo:hi].cpu().numpy(), R.rs_accumulate([exp, exp], "bf16", None, first=True))
    del dev, part, g


def test_rs_argument_errors():
    t = torch.zeros(64, dtype=torch.float32, device="cuda")
    for call, name in [
        (lambda: sh.rs_reduce([t], "fp32", t, "fp32", 40), "SCHEMA"),             # n % 16
        (lambda: sh.rs_reduce([t], "fp32", t, "fp32", 32, g0=8), "SCHEMA"),       # g0 % 16
        (lambda: sh.rs_reduce([t] * 9, "fp32", t, "fp32", 32), "ARG"),            # > 8 inputs
        (lambda: sh.rs_reduce([t[1:]], "fp32", t, "fp32", 16), "ALIGN"),          # misaligned input
        (lambda: sh.rs_accumulate([t], "fp32", t[2:], 16, True), "ALIGN"),
    ]:
        with pytest.raises(sh.SshdpError) as e:
            call()
        assert e.value.name == name
    sh.rs_reduce([t], "fp32", t, "fp32", 0)                                       # empty is a no-op
