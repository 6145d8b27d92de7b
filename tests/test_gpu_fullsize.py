"""GPU parity at the workloads' full sizes, in the launch configuration bench.py
times (the same plan, tile tables and kernels), on outputs the oracle can
compute one unit at a time.

* dense block d=2048 (the bench workload): several heads, the O projection,
  a tall MLP matrix and the wide one against the oracle's fp64 Newton-Schulz;
  both norm vectors (AdamW); G bit-exact on the packed QKV and the O region.
* MoE 64 experts: zero-gradient experts bit-identical, sampled non-zero
  experts (both orientations) against the oracle; G bit-exact on sampled
  expert regions.
* flat ragged shard of 5e8 elements (fused AdamW + G): sampled tensors'
  w, m, v against the oracle over two steps (a fresh gradient in the second),
  their codes and scales bit-exact, every padding run untouched.
* dense block d=8192: sampled heads, the 8192 x 8192 O projection and the
  28672 x 8192 gate projection against the oracle's fp64 iteration (about 60
  TFLOP of host BLAS, a few minutes on the host's cores; each Newton-Schulz
  step reports as it ends); the other two 8192 x 28672 units against the same
  quintic iteration run by torch in fp32 on the GPU (an extra check); G
  bit-exact on sampled regions.
"""

import numpy as np
import pytest

import oracle
from oracle.views import resolve_views, unit_indices
import mxfp8_weight_repack_amd as sh
import workloads
from gpu_util import DeviceState, adam_elementwise_ok, rel_fro, say, MUON, ADAM

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

NS_TOL = 2e-2


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sh.lib()


def _run(wl):
    st = DeviceState(wl)
    st.step(1)
    torch.cuda.synchronize()
    return st


def _check_muon_unit(st, res, i, w0, g, progress=False):
    r = res[i]
    idx = unit_indices(r)
    w_gpu = st.w[torch.from_numpy(idx.ravel()).cuda()].cpu().numpy().reshape(idx.shape)
    if progress:
        # f0 from m = 0 gives m = g, u = bf16(g); then the oracle's f1 step by step
        say(f"  unit {i} {r['rows']}x{r['cols']}: float64 oracle iteration on the host ...")
        vdir = oracle.newton_schulz(oracle.bf16_rne(g[idx]),
                                    progress=lambda k: say(f"    oracle Newton-Schulz step {k}/5 done"))
    else:
        _, _, vdir = oracle.muon_update_unit(w0[idx], g[idx], np.zeros(idx.shape, np.float32),
                                             oracle.OracleHyper())
    v_gpu = (w0[idx].astype(np.float64) - w_gpu) / np.float32(MUON["lr"])
    e = rel_fro(v_gpu, vdir)
    say(f"  unit {i} {r['rows']}x{r['cols']}: rel-Frobenius {e:.3e}")
    assert e <= NS_TOL, (i, e)


def _check_requant_region(st, r, layout):
    idx = unit_indices(r).ravel()
    ti = torch.from_numpy(idx).cuda()
    w = st.w[ti].cpu().numpy().reshape(r["rows"], r["cols"])
    codes = st.codes[ti].cpu().numpy().reshape(r["rows"], r["cols"])
    sidx = oracle.scale_index(layout, r["abs"], r["rows"], r["cols"])
    scales = st.scales[torch.from_numpy(sidx.ravel()).cuda()].cpu().numpy().reshape(sidx.shape)
    from oracle.mxfp8 import quantize_blocks_fast
    c_ref, s_ref = quantize_blocks_fast(w)
    assert np.array_equal(codes, c_ref)
    assert np.array_equal(scales, s_ref)


def test_dense_block_d2048_full_size():
    wl = workloads.config(2)
    say(f"full size: {wl.name}")
    w0, g = wl.arrays()
    st = _run(wl)
    res = resolve_views(wl.nodes, wl.root_numel, wl.scale_layout)
    muon = [i for i, r in enumerate(res) if r["is_unit"] and r["optimizer"] == "muon"]
    heads = [i for i in muon if res[i]["parent"] == 0]
    others = [i for i in muon if res[i]["parent"] != 0]
    for i in heads[:2] + heads[-2:] + others:           # O, gate (tall), up (tall), down (wide)
        _check_muon_unit(st, res, i, w0, g)
    for i, r in enumerate(res):
        if r["is_unit"] and r["optimizer"] == "adamw":
            idx = unit_indices(r)
            z = np.zeros(idx.shape, np.float32)
            w_ref, _, _ = oracle.adamw_step(w0[idx], g[idx], z, z, 1, **ADAM)
            w_gpu = st.w[torch.from_numpy(idx.ravel()).cuda()].cpu().numpy().reshape(idx.shape)
            assert np.max(np.abs(w_gpu - w_ref)) <= 1e-6 * np.max(np.abs(w_ref))
            assert adam_elementwise_ok(w_gpu, w_ref) <= 1.0
    q = [r for r in res if r["quantize"]]
    for r in q[:2]:
        _check_requant_region(st, r, wl.scale_layout)


def test_moe_64_experts_full_size():
    wl = workloads.config(3)
    say(f"full size: {wl.name}")
    w0, g = wl.arrays()
    st = _run(wl)
    res = resolve_views(wl.nodes, wl.root_numel, wl.scale_layout)
    for i in wl.zero_grad_units:
        idx = unit_indices(res[i]).ravel()
        w_gpu = st.w[torch.from_numpy(idx).cuda()].cpu().numpy()
        assert np.array_equal(w_gpu.view(np.uint32), w0[idx].view(np.uint32)), i
    muon = [i for i, r in enumerate(res) if r["is_unit"] and r["optimizer"] == "muon"
            and i not in wl.zero_grad_units]
    tall = [i for i in muon if res[i]["rows"] > res[i]["cols"]]
    wide = [i for i in muon if res[i]["rows"] < res[i]["cols"]]
    for i in wide[:2] + tall[:2] + [wide[-1], tall[-1]]:
        _check_muon_unit(st, res, i, w0, g)
    for r in [r for r in res if r["quantize"]]:        # first expert (+ more) of every bank
        _check_requant_region_tile(st, r, dict(r, rows=2048))


def _check_requant_region_tile(st, region, sub):
    """Quantise the first sub['rows'] rows of a TILE32X4 region on the oracle
    and compare codes and the matching scale bytes."""
    from oracle.mxfp8 import quantize_blocks_fast
    rows, cols = sub["rows"], region["cols"]
    idx = (region["abs"] + np.arange(rows * cols, dtype=np.int64))
    ti = torch.from_numpy(idx).cuda()
    w = st.w[ti].cpu().numpy().reshape(rows, cols)
    codes = st.codes[ti].cpu().numpy().reshape(rows, cols)
    c_ref, s_ref = quantize_blocks_fast(w)
    assert np.array_equal(codes, c_ref)
    sidx = oracle.scale_index("tile32x4", region["abs"], region["rows"], cols)[:rows]
    scales = st.scales[torch.from_numpy(sidx.ravel()).cuda()].cpu().numpy().reshape(sidx.shape)
    assert np.array_equal(scales, s_ref)


def _torch_ns32(u, a=3.4445, b=-4.7750, c=2.0315, eps=1e-7, steps=5):
    X = u.float()
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.t().contiguous()
    X = X / (torch.linalg.norm(X.double()).float() + eps)
    for _ in range(steps):
        A = X @ X.t().contiguous()
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.t().contiguous() if tall else X


@pytest.mark.timeout(1200)
def test_dense_block_d8192_full_size():
    wl = workloads.config(5)
    say(f"full size: {wl.name}")
    w0, g = wl.arrays()
    st = _run(wl)
    res = resolve_views(wl.nodes, wl.root_numel, wl.scale_layout)
    muon = [i for i, r in enumerate(res) if r["is_unit"] and r["optimizer"] == "muon"]
    heads = [i for i in muon if res[i]["parent"] == 0]
    for i in heads[:2] + heads[-1:]:
        _check_muon_unit(st, res, i, w0, g)
    large = [j for j in muon if res[j]["parent"] != 0]
    o_proj = [j for j in large if res[j]["rows"] == res[j]["cols"]]
    tall = [j for j in large if res[j]["rows"] > res[j]["cols"]]
    assert len(o_proj) == 1 and len(tall) == 2
    # the O projection (8192 x 8192) and the gate projection (28672 x 8192, iterated on its
    # transpose): against the float64 oracle
    for i in o_proj + tall[:1]:
        _check_muon_unit(st, res, i, w0, g, progress=True)
    # the other two MLP units: against torch's fp32 iteration of the same map, on the GPU
    for i in [j for j in large if j not in o_proj + tall[:1]]:
        r = res[i]
        a0 = r["abs"]
        n = r["rows"] * r["cols"]
        u = torch.from_numpy(oracle.bf16_rne(g[a0:a0 + n])).cuda().reshape(r["rows"], r["cols"])
        v_ref = _torch_ns32(u)
        w_before = torch.from_numpy(w0[a0:a0 + n]).cuda().reshape(r["rows"], r["cols"])
        v_gpu = (w_before.double() - st.w[a0:a0 + n].reshape(r["rows"], r["cols"]).double()) / np.float32(0.02)
        e = (torch.linalg.norm(v_gpu - v_ref.double()) / torch.linalg.norm(v_ref.double())).item()
        say(f"  unit {i} {r['rows']}x{r['cols']} vs torch fp32: rel-Frobenius {e:.3e}")
        assert e <= NS_TOL, (i, e)
        del u, v_ref, w_before, v_gpu
    q = [r for r in res if r["quantize"]]
    for r in q:
        sub = dict(r, rows=32)
        _check_requant_region_tile(st, r, sub)


def test_flat_shard_5e8_full_size():
    wl = workloads.config(4)
    say(f"full size: {wl.name}")
    w0, g = wl.arrays()
    g2 = wl.gradient(2)                                     # a fresh gradient for the second step
    st = DeviceState(wl)
    st.step(1)
    st.g.copy_(torch.from_numpy(g2))
    st.step(2)
    torch.cuda.synchronize()
    res = resolve_views(wl.nodes, wl.root_numel, wl.scale_layout)
    units = [i for i, r in enumerate(res) if r["is_unit"]]
    rng = np.random.default_rng(4)
    pick = sorted(set(rng.choice(units, 12, replace=False).tolist() + [units[0], units[-1]]))
    for i in pick:
        r = res[i]
        a, n = r["abs"], r["rows"] * r["cols"]
        if n > 4_000_000:                                   # a large tensor: check a window of it
            a, n = a + (n // 2) // 32 * 32, 1 << 20
        sl = slice(a, a + n)
        z = np.zeros(n, np.float32)
        w1, m1, v1 = oracle.adamw_step(w0[sl], g[sl], z, z, 1, **ADAM)
        w2, m2, v2 = oracle.adamw_step(w1, g2[sl], m1, v1, 2, **ADAM)
        tw = st.w[a:a + n].cpu().numpy()
        tm = st.m[a:a + n].cpu().numpy()
        tv = st.v[a:a + n].cpu().numpy()
        assert np.max(np.abs(tw - w2)) <= 1e-6 * np.max(np.abs(w2)), i
        assert adam_elementwise_ok(tw, w2) <= 1.0, i
        assert np.max(np.abs(tm - m2)) <= 1e-6 * np.max(np.abs(m2)), i
        assert np.max(np.abs(tv - v2)) <= 1e-5 * np.max(np.abs(v2)), i
        # G on the GPU-updated weight, bit-exact (1x32 blocks along the flat region)
        # (a 1-D tensor's last block runs into its zero padding, which G quantises with it)
        from oracle.mxfp8 import quantize_blocks_fast
        nq = (n + 31) // 32 * 32
        tq = st.w[a:a + nq].cpu().numpy()
        c_ref, s_ref = quantize_blocks_fast(tq.reshape(-1, 32))
        assert np.array_equal(st.codes[a:a + nq].cpu().numpy(), c_ref.ravel()), i
        assert np.array_equal(st.scales[a // 32:(a + nq) // 32].cpu().numpy(), s_ref.ravel()), i
        say(f"  tensor {i} ({r['rows']}x{r['cols']}): ok")
    for s0, n in wl.padding:
        assert not torch.any(st.w[s0:s0 + n]).item() and not torch.any(st.m[s0:s0 + n]).item()
