"""GPU parity: the HIP library (through its C ABI) against the oracle on the
same seeded inputs.

Gates (stated per test):
* MXFP8 codes and scales: bit-exact when both sides quantise the same fp32
  weight (the GPU-updated weight is fed to the oracle's quantiser);
* AdamW main weights: normwise relative error <= 1e-6
  (max |w_gpu - w_ref| / max |w_ref|), and elementwise
  |w_gpu - w_ref| <= 1e-6 |w_ref| + 4 lr 2^-24;
* Newton-Schulz: per unit, relative Frobenius error <= 2e-2 of the direction
  recovered from the weight change, v = (w_before - w_after) / lr;
* zero-gradient units: bit-identical weights; elements outside every unit:
  untouched.
"""

import dataclasses

import numpy as np
import pytest

import oracle
from oracle.views import ViewError, resolve_views, unit_indices
import mxfp8_weight_repack_amd as sh
import workloads
from gpu_util import DeviceState, adam_elementwise_ok, oracle_step, rel_fro, say, MUON, ADAM

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

NS_TOL = 2e-2
ADAM_TOL = 1e-6


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sh.lib()


def _bf16_host(x):
    return oracle.bf16_rne(x).astype(np.float64)


# ----------------------------------------------------------------------------- GEMM
@pytest.mark.parametrize("tile,M,N,K,batch", [(128, 128, 256, 192, 2), (128, 384, 128, 640, 3),
                                              (256, 256, 512, 320, 2), (256, 512, 256, 128, 1)])
def test_gemm_nt_against_fp64(tile, M, N, K, batch):
    say(f"gemm tile={tile} M={M} N={N} K={K} batch={batch}")
    r = np.random.default_rng(M * 7 + N + K + tile)
    P = r.standard_normal((batch, M, K)).astype(np.float32)
    Q = r.standard_normal((batch, N, K)).astype(np.float32)
    D = r.standard_normal((batch, M, N)).astype(np.float32)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()
    tP, tQ = bf(P), bf(Q)
    tD = bf(np.ascontiguousarray(D.transpose(0, 2, 1)))          # the entry takes D transposed
    O = torch.zeros(batch, M, N, dtype=torch.bfloat16, device="cuda")
    OT = torch.zeros(batch, N, M, dtype=torch.bfloat16, device="cuda")
    sh.gemm_bf16_nt(tP, tQ, tD, O, OT, M, N, K, batch, 0.75, -1.5, tile,
                    torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = 0.75 * np.einsum("bik,bjk->bij", _bf16_host(P), _bf16_host(Q)) - 1.5 * _bf16_host(D)
    got = O.float().cpu().numpy().astype(np.float64)
    scale = np.sqrt(K) + 2.0
    assert np.max(np.abs(got - ref)) <= 2 ** -7 * scale * 1.5 + 1e-3
    assert rel_fro(got, ref) < 4e-3
    assert torch.equal(OT, O.transpose(1, 2).contiguous())


@pytest.mark.parametrize("tile,M,N,K,batch", [(1281, 128, 128, 192, 2), (1281, 384, 384, 640, 3),
                                              (2561, 256, 256, 320, 2), (2561, 512, 512, 128, 1)])
def test_gemm_kmajor_against_fp64(tile, M, N, K, batch):
    """The K-major operand path (transposing LDS reads): O = alpha P^T Q with
    P K x M and Q K x N row-major, M = N (one row pitch, as for the Gram read
    from X^T)."""
    say(f"gemm K-major tile={tile} M={M} N={N} K={K} batch={batch}")
    r = np.random.default_rng(M * 7 + N + K + tile)
    P = r.standard_normal((batch, K, M)).astype(np.float32)
    Q = r.standard_normal((batch, K, N)).astype(np.float32)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()
    O = torch.zeros(batch, M, N, dtype=torch.bfloat16, device="cuda")
    OT = torch.zeros(batch, N, M, dtype=torch.bfloat16, device="cuda")
    sh.gemm_bf16_nt(bf(P), bf(Q), None, O, OT, M, N, K, batch, 0.75, 0.0, tile,
                    torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = 0.75 * np.einsum("bki,bkj->bij", _bf16_host(P), _bf16_host(Q))
    got = O.float().cpu().numpy().astype(np.float64)
    scale = np.sqrt(K) + 2.0
    assert np.max(np.abs(got - ref)) <= 2 ** -7 * scale * 1.5 + 1e-3
    assert rel_fro(got, ref) < 4e-3
    assert torch.equal(OT, O.transpose(1, 2).contiguous())


# ----------------------------------------------------------------------------- G alone
def _specials(w, wl):
    """Plant NaN/Inf/-0/subnormal/zero blocks inside the quantised regions."""
    w = w.copy()
    res = resolve_views(wl.nodes, wl.root_numel)
    q = [r for r in res if r["quantize"]]
    a = q[0]["abs"]
    w[a:a + 32] = 0.0
    w[a + 32:a + 64] = -0.0
    w[a + 64 + 5] = np.nan
    w[a + 96 + 31] = np.inf
    w[a + 128:a + 160] = np.float32(1e-41)
    w[a + 160] = np.float32(448.0)
    w[a + 192:a + 224] *= np.float32(1e30)
    return w


@pytest.mark.parametrize("case", ["c1", "c2s", "c3s", "c4s", "c5s", "ragged"])
@pytest.mark.parametrize("layout", ["rowmajor", "tile32x4", "block32x32"])
def test_requant_bit_exact(case, layout):
    wl = workloads.ragged_mix() if case == "ragged" else workloads.config(int(case[1]), small=case.endswith("s"))
    if layout == "tile32x4" and wl.scale_layout != "tile32x4":
        pytest.skip("workload has quantised regions that are not 32x128 tiles")
    if layout == "block32x32":
        try:
            resolve_views(wl.nodes, wl.root_numel, layout)
        except ViewError:
            pytest.skip("workload has quantised regions that are not whole 32x32 blocks")
    say(f"requant {wl.name} {layout}")
    w0, _ = wl.arrays()
    w = _specials(w0, wl)
    st = DeviceState(wl, w=w, layout=layout)
    st.codes.fill_(0xAB)
    st.scales.fill_(0xCD)
    sh.requant_mxfp8(st.plan, st.w, st.codes, st.scales, st.stream())
    h = st.host()
    codes = np.full(wl.root_numel, 0xAB, np.uint8)
    scales = np.full(st.stats["scale_bytes"], 0xCD, np.uint8)
    res = resolve_views(wl.nodes, wl.root_numel, layout)
    oracle.requant_root(w, res, layout, codes, scales)
    assert np.array_equal(h["codes"], codes)
    assert np.array_equal(h["scales"], scales)
    assert np.array_equal(h["w"].view(np.uint32), w.view(np.uint32))


# ----------------------------------------------------------------------------- AdamW alone
def test_adamw_alone_matches_oracle_over_steps():
    """Four AdamW steps with a fresh gradient each step (so the moment
    recurrences, not only the bias correction, decide the result)."""
    wl = workloads.config(4, small=True)
    say(f"adamw {wl.name}")
    w0, _ = wl.arrays()
    st = DeviceState(wl)
    w, m, v = w0.copy(), np.zeros_like(w0), np.zeros_like(w0)
    res = resolve_views(wl.nodes, wl.root_numel)
    for t in (1, 2, 3, 4):
        g = wl.gradient(t)
        st.g.copy_(torch.from_numpy(g))
        sh.update_adamw(st.plan, st.bufs(), sh.adamw_hp(**ADAM), t, st.stream())
        for r in res:
            if r["is_unit"]:
                idx = unit_indices(r)
                w[idx], m[idx], v[idx] = oracle.adamw_step(w[idx], g[idx], m[idx], v[idx], t, **ADAM)
        h = st.host()
        assert np.max(np.abs(h["w"] - w)) <= ADAM_TOL * np.max(np.abs(w))
        e = adam_elementwise_ok(h["w"], w)
        say(f"  step {t}: elementwise AdamW error / bound {e:.3f}")
        assert e <= 1.0, t
        assert np.max(np.abs(h["m"] - m)) <= 1e-6 * np.max(np.abs(m))
        assert np.max(np.abs(h["v"] - v)) <= 1e-5 * np.max(np.abs(v))
    pad = np.ones(wl.root_numel, bool)
    for r in res:
        if r["is_unit"]:
            pad[unit_indices(r).ravel()] = False
    assert np.all(h["w"][pad] == 0) and np.all(h["m"][pad] == 0) and np.all(h["v"][pad] == 0)


# ----------------------------------------------------------------------------- whole step
CASES = ["c1", "c2s", "c3s", "c4s", "c5s", "ragged"]


def _wl(case):
    return workloads.ragged_mix() if case == "ragged" else workloads.config(int(case[1]),
                                                                            small=case.endswith("s"))


def check_step(wl, layout, h, ref, dirs, w0, muon_lr=MUON["lr"], units=None):
    res = resolve_views(wl.nodes, wl.root_numel, layout)
    touched = np.zeros(wl.root_numel, bool)
    worst = 0.0
    for i, r in enumerate(res):
        if not r["is_unit"]:
            continue
        idx = unit_indices(r)
        touched[idx.ravel()] = True
        if units is not None and i not in units:
            continue
        if r["optimizer"] == "muon":
            if i in wl.zero_grad_units:
                assert np.array_equal(h["w"][idx].view(np.uint32), w0[idx].view(np.uint32)), i
                continue
            v_gpu = (w0[idx].astype(np.float64) - h["w"][idx].astype(np.float64)) / np.float32(muon_lr)
            e = rel_fro(v_gpu, dirs[i])
            worst = max(worst, e)
            assert e <= NS_TOL, (i, r["rows"], r["cols"], e)
            assert np.max(np.abs(h["m"][idx] - ref["m"][idx])) <= 1e-6 * max(np.max(np.abs(ref["m"][idx])), 1e-30)
        else:
            ww, wr = h["w"][idx], ref["w"][idx]
            assert np.max(np.abs(ww - wr)) <= ADAM_TOL * np.max(np.abs(wr)), i
            assert adam_elementwise_ok(ww, wr) <= 1.0, i
    if units is None:
        assert np.array_equal(h["w"][~touched].view(np.uint32), w0[~touched].view(np.uint32))
        assert np.all(h["m"][~touched] == 0) and np.all(h["v"][~touched] == 0)
    # G on the GPU-updated weight: bit-exact against the oracle's quantiser
    codes = np.zeros(wl.root_numel, np.uint8)
    scales = np.zeros(h["scales"].size, np.uint8)
    oracle.requant_root(h["w"], res, layout, codes, scales)
    qmask = np.zeros(wl.root_numel, bool)
    smask = np.zeros(scales.size, bool)
    for r in res:
        if r["quantize"]:
            qmask[unit_indices(r).ravel()] = True
            smask[oracle.scale_index(layout, r["abs"], r["rows"], r["cols"]).ravel()] = True
    assert np.array_equal(h["codes"][qmask], codes[qmask])
    assert np.array_equal(h["scales"][smask], scales[smask])
    return worst


@pytest.mark.parametrize("case", CASES)
def test_update_step_parity(case):
    wl = _wl(case)
    say(f"update_step {wl.name} ({wl.scale_layout})")
    w0, g = wl.arrays()
    st = DeviceState(wl)
    st.step(1)
    h = st.host()
    z = np.zeros_like(w0)
    ref, dirs = oracle_step(wl, wl.scale_layout, w0, g, z, z, 1)
    worst = check_step(wl, wl.scale_layout, h, ref, dirs, w0)
    say(f"  worst NS rel-Frobenius {worst:.3e}")


@pytest.mark.parametrize("kind", ["g_only", "muon_only", "adamw_g"])
def test_update_step_degenerate_plans(kind):
    """A plan without Muon units, without AdamW units or without anything to
    quantise: the step takes NULL for the hyper-parameters and buffers of the
    missing part (as the ABI allows) and still matches the oracle; a quantised
    region holding no unit gets plain G (not the fused AdamW pass)."""
    wl = workloads.degenerate(kind)
    say(f"update_step {wl.name}")
    S = DeviceState(wl)
    n = S.stats
    muon, adam, quant = n["n_muon_units"] > 0, n["n_adamw_units"] > 0, n["n_quant_regions"] > 0
    if kind == "g_only" or kind == "adamw_g":
        assert n["fused_quant_elems"] == (0 if kind == "g_only" else 4 * 224)
    b = sh.buffers(S.w, S.g if muon or adam else None, S.m if muon or adam else None, S.v if adam else None,
                   S.codes if quant else None, S.scales if quant else None)
    if quant:
        with pytest.raises(sh.SshdpError) as e:                # G needs its code and scale roots
            sh.update_step(S.plan, sh.buffers(S.w, S.g, S.m, S.v), sh.muon_hp(**MUON), sh.adamw_hp(**ADAM), 1,
                           S.ws, S.ws_bytes, S.stream())
        assert e.value.name == "ARG"
    sh.update_step(S.plan, b, sh.muon_hp(**MUON) if muon else None, sh.adamw_hp(**ADAM) if adam else None, 1,
                   S.ws if muon else None, S.ws_bytes if muon else 0, S.stream())
    h = S.host()
    w0, g = wl.arrays()
    z = np.zeros_like(w0)
    ref, dirs = oracle_step(wl, wl.scale_layout, w0, g, z, z, 1)
    check_step(wl, wl.scale_layout, h, ref, dirs, w0)
    if quant:
        assert np.any(h["codes"] != 0)


@pytest.mark.parametrize("policy,gram", [("small", "auto"), ("large", "auto"), ("auto", "auto"),
                                         ("small", "nt"), ("auto", "nt")])
def test_update_step_parity_tile_policies(policy, gram):
    """Newton-Schulz products split into a 256-tile leading block and 128-tile
    strips (Gram/poly: the column strip and its mirror; update: the L-shaped
    rest) against the oracle, with every product in 128-tiles, and with the
    planner's own choice; each also with every Gram reading X row-major
    (gram="nt") instead of X^T."""
    wl = workloads.mixed_tiles()
    say(f"update_step {wl.name} tiles={policy} gram={gram}")
    st = DeviceState(wl, plan_kw=dict(ns_tiles=policy, ns_gram=gram))
    groups = st.plan.groups()
    if gram == "nt":
        assert all(g["gram_kmajor"] == 0 for g in groups)
    else:
        assert all(g["gram_kmajor"] == (g["gram256"] == 0) for g in groups)
    if policy == "large":
        assert any(0 < g["gram256"] < g["r_pad"] for g in groups)
        assert any(0 < g["upd256_rows"] < g["r_pad"] for g in groups)
        assert any(0 < g["upd256_cols"] < g["c_pad"] for g in groups)
    if policy == "small":
        assert all(g["gram256"] == g["upd256_rows"] == 0 for g in groups)
    w0, g = wl.arrays()
    st.step(1)
    h = st.host()
    z = np.zeros_like(w0)
    ref, dirs = oracle_step(wl, wl.scale_layout, w0, g, z, z, 1)
    worst = check_step(wl, wl.scale_layout, h, ref, dirs, w0)
    say(f"  worst NS rel-Frobenius {worst:.3e}")


_LONG_K_REF = {}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("policy", ["auto", "small"])
def test_update_step_parity_long_k_units(policy):
    """r = 4096, c = 4224 units (wide and tall) against the float64 oracle: the
    default plan runs their Gram and polynomial in 256-tiles plus a 128 strip
    (row-major X operands) and the update with K = 4096 in the long-K tile
    order; with every product in 128-tiles the Gram reads X^T (K-major) at
    K = 4224.  The oracle's result is computed once for both plans."""
    wl = workloads.long_k_units()
    say(f"update_step {wl.name} tiles={policy}")
    st = DeviceState(wl, plan_kw=dict(ns_tiles=policy))
    (gi,) = st.plan.groups()
    if policy == "auto":
        assert (gi["gram256"], gi["upd256_rows"], gi["upd256_cols"], gi["gram_kmajor"]) == (4096, 4096, 4096, 0)
    else:
        assert (gi["gram256"], gi["upd256_rows"], gi["gram_kmajor"]) == (0, 0, 1)
    w0, g = wl.arrays()
    st.step(1)
    h = st.host()
    if not _LONG_K_REF:
        z = np.zeros_like(w0)
        say("  float64 oracle on the host ...")
        _LONG_K_REF["ref"] = oracle_step(wl, wl.scale_layout, w0, g, z, z, 1)
    ref, dirs = _LONG_K_REF["ref"]
    worst = check_step(wl, wl.scale_layout, h, ref, dirs, w0)
    say(f"  worst NS rel-Frobenius {worst:.3e}")


@pytest.mark.parametrize("case", ["c2s", "c3s", "ragged"])
def test_ns_executed_counts_only_nonzero_units(case):
    """sshdp_ns_executed after a step: per group, the Muon units whose gradient
    (hence momentum, from zero) is not all zero, and the MFMA flops their tiles
    ran -- all of the plan's tile flops when no unit is zero (the d=2048 twin),
    that total scaled by the share of live units for the one-group MoE bank
    (2 of 8 experts with zero gradient), less than it for the ragged mix."""
    wl = _wl(case)
    say(f"ns_executed {wl.name}")
    st = DeviceState(wl)
    st.step(1)
    units, flops = st.plan.ns_executed(st.ws, st.ws_bytes, st.stream())
    groups = st.plan.groups()
    live = [0] * len(groups)
    zero = set(wl.zero_grad_units)
    for i, n in enumerate(wl.nodes):
        if n["is_unit"] and n["optimizer"] == "muon" and i not in zero:
            live[st.plan.node(i)[1]] += 1
    assert units == live, (units, live)
    total = st.plan.stats()["ns_tile_flops"]
    if case == "c2s":
        assert flops == pytest.approx(total, rel=1e-12)
    elif case == "c3s":
        (gi,) = groups
        assert units[0] == gi["n_units"] - 6
        assert flops == pytest.approx(total * units[0] / gi["n_units"], rel=1e-12)
    else:
        assert 0 < flops < total


def test_profiling_brackets_kernel_classes_without_changing_results():
    """sshdp_profile_enable/_read on the d=2048 twin: a profiled step gives the
    same bits as an unprofiled one; every class the step runs reports launches
    and time; the Newton-Schulz window (fork to join) is at least the sum of the
    launch stream's Gram, poly and update launches inside it; a read resets the
    counts, and a step with profiling off records nothing."""
    wl = workloads.config(2, small=True)
    say(f"profiling {wl.name}")
    a, b = DeviceState(wl), DeviceState(wl)
    a.plan.profile(True)
    a.step(1)
    b.step(1)
    ha, hb = a.host(), b.host()
    for k in ha:
        assert np.array_equal(ha[k], hb[k]), k
    prof = a.plan.profile_read()
    for c in ("momentum", "norm", "ns_gram", "ns_poly", "ns_update", "ns_phase", "requant", "adamw",
              "lane0_gram", "lane0_poly", "lane0_update", "lane0_update_last"):
        ms, n = prof[c]
        assert n > 0 and ms > 0.0, (c, prof[c])
    assert prof["ns_phase"][1] == 1 and prof["lane0_update_last"][1] == 1
    lane0 = sum(prof[c][0] for c in ("lane0_gram", "lane0_poly", "lane0_update", "lane0_update_last"))
    assert prof["ns_phase"][0] >= lane0 * (1 - 1e-3), prof
    assert all(n == 0 and ms == 0.0 for ms, n in a.plan.profile_read().values())
    a.plan.profile(False)
    a.step(2)
    a.host()
    assert all(n == 0 for _, n in a.plan.profile_read().values())


@pytest.mark.timeout(600)
def test_update_step_parity_longest_edge():
    """Muon units at the longest edge a plan accepts (c = 4194176), wide and
    tall, with r = 2 and 4: one 128-tile Gram per unit over K = 4194176 from
    X^T (its buffer resource at the 32-bit offset limit), B as a bf16 pair,
    32767 update tiles, G over 131068 blocks a row; against the float64 oracle."""
    wl = workloads.longest_edge_units()
    say(f"update_step {wl.name}")
    st = DeviceState(wl)
    gs = st.plan.groups()
    assert [(g["c_pad"], g["gram_kmajor"], g["split_b"]) for g in gs] == [(4194176, 1, 1)] * 2
    w0, g = wl.arrays()
    st.step(1)
    h = st.host()
    z = np.zeros_like(w0)
    say("  float64 oracle on the host ...")
    ref, dirs = oracle_step(wl, wl.scale_layout, w0, g, z, z, 1)
    worst = check_step(wl, wl.scale_layout, h, ref, dirs, w0)
    say(f"  worst NS rel-Frobenius {worst:.3e}")


@pytest.mark.parametrize("cid", [102, 103, 104])
def test_update_step_parity_random_shapes(cid):
    """Seeded random unit shapes, with 256-tiles wherever a 256-aligned block
    exists (the rest in 128-tile strips).  Every Muon unit's direction is within
    2e-2 of the float64 oracle, including a 32 x 507 unit whose singular values
    are tightly clustered (its group keeps B as a bf16 pair, as every group
    with r_pad = 128 does).  AdamW units as in every step test."""
    wl = workloads.random_units(cid)
    say(f"update_step {wl.name} seed {cid}: " + ", ".join(f"{n['rows']}x{n['cols']}" for n in wl.nodes if n["is_unit"]))
    st = DeviceState(wl, plan_kw=dict(ns_tiles="large"))
    for gi in st.plan.groups():
        assert gi["split_b"] == (gi["r_pad"] == 128), gi
    w0, g = wl.arrays()
    st.step(1)
    h = st.host()
    z = np.zeros_like(w0)
    ref, dirs = oracle_step(wl, wl.scale_layout, w0, g, z, z, 1)
    res = resolve_views(wl.nodes, wl.root_numel, wl.scale_layout)
    muon = [i for i, r in enumerate(res) if r["is_unit"] and r["optimizer"] == "muon"]
    for i in muon:
        idx = unit_indices(res[i])
        v_gpu = (w0[idx].astype(np.float64) - h["w"][idx].astype(np.float64)) / np.float32(MUON["lr"])
        e_ref = rel_fro(v_gpu, dirs[i])
        say(f"  unit {res[i]['rows']}x{res[i]['cols']}: vs fp64 {e_ref:.2e}")
        assert e_ref <= NS_TOL, (i, res[i]["rows"], res[i]["cols"], e_ref)
        assert np.max(np.abs(h["m"][idx] - ref["m"][idx])) <= 1e-6 * np.max(np.abs(ref["m"][idx]))
    others = [i for i, r in enumerate(res) if r["is_unit"] and i not in muon]
    check_step(wl, wl.scale_layout, h, ref, dirs, w0, units=others)


@pytest.mark.parametrize("case", ["c1", "c2s", "c3s"])
def test_update_step_parity_block32x32(case):
    """The whole step with one scale per 32x32 block: AdamW runs unfused, then
    G on the updated weights; codes and scales bit-exact."""
    wl = _wl(case)
    say(f"update_step {wl.name} (block32x32)")
    w0, g = wl.arrays()
    st = DeviceState(wl, layout="block32x32")
    assert st.stats["scale_bytes"] == (wl.root_numel + 1023) // 1024
    st.step(1)
    h = st.host()
    z = np.zeros_like(w0)
    ref, dirs = oracle_step(wl, "block32x32", w0, g, z, z, 1)
    check_step(wl, "block32x32", h, ref, dirs, w0)


def test_bf16_cast_regions_in_the_step_and_alone():
    """G as a bfloat16 cast: the O projection (Muon) and both norms (AdamW)
    of the small dense block are bf16 regions, the rest MXFP8.  After the
    step, the bf16 root equals the oracle's cast of the GPU-updated weights
    bit for bit (and nothing outside the bf16 regions is written); updates and
    MXFP8 bytes meet the usual gates; the cast entry alone matches too."""
    from test_oracle_bf16_cast import bf16_variant
    base = workloads.config(2, small=True)
    wl = dataclasses.replace(base, name=base.name + " (bf16 regions)", nodes=bf16_variant(base))
    say(f"bf16 cast {wl.name}")
    w0, g = wl.arrays()
    st = DeviceState(wl)
    out = torch.full((wl.root_numel,), 0x1234, dtype=torch.int16, device="cuda")
    bufs = sh.buffers(st.w, st.g, st.m, st.v, st.codes, st.scales, out)
    sh.update_step(st.plan, bufs, sh.muon_hp(**MUON), sh.adamw_hp(**ADAM), 1, st.ws, st.ws_bytes, st.stream())
    h = st.host()
    got = out.cpu().numpy().view(np.uint16)
    z = np.zeros_like(w0)
    ref, dirs = oracle_step(wl, wl.scale_layout, w0, g, z, z, 1)
    check_step(wl, wl.scale_layout, h, ref, dirs, w0)
    exp = np.full(wl.root_numel, 0x1234, np.uint16)
    res = resolve_views(wl.nodes, wl.root_numel, wl.scale_layout)
    oracle.cast_root_bf16(h["w"], res, exp)
    assert np.array_equal(got, exp)
    # the cast entry alone, on planted specials
    w = h["w"].copy()
    a = [r for r in res if r["cast"]][0]["abs"]
    w[a:a + 8] = [np.nan, np.inf, -np.inf, -0.0, 1e-41, 3.4e38, 1.00390625, -1.01171875]
    wt = torch.from_numpy(w).cuda()
    out.fill_(0x1234)
    sh.cast_bf16(st.plan, wt, out, st.stream())
    torch.cuda.synchronize()
    exp = np.full(wl.root_numel, 0x1234, np.uint16)
    oracle.cast_root_bf16(w, res, exp)
    got = out.cpu().numpy().view(np.uint16)
    nan = np.isnan(w)
    assert np.array_equal(got[~nan], exp[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)


def test_update_step_equals_separate_calls_bitwise():
    wl = workloads.config(4, small=True)
    for w_l in (wl, workloads.ragged_mix(), workloads.config(2, small=True)):
        say(f"fused vs separate {w_l.name}")
        a = DeviceState(w_l)
        b = DeviceState(w_l)
        a.step(1)
        sh.update_muon(b.plan, b.bufs(), sh.muon_hp(**MUON), b.ws, b.ws_bytes, b.stream())
        sh.update_adamw(b.plan, b.bufs(), sh.adamw_hp(**ADAM), 1, b.stream())
        sh.requant_mxfp8(b.plan, b.w, b.codes, b.scales, b.stream())
        ha, hb = a.host(), b.host()
        for k in ha:
            assert np.array_equal(ha[k].view(np.uint8), hb[k].view(np.uint8)), k


def test_determinism_and_resume():
    """Two runs are bitwise equal; N steps == k steps, state copied out and
    reloaded into fresh buffers, then N-k steps (the caller owns all state)."""
    wl = workloads.config(2, small=True)
    say(f"determinism/resume {wl.name}")
    a = DeviceState(wl)
    for t in (1, 2, 3, 4):
        a.step(t)
    ha = a.host()
    b = DeviceState(wl)
    for t in (1, 2):
        b.step(t)
    hb = b.host()
    c = DeviceState(wl, w=hb["w"], m=hb["m"], v=hb["v"])
    for t in (3, 4):
        c.step(t)
    hc = c.host()
    for k in ("w", "m", "v", "codes"):
        assert np.array_equal(ha[k].view(np.uint8), hc[k].view(np.uint8)), k
    d = DeviceState(wl)
    for t in (1, 2, 3, 4):
        d.step(t)
    hd = d.host()
    for k in ha:
        assert np.array_equal(ha[k].view(np.uint8), hd[k].view(np.uint8)), k


def test_update_step_captured_in_a_hip_graph():
    """The whole step (side streams forked and joined by events) captured into
    a HIP graph and replayed three times, with eager work and synchronisation
    between replays: after every replay the state equals the same number of
    eager calls bit for bit.  The step counter is baked into the capture, so
    both sides repeat step 1."""
    for wl in (workloads.config(2, small=True), workloads.ragged_mix()):
        say(f"graph capture {wl.name}")
        eager = DeviceState(wl)
        cap = DeviceState(wl)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=side):
            sh.update_step(cap.plan, cap.bufs(), sh.muon_hp(**MUON), sh.adamw_hp(**ADAM), 1, cap.ws, cap.ws_bytes,
                           side.cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(cap.w, eager.w)            # capturing ran nothing
        for k in range(3):
            graph.replay()
            eager.step(1)
            torch.cuda.synchronize()
            hc, he = cap.host(), eager.host()
            for key in he:
                assert np.array_equal(hc[key].view(np.uint8), he[key].view(np.uint8)), (wl.name, k, key)
            eager.g.mul_(1.0)                         # unrelated eager work between replays
        del graph


def test_multi_step_against_oracle():
    """Three steps with a fresh gradient each: momentum and AdamW state evolve
    on both sides."""
    wl = workloads.config(1)
    say(f"3 steps {wl.name}")
    w0, _ = wl.arrays()
    st = DeviceState(wl)
    w, m, v = w0.copy(), np.zeros_like(w0), np.zeros_like(w0)
    for t in (1, 2, 3):
        g = wl.gradient(t)
        st.g.copy_(torch.from_numpy(g))
        st.step(t)
        h = st.host()
        ref, dirs = oracle_step(wl, wl.scale_layout, w, g, m, v, t)
        # compare against the oracle started from the GPU's own previous state
        check_step(wl, wl.scale_layout, h, ref, dirs, w)
        w, m, v = h["w"].copy(), h["m"].copy(), h["v"].copy()


def test_options_nesterov_scale_mode_weight_decay():
    wl = workloads.ragged_mix()
    say(f"options {wl.name}")
    w0, g = wl.arrays()
    st = DeviceState(wl, plan_kw=dict(nesterov=True, scale_mode=1))
    muon = dict(lr=0.02, momentum=0.9, weight_decay=0.05)
    m0 = (np.random.default_rng(5).standard_normal(w0.size) * 1e-3).astype(np.float32)
    st.m.copy_(torch.from_numpy(m0))
    st.step(1, muon=muon)
    h = st.host()
    hp = oracle.OracleHyper(lr=0.02, momentum=0.9, weight_decay=0.05, nesterov=True, scale_mode=1)
    res = resolve_views(wl.nodes, wl.root_numel)
    for i, r in enumerate(res):
        if not (r["is_unit"] and r["optimizer"] == "muon"):
            continue
        idx = unit_indices(r)
        w_ref, m_ref, vdir = oracle.muon_update_unit(w0[idx], g[idx], m0[idx], hp)
        s = oracle.muon_scale(1, r["rows"], r["cols"])
        decay = np.float32(1 - np.float64(np.float32(0.02)) * np.float64(np.float32(0.05)))
        v_gpu = (w0[idx].astype(np.float64) * decay - h["w"][idx]) / (np.float32(0.02) * s)
        assert rel_fro(v_gpu, vdir) <= NS_TOL, i
        assert np.max(np.abs(h["m"][idx] - m_ref)) <= 1e-6 * np.max(np.abs(m_ref))


def test_argument_errors_on_device():
    wl = workloads.config(1)
    st = DeviceState(wl)
    with pytest.raises(sh.SshdpError) as e:
        sh.update_step(st.plan, st.bufs(), sh.muon_hp(), sh.adamw_hp(), 0, st.ws, st.ws_bytes, st.stream())
    assert e.value.name == "ARG"
    with pytest.raises(sh.SshdpError) as e:
        sh.update_muon(st.plan, st.bufs(), sh.muon_hp(), st.ws, st.ws_bytes - 256, st.stream())
    assert e.value.name == "WORKSPACE"
    b = sh.buffers(st.w.data_ptr() + 4, st.g, st.m, st.v, st.codes, st.scales)
    with pytest.raises(sh.SshdpError) as e:
        sh.update_step(st.plan, b, sh.muon_hp(), sh.adamw_hp(), 1, st.ws, st.ws_bytes, st.stream())
    assert e.value.name == "ALIGN"
    # nothing was launched: state unchanged
    h = st.host()
    w0, _ = wl.arrays()
    assert np.array_equal(h["w"], w0) and np.all(h["m"] == 0)


def test_requant_every_float_in_key_binades():
    """G on blocks whose amax is 448 (scale 2^0), so every other element is
    encoded as itself: every float32 of the binades [2^-12, 2^-6) (E4M3
    subnormals and their rounding), [1, 2) and [256, 448], both signs, against
    torch's float32 -> float8_e4m3fn conversion (a library routine)."""
    say("requant exhaustive binades")
    vals = []
    m = np.arange(1 << 23, dtype=np.uint32)
    for ex in (-12, -11, -10, -9, -8, -7, 0, 8):
        y = ((np.uint32(ex + 127) << 23) | m).view(np.float32)
        if ex == 8:
            y = y[y <= 448]
        vals += [y, -y]
    y = np.concatenate(vals)
    nblk = -(-y.size // 31)
    blocks = np.zeros((nblk, 32), np.float32)
    blocks[:, 0] = 448.0
    flat = blocks[:, 1:].reshape(-1)
    flat[:y.size] = y
    blocks[:, 1:] = flat.reshape(nblk, 31)
    root = blocks.reshape(-1)
    n = root.size
    nodes = [dict(parent=-1, offset=0, rows=nblk, cols=32, row_stride=32, is_unit=False, optimizer=None,
                  quantize=True)]
    plan = sh.Plan(nodes, n, layout="rowmajor")
    w = torch.from_numpy(root).cuda()
    codes = torch.zeros(n, dtype=torch.uint8, device="cuda")
    scales = torch.zeros(plan.stats()["scale_bytes"], dtype=torch.uint8, device="cuda")
    sh.requant_mxfp8(plan, w, codes, scales, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.all(scales == 127)
    ref = torch.from_numpy(root).to(torch.float8_e4m3fn).view(torch.uint8)
    assert torch.equal(codes.cpu(), ref)
