"""sshdp_update_step_noalloc (the step with the library's built-in scratch as
its workspace) against sshdp_update_step with a caller workspace, through the
C ABI: the same plan and seeded roots give bit-identical w, m, v, codes and
scales, on calls in a row -- a MoE bank (zero-gradient experts, an AdamW
router), then a smaller attention block, then the MoE bank again from fresh
roots (the scratch keeps the previous call's contents, which nothing may
read).  A plan whose workspace exceeds the scratch is refused before anything
runs."""

import numpy as np
import pytest

import mxfp8_weight_repack_amd as sh
import workloads
from gpu_util import DeviceState, say, MUON, ADAM

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sh.lib()


def _pair(wl, steps):
    """(reference state after `steps` update_step calls, state after as many
    noalloc calls), each from fresh roots."""
    ref = DeviceState(wl)
    got = DeviceState(wl)
    assert ref.stats["workspace_bytes"] <= sh.NOALLOC_SCRATCH_BYTES
    for t in range(1, steps + 1):
        ref.step(t)
        sh.update_step_noalloc(got.plan, got.bufs(), sh.muon_hp(**MUON), sh.adamw_hp(**ADAM), t, got.stream())
    return ref.host(), got.host()


def test_noalloc_matches_update_step_on_calls_in_a_row():
    cases = [(workloads.config(3, small=True), 2), (workloads.config(1), 1), (workloads.config(3, small=True), 1)]
    sizes = []
    for wl, steps in cases:
        say(f"noalloc {wl.name}: {steps} step(s)")
        h_ref, h_got = _pair(wl, steps)
        for k in h_ref:
            assert np.array_equal(h_ref[k].view(np.uint8), h_got[k].view(np.uint8)), (wl.name, k)
        sizes.append(wl.root_numel)
    assert sizes[1] < sizes[0]                      # the second call's input is the smaller


def test_noalloc_refuses_plans_beyond_the_scratch():
    wl = workloads.config(2)                        # the d=2048 block needs ~300 MiB of workspace
    plan = sh.Plan(wl.nodes, wl.root_numel, layout=wl.scale_layout)
    assert plan.stats()["workspace_bytes"] > sh.NOALLOC_SCRATCH_BYTES
    with pytest.raises(sh.SshdpError) as e:
        sh.update_step_noalloc(plan, sh.buffers(), sh.muon_hp(**MUON), sh.adamw_hp(**ADAM), 1,
                               torch.cuda.current_stream().cuda_stream)
    assert e.value.name == "SCRATCH"
    torch.cuda.synchronize()
