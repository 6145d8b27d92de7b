"""The work tables the planner builds, checked on the host.  For every workload
and tile policy: each unit's Newton-Schulz Gram and polynomial tiles cover the
upper triangle of its r_pad x r_pad product exactly once in 128 x 128 cells
(the lower triangle is the mirror the kernels store), its update tiles cover the
r_pad x c_pad product exactly once, and every tile of a group is on that group's
stream; f0 tiles cover each Muon unit once, within its stream's range; every
AdamW element is in exactly one segment and is updated exactly once by a step
(unfused segments plus the fused requant chunks); requant chunks cover every
quantised region exactly once.  A missing or doubled item would leave part of
the state unwritten or updated twice.  Built with g++ from plan.cpp and api.hip against the stand-in
runtime of tests/host_api_check.cpp; no GPU is used."""

import os
import shutil
import struct
import subprocess

import pytest

from mxfp8_weight_repack_amd._lib import LAYOUT, node_array
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp8_weight_repack_amd", "csrc")
ROCM = "/opt/rocm"


def test_work_tables_cover_every_cell_once(tmp_path):
    if not (os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")) and shutil.which("g++")):
        pytest.skip("ROCm headers or g++ missing")
    exe = tmp_path / "tilechk"
    cmd = ["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", ROCM + "/include", os.path.join(CSRC, "plan.cpp"), "-x", "c++", os.path.join(CSRC, "api.hip"),
           "-x", "none", os.path.join(ROOT, "tests", "host_api_check.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    wls = [workloads.config(c, small=s) for c in (1, 2, 3, 5) for s in (False, True)]
    wls += [workloads.config(4, small=True)] + [workloads.degenerate(k) for k in ("g_only", "muon_only", "adamw_g")]
    wls += [workloads.ragged_mix(), workloads.mixed_tiles(), workloads.long_k_units()]
    wls += [workloads.random_units(cid) for cid in (102, 103, 104)]
    data = tmp_path / "trees.bin"
    with open(data, "wb") as f:
        for wl in wls:
            f.write(struct.pack("<iqiI", len(wl.nodes), wl.root_numel, LAYOUT[wl.scale_layout], 0))
            f.write(bytes(node_array(wl.nodes)))
    r = subprocess.run([str(exe), str(data), "tiles"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-2000:])
    words = r.stdout.split()
    assert words[0] == "ok" and int(words[2]) == len(wls), r.stdout
    assert int(words[4]) >= 4 * len(wls), r.stdout      # every policy plans; TILES_LARGE may refuse none
    # the check itself: a dropped and a doubled tile are both caught
    for plant, rc, words in (("drop", 9, "covered 0 times"), ("dup", 9, "covered 2 times"),
                             ("seg", 12, "updated 2 times")):
        r = subprocess.run([str(exe), str(data), "tiles"], capture_output=True, text=True, timeout=600,
                           env=dict(os.environ, TILECHK_PLANT=plant))
        assert r.returncode == rc and words in r.stdout, (plant, r.returncode, r.stdout[-500:])
