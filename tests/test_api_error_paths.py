"""Error paths of the launching entry points, on the host: plan.cpp and api.hip
built with g++ against a stand-in of the HIP runtime calls they make and of the
kernel launchers (tests/host_api_check.cpp), the n-th launch made to fail for
every n.  Each failing step returns SSHDP_ERR_HIP and leaves every side stream
it forked joined back into the caller's stream (SS-HSDP Appendix A: stages are
ordered within an update group; an error must not leave work unordered after
the caller's later work).  No GPU is used."""

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


@pytest.mark.parametrize("cid", [2, 3])
def test_failed_launch_leaves_side_streams_joined(tmp_path, cid):
    if not (os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")) and shutil.which("g++")):
        pytest.skip("ROCm headers or g++ missing")
    exe = tmp_path / "apichk"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", ROCM + "/include",
           os.path.join(CSRC, "plan.cpp"), "-x", "c++", os.path.join(CSRC, "api.hip"), "-x", "none",
           os.path.join(ROOT, "tests", "host_api_check.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    wl = workloads.config(cid)
    data = tmp_path / "tree.bin"
    with open(data, "wb") as f:
        f.write(struct.pack("<iqiI", len(wl.nodes), wl.root_numel, LAYOUT[wl.scale_layout], 0))
        f.write(bytes(node_array(wl.nodes)))
    r = subprocess.run([str(exe), str(data)], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-3000:])
    words = r.stdout.split()
    assert words[0] == "ok", r.stdout
    checked, launches, side = int(words[2]), int(words[4]), int(words[6])
    assert launches > 10 and checked == 2 * (launches + 1)
    assert side == (1 if cid == 2 else 0)        # the dense block forks a side stream; the MoE bank is one group
