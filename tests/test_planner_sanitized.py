"""The planner (csrc/plan.cpp) built for the host with AddressSanitizer and
UndefinedBehaviorSanitizer (g++), run over every workload, the ragged and
random trees under each tile policy, and trees that each planning rule must
reject: no sanitizer report, and the same plans (stats, groups) as the
library's own host-only plans.  Skipped where ROCm's headers or runtime
library are missing."""

import os
import shutil
import struct
import subprocess

import pytest

import mxfp8_weight_repack_amd as sh
from mxfp8_weight_repack_amd._lib import LAYOUT, NS_GRAM, NS_TILES, node_array
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp8_weight_repack_amd", "csrc")
ROCM = "/opt/rocm"


def _trees():
    out = []
    for cid in (1, 2, 3, 4, 5):
        for small in (False, True):
            if cid == 1 and small:
                continue
            wl = workloads.config(cid, small=small)
            out.append((wl.nodes, wl.root_numel, wl.scale_layout, "auto"))
    for wl in (workloads.ragged_mix(), workloads.mixed_tiles(), workloads.random_units(102),
               workloads.random_units(105, n=12)):
        for pol in ("auto", "small", "large"):
            out.append((wl.nodes, wl.root_numel, "rowmajor", pol))
    wl = workloads.config(2, small=True)
    out.append((wl.nodes, wl.root_numel, "block32x32", "auto"))
    for pol in ("auto+nt", "small+nt"):                              # every Gram reading X row-major
        out.append((wl.nodes, wl.root_numel, "tile32x4", pol))
    for kind in ("g_only", "muon_only", "adamw_g"):
        wl = workloads.degenerate(kind)
        out.append((wl.nodes, wl.root_numel, wl.scale_layout, "auto"))
    big = dict(parent=-1, offset=0, rows=1024, cols=1048704, row_stride=1048704, is_unit=True, optimizer="muon",
               quantize=False)                                       # X^T past 2^31 bytes: row-major Gram
    out.append(([big], 1024 * 1048704, "rowmajor", "auto"))
    # rejected trees: overlap, bad parent, out of bounds, misaligned MXFP8 region, bad Muon unit
    base = dict(parent=-1, offset=0, rows=64, cols=64, row_stride=64, is_unit=True, optimizer="muon",
                quantize=False)
    bad = [
        [base, dict(base, offset=32)],                                   # overlapping units
        [dict(base, parent=1)],                                          # parent not earlier
        [dict(base, offset=4096)],                                       # beyond the root
        [dict(base, optimizer="adamw", quantize=True, offset=16, rows=1, cols=64)],   # MXFP8 start % 32
        [dict(base, rows=1, cols=64)],                                   # 1-row Muon unit
    ]
    for nodes in bad:
        out.append((nodes, 4096, "rowmajor", "auto"))
    long = dict(base, rows=128, cols=4194304, row_stride=4194304)       # Muon edge beyond 4194176
    out.append(([long], 128 * 4194304, "rowmajor", "auto"))
    return out


def _write(path, trees):
    with open(path, "wb") as f:
        for nodes, root, layout, pol in trees:
            tiles, _, gram = pol.partition("+")
            f.write(struct.pack("<iqiI", len(nodes), root, LAYOUT[layout], NS_TILES[tiles] | NS_GRAM[gram or "auto"]))
            f.write(bytes(node_array(nodes)))


def _expected(nodes, root, layout, pol):
    tiles, _, gram = pol.partition("+")
    try:
        p = sh.Plan(nodes, root, layout=layout, host_only=True, ns_tiles=tiles, ns_gram=gram or "auto")
    except sh.SshdpError as e:
        return ("status", e.code)
    st = p.stats()
    groups = [(g["r"], g["c"], g["r_pad"], g["c_pad"], g["n_units"], g["gram256"], g["upd256_rows"],
               g["upd256_cols"], g["gram_kmajor"]) for g in p.groups()]
    return ("ok", st["workspace_bytes"], st["scale_bytes"], st["n_groups"], st["ns_tile_flops"], groups)


def _parse(line):
    parts = line.split()
    if parts[1] == "status":
        return ("status", int(parts[2]))
    ws, scale, ng, fl = int(parts[3]), int(parts[5]), int(parts[7]), float(parts[9])
    body = line.split("tileflops")[1].split("[")[1:]
    groups = [tuple(int(x) for x in b.strip().rstrip("]").split()) for b in body]
    return ("ok", ws, scale, ng, fl, groups)


def test_planner_under_address_and_ub_sanitizers(tmp_path):
    if not (os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h"))
            and os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")) and shutil.which("g++")):
        pytest.skip("ROCm headers / runtime or g++ missing")
    exe = tmp_path / "planchk"
    cmd = ["g++", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-g", "-O1",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", ROCM + "/include",
           os.path.join(CSRC, "plan.cpp"), os.path.join(ROOT, "tests", "host_planner_check.cpp"),
           "-L", ROCM + "/lib", "-lamdhip64", "-Wl,-rpath," + ROCM + "/lib", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    trees = _trees()
    data = tmp_path / "trees.bin"
    _write(data, trees)
    supp = tmp_path / "lsan.supp"
    supp.write_text("leak:libamdhip64\nleak:libhsa-runtime64\nleak:librocprofiler-register\n")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               LSAN_OPTIONS=f"suppressions={supp}", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe), str(data)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    lines = r.stdout.strip().splitlines()
    assert len(lines) == len(trees)
    for line, t in zip(lines, trees):
        assert _parse(line) == _expected(*t), line
