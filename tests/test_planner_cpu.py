"""The planners on the host: tests/planner_check.cpp compiles the library's
host code (csrc/wq_api.cpp) with the built kernel objects and replays, for
the dense 64-layer pass and 400 random passes, the walk the persistent
kernel makes over the plan, checking coverage and the blocked-split
invariants; and, for the single products and 3000 random shapes, the
split-tile kernel's partition (every tile step once, slot and arrival
bounds, parts per tile).  No GPU is used."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_weight_streaming_amd", "csrc")
BUILD = os.path.join(ROOT, "fp8_weight_streaming_amd", "_build")
KERNEL_OBJECTS = ["wq_kernels.hip.o", "wq_tile.hip.o", "wq_quant.hip.o", "wq_probe.hip.o"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def test_planner_walk_covers_every_unit_once(tmp_path):
    objs = [os.path.join(BUILD, o) for o in KERNEL_OBJECTS]
    missing = [o for o in objs if not os.path.exists(o)]
    assert not missing, "build the library first (python -m fp8_weight_streaming_amd.build): missing %s" % missing
    exe = str(tmp_path / "planner_check")
    cmd = [hipcc(), "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "c++", os.path.join(ROOT, "tests", "planner_check.cpp"),
           "-x", "none", *objs, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    tail = r.stdout.strip().splitlines()[-1] if r.stdout.strip() else ""
    assert r.returncode == 0 and tail.startswith("all ok"), r.stdout[-4000:] + r.stderr[-2000:]
    dense = [l for l in r.stdout.splitlines() if l.split()[0] == "dense64" and l.split()[1] != "plain" and "cus=256" in l]
    assert len(dense) == 3 and all("blocked mats=64" in l and "tasks=0" in l for l in dense), dense
    split = [l for l in r.stdout.splitlines() if l.startswith("tile split:")]
    assert split and "17408x5120: ok=1" in split[0] and "5120x17408: ok=1" in split[0], split
