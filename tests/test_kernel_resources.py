"""Register and scratch budget of the persistent drafter kernel, checked at compile time (no GPU).

Any private (scratch) segment in a kernel makes the dispatcher set up scratch for all 256 blocks at launch, which
delays the last blocks by about 12 us; the persistent kernel's blocks wait for each other, so every launch would pay
it. The check compiles k_team.hip for gfx950 with the compiler's resource report and requires no scratch in every
instance."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mtp_drafter_step_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_persistent_kernel_uses_no_scratch(tmp_path):
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip", "--cuda-device-only",
           "-c", os.path.join(CSRC, "k_team.hip"), "-o", str(tmp_path / "k_team.o"),
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    names = re.findall(r"remark: Function Name: (\S+)", r.stderr)
    scratch = [int(x) for x in re.findall(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
    assert len(names) == len(scratch) and names
    team = [(n, s) for n, s in zip(names, scratch) if "k_team" in n]
    assert len(team) == 10, team  # one instance per supported backbone width and kv head count (1, 2)
    assert all(s == 0 for _, s in team), team
