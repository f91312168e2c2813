"""Register budget of the MFMA kernels, checked at compile time (no GPU).

The bf16 GEMMs run two waves per SIMD with 128 accumulator registers per
lane.  A VGPR spill inside their K loop reloads through memory, whose wait
also drains every operand load in flight; a change to the pipeline's code
shape once took the down GEMM from 221 registers and no spills to 934
spilled registers without any error.  Each kernel must keep its scratch at
zero bytes and its occupancy at two waves per SIMD."""
import re
import subprocess
from pathlib import Path

import pytest

from fine_grained_moe_router_amd import build as hipbuild

KERNELS = ("k_gate_up_bf16", "k_down_bf16", "k_router_bf16")


def resource_remarks(src: Path) -> dict:
    cmd = [hipbuild.HIPCC, *hipbuild.FLAGS, "--cuda-device-only", "-c", str(src), "-o", "/dev/null",
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z /\[\]]+?): (\d+) \[", line)
        if m and cur:
            out[cur][m.group(1).strip()] = int(m.group(2))
    return out


@pytest.mark.parametrize("src", ["expert_gemm.hip", "route.hip"])
def test_mfma_kernels_do_not_spill(src):
    res = resource_remarks(hipbuild.CSRC / src)
    found = {k: v for k, v in res.items() if any(n in k for n in KERNELS)}
    assert found, sorted(res)
    for name, r in found.items():
        assert r["VGPRs Spill"] == 0, (name, r)
        assert r["ScratchSize [bytes/lane]"] == 0, (name, r)
        assert r["Occupancy [waves/SIMD]"] >= 2, (name, r)
