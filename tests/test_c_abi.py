"""The C ABI from C (no GPU): include/moe.h compiles as strict C11 and as
C++, and a plain C program linked against libmoe.so makes the host-side
calls (status strings, workspace sizes, argument errors) through it."""
import os
import subprocess
from pathlib import Path

import pytest

from fine_grained_moe_router_amd import build as hipbuild

ROOT = Path(__file__).resolve().parents[1]
USE_ALL = r"""
#include <string.h>

#include "moe.h"
/* every entry point the header declares, through a pointer of the exact
 * type a C caller would write for it */
size_t (*p_ws)(const moe_config *, int) = moe_workspace_bytes;
int (*p_route)(const moe_config *, const void *, const void *, const float *, const float *,
               const uint32_t *, float *, int32_t *, float *, int32_t *, void *, void *, size_t,
               void *) = moe_route;
int (*p_fwd)(const moe_config *, const void *, const int32_t *, const float *, const void *,
             const void *, const void *, const void *, void *, void *, size_t, void *) = moe_forward;
int (*p_fwd_static)(const moe_config *, const void *, const int32_t *, const float *, const void *,
                    const void *, const void *, const void *, void *, void *) = moe_forward_static;
int (*p_stats)(const moe_config *, const int32_t *, const void *, float, float *, float *, float *,
               void *) = moe_balance_stats;
int (*p_seq)(const moe_config *, const float *, const float *, const int32_t *, const int32_t *,
             int32_t, float, float *, float *, float *, void *, size_t, void *) = moe_seq_balance_stats;
int (*p_dev)(const moe_config *, const float *, const float *, int32_t, float, float *, float *,
             float *, void *) = moe_device_balance_stats;
int (*p_bias)(const moe_config *, const int32_t *, int64_t, float, float *, void *) = moe_bias_update;
const char *(*p_status)(int) = moe_status_string;
int (*p_prof_on)(int) = moe_profile_enable;
int (*p_prof_get)(moe_stage_times *) = moe_profile_collect;
int main(void) {
    moe_config c;
    moe_stage_times st;
    memset(&c, 0, sizeof c);
    memset(&st, 0, sizeof st);
    return p_ws && p_route && p_fwd && p_fwd_static && p_stats && p_seq && p_dev && p_bias &&
                   p_status && p_prof_on && p_prof_get ? 0 : 1;
}
"""


@pytest.mark.parametrize("compiler,std", [("gcc", "-std=c11"), ("g++", "-std=c++17")])
def test_header_compiles_cleanly(tmp_path, compiler, std):
    ext = "c" if compiler == "gcc" else "cpp"
    src = tmp_path / f"use_all.{ext}"
    src.write_text(USE_ALL)
    flags = ["-Wall", "-Wextra", "-Werror", "-pedantic"]
    r = subprocess.run([compiler, std, *flags, f"-I{ROOT / 'include'}", "-c", str(src), "-o",
                        str(tmp_path / "use_all.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_program_makes_host_calls(tmp_path):
    exe = hipbuild.build_c_caller(out=tmp_path / "moe_c_caller")
    env = dict(os.environ, LD_LIBRARY_PATH=str(hipbuild.PKG))   # the in-tree libmoe.so
    r = subprocess.run([str(exe), "--host"], capture_output=True, text=True, timeout=60, env=env)
    assert r.returncode == 0 and "host checks ok" in r.stdout, (r.stdout, r.stderr)
