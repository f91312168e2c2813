"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m fine_grained_moe_router_amd.build
Each .hip source compiles to an object in _build/ (in parallel), then the
objects link into fine_grained_moe_router_amd/libmoe.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = ROOT / "_build"
LIB = PKG / "libmoe.so"
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    f"-I{INCLUDE}", f"-I{CSRC}",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def sources():
    return sorted(CSRC.glob("*.hip"))


def _compile(src: Path, build_dir: Path = BUILD) -> Path:
    obj = build_dir / (src.stem + ".o")
    cmd = [HIPCC, *FLAGS, "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: Path = LIB) -> Path:
    """Compile every source and link `out`."""
    BUILD.mkdir(parents=True, exist_ok=True)
    srcs = sources()
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = out.with_name(out.name + ".tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


CALLER_SRC = ROOT / "tests" / "c_caller" / "moe_c_caller.c"
CALLER = PKG / "moe_c_caller"
ROCM = Path(os.environ.get("ROCM_PATH", "/opt/rocm"))


def build_c_caller(verbose: bool = False, out: Path = CALLER) -> Path:
    """Compile the C program that drives the library through include/moe.h
    (a plain C11 host program: gcc, the HIP runtime's C API, libmoe.so)."""
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-D__HIP_PLATFORM_AMD__", "-isystem", str(ROCM / "include"), f"-I{INCLUDE}",
           str(CALLER_SRC), f"-L{PKG}", "-lmoe", f"-L{ROCM / 'lib'}", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN", f"-Wl,-rpath,{ROCM / 'lib'}", "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on {CALLER_SRC.name}:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    build_c_caller(verbose=True)
    sys.exit(0)
