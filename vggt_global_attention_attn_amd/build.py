"""Build libvggt_attn.so in-tree with hipcc for gfx950.

    python -m vggt_global_attention_attn_amd.build

Every HIP source is compiled with packed-fp32 VALU instructions disabled; the host-only plan
and C ABI sources are plain C++17.  The result lands next to this file, where the Python
binding loads it."""
from __future__ import annotations

import os
import shlex
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libvggt_attn.so")

HIP_SOURCES = ["pack.hip", "attn.hip", "scratch.hip"]
CXX_SOURCES = ["plan.cpp", "capi.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def commands(out: str = LIB, extra: list[str] | None = None) -> list[list[str]]:
    extra = extra or []
    objdir = os.path.join(ROOT, "_build", os.path.basename(out))
    os.makedirs(objdir, exist_ok=True)
    cmds, objs = [], []
    common = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]
    for src in HIP_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmds.append([hipcc(), "-x", "hip", f"--offload-arch={ARCH}", *common,
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-honor-nans",
                     "-c", os.path.join(CSRC, src), "-o", obj, *extra])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmds.append([hipcc(), *common, "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, src), "-o", obj, *extra])
        objs.append(obj)
    cmds.append([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out + ".tmp", *objs])
    return cmds


def build(verbose: bool = False, out: str = LIB, extra: list[str] | None = None) -> str:
    """Compile every source and link the shared library; returns its path.  `extra` adds
    compiler flags (e.g. -D tile-shape macros of attn.hip)."""
    for cmd in commands(out, extra):
        if verbose:
            print(" ".join(shlex.quote(c) for c in cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        noise = "'-packed-fp32-ops' is not a recognized feature"
        msg = "\n".join(line for line in (res.stderr + res.stdout).splitlines() if noise not in line)
        if res.returncode != 0:
            raise RuntimeError(f"build step failed ({res.returncode}):\n{' '.join(cmd)}\n{msg}")
        if verbose and msg.strip():
            print(msg, flush=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
    print(LIB)
