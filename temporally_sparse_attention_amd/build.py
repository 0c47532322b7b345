"""Build step: compile the HIP kernels and the C ABI into liblite_attn.so (in-tree, gfx950)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "liblite_attn.so"
SOURCES = ["lite_attn_kernels.hip", "lite_attn_aux.hip", "lite_attn_api.hip"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_command(out_path: str, extra=()) -> list:
    return [
        hipcc(), "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
        # keep the compiler from forming packed fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I" + INCLUDE, "-I" + CSRC,
        *[os.path.join(CSRC, s) for s in SOURCES],
        *extra,
        "-o", out_path,
    ]


def build(verbose: bool = False, extra=()) -> str:
    out = os.path.join(PKG, LIB_NAME)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = compile_command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=PKG, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("building %s failed" % LIB_NAME)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
