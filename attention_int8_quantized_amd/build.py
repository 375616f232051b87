"""Build the attnq8 shared library for gfx950 with hipcc (in-tree)."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libattnq8.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["attnq8.hip"]
DEPENDS = ["attnq8.hip", "append_kernel.h", "attend_kernel.h", "device_utils.h", "head_kernel.h", "own_kernel.h", "stream_kernel.h"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_command(out: str = LIB_PATH):
    return [
        hipcc(),
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-shared",
        "-fPIC",
        "-Wall",
        # packed fp32 instructions are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile libattnq8.so next to this file; returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    if verbose and res.stderr.strip():
        # host-pass notes about the packed-fp32 feature are expected
        noise = "is not a recognized feature for this target"
        lines = [l for l in res.stderr.splitlines() if noise not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
