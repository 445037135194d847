"""Builds the HIP library libtk_topk.so in-tree for gfx950 with hipcc."""

from __future__ import annotations

import os
import shlex
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libtk_topk.so")
ARCH = os.environ.get("TK_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = [os.path.join(CSRC, "tk_kernels.hip"), os.path.join(CSRC, "tk_sample.hip"), os.path.join(CSRC, "tk_f32.hip"),
           os.path.join(CSRC, "tk_wide.hip"), os.path.join(CSRC, "tk_head.hip"),
           os.path.join(CSRC, "tk_api.cpp")]

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def command(output: str = LIBRARY) -> list[str]:
    info = f"{ARCH} {' '.join(FLAGS[1:5])}"
    return [HIPCC, *FLAGS, "-shared", f"-I{INCLUDE}", f"-I{CSRC}", f'-DTK_BUILD_INFO="{info}"',
            "-x", "hip", *SOURCES, "-o", output]


def build(output: str = LIBRARY, verbose: bool = False) -> str:
    """Compile the library (always recompiles); returns its path."""
    tmp = output + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"hipcc failed with exit code {proc.returncode}")
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
