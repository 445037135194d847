"""Builds the HIP library libtk_topk.so in-tree for gfx950 with hipcc, and
beside it libtk_topk_stamps.so: the same sources with -DTK_STAGE_STAMPS, whose
scan kernels also record stage timestamps (a measurement build, loaded only
by bench.py --stage-timeline)."""

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
STAMP_LIBRARY = os.path.join(PKG, "libtk_topk_stamps.so")
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


def command(output: str = LIBRARY, stamps: bool = False) -> list[str]:
    info = f"{ARCH} {' '.join(FLAGS[1:5])}" + (" stage-stamps" if stamps else "")
    return [HIPCC, *FLAGS, "-shared", f"-I{INCLUDE}", f"-I{CSRC}", f'-DTK_BUILD_INFO="{info}"',
            *(["-DTK_STAGE_STAMPS"] if stamps else []), "-x", "hip", *SOURCES, "-o", output]


def build(output: str = LIBRARY, verbose: bool = False, stamps: bool | None = None) -> str:
    """Compile the library (always recompiles); returns its path.  Building
    the default library also builds the stamp library beside it, in parallel
    (stamps=False skips it)."""
    jobs = [(output, False)]
    if stamps or (stamps is None and output == LIBRARY):
        jobs.append((STAMP_LIBRARY, True))
    procs = []
    for out, st in jobs:
        cmd = command(out + ".tmp", st)
        if verbose:
            print(" ".join(shlex.quote(c) for c in cmd), flush=True)
        procs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = None
    for out, proc in procs:
        text, _ = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(text)
            failed = failed or f"hipcc failed with exit code {proc.returncode} ({os.path.basename(out)})"
    if failed:
        raise RuntimeError(failed)
    for out, _ in procs:
        os.replace(out + ".tmp", out)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
