"""The host side of the C ABI and the CPU oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

tests/hoststub/ builds tk_api.cpp with g++ over a stand-in device layer (one
fake device; allocations in host memory; launches that only check their
scratch ranges; any HIP call can be made to fail) and drives it:
every fallible HIP call of every launching entry point fails in turn, from a
fresh and a warm stream, and the call must report TK_ERR_DEVICE (or go on
where the call is optional), free what it allocated, and leave later calls
working; the allocation-free entry point must never allocate; the oracle is
checked against the rank definition on random small rows.  The same driver
runs once plainly and once with -fsanitize=address,undefined."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STUB = os.path.join(ROOT, "tests", "hoststub")
SANITIZE = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]


def _build(out_dir, extra):
    flags = ["-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{ROOT}/include",
             f"-I{ROOT}/wide_row_bf16_amd/csrc", f"-I{STUB}", *extra]
    objs = []
    for cc, std, src in (("gcc", "-std=c11", f"{ROOT}/oracle/tk_oracle.c"),
                         ("g++", "-std=c++17", f"{ROOT}/wide_row_bf16_amd/csrc/tk_api.cpp"),
                         ("g++", "-std=c++17", f"{STUB}/hip_stub.cpp"),
                         ("g++", "-std=c++17", f"{STUB}/host_driver.cpp")):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        subprocess.run([cc, std, *flags, "-c", src, "-o", obj], check=True)
        objs.append(obj)
    exe = os.path.join(out_dir, "host_driver")
    subprocess.run(["g++", *extra, *objs, "-o", exe, "-lpthread", "-lm"], check=True)
    return exe


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"),
                    reason="needs g++ and the HIP headers")
@pytest.mark.parametrize("mode", ["plain", "asan+ubsan"])
def test_host_driver(mode, tmp_path):
    exe = _build(str(tmp_path), SANITIZE if mode != "plain" else [])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    proc = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert proc.returncode == 0, proc.stdout[-3000:] + proc.stderr[-5000:]
    assert "host driver: all checks passed" in proc.stdout
    assert "swept noalloc" in proc.stdout and "oracle:" in proc.stdout
