"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the host-sanitized library (block_sparse_attention_plan_amd.build with
sanitize=True, under _build/asan/), compiles tests/abi_host_check.cpp against
it with the same sanitizers, and runs it.  Every ABI call in that program
returns from host validation before any HIP call, so no GPU is needed.  A
memory error or undefined behaviour in the validation, plan geometry or error
reporting aborts the program.  Leak checking is off: the HIP runtime the
library links keeps allocations until exit.
"""

import os
import subprocess

import pytest

from block_sparse_attention_plan_amd import build as B

CLANG = "/opt/rocm/llvm/bin/clang++"
HERE = os.path.dirname(os.path.abspath(__file__))


def test_abi_host_checks_under_sanitizers(tmp_path):
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    if not os.path.exists(CLANG):
        pytest.skip("clang++ of the ROCm toolchain not found")
    lib = B.build(sanitize=True)
    exe = str(tmp_path / "abi_host_check")
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
    subprocess.run([CLANG, "-std=c++17", "-O1", "-g", *san, "-I", os.path.join(B.REPO_DIR, "include"),
                    os.path.join(HERE, "abi_host_check.cpp"), "-L", os.path.dirname(lib), "-lbsa",
                    f"-Wl,-rpath,{os.path.dirname(lib)}", "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1",
               LD_LIBRARY_PATH=os.pathsep.join(
                   p for p in ("/opt/rocm/lib", os.environ.get("LD_LIBRARY_PATH", "")) if p))
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "abi host checks ok" in r.stdout
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
