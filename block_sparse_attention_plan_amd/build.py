"""Build libbsa.so (gfx950) in-tree with hipcc.

    python -m block_sparse_attention_plan_amd.build [--jobs N] [--sanitize]

Each csrc/*.hip file is compiled to an object under _build/ and the objects
are linked into block_sparse_attention_plan_amd/libbsa.so.  Every call
rebuilds from scratch, so the library always matches the sources.  With
--sanitize the host code is built with AddressSanitizer and
UndefinedBehaviorSanitizer into _build/asan/libbsa.so instead, for the host
ABI checks (tests/abi_host_check.cpp).
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(REPO_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libbsa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(REPO_DIR, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def sources() -> list:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd: list) -> None:
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the C ABI
# layer (argument validation, plan geometry, error reporting).  Each
# -fsanitize= applies to the host compilation only: device code is built as
# in the release library.  The shared library leaves the sanitizer runtime
# to the executable that loads it.
SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
]
SANITIZED_LIB = os.path.join(BUILD_DIR, "asan", "libbsa.so")


def build(jobs: int = 8, verbose: bool = False, sanitize: bool = False) -> str:
    """Build the release library (in the package), or with sanitize=True the
    host-sanitized one under _build/asan/ (for the host ABI checks)."""
    cc = hipcc()
    out_dir = os.path.dirname(SANITIZED_LIB) if sanitize else BUILD_DIR
    lib_path = SANITIZED_LIB if sanitize else LIB_PATH
    extra = SANITIZE_FLAGS if sanitize else []
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(out_dir, os.path.basename(s)[:-4] + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        cmd = [cc, *HIPCC_FLAGS, *extra, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        _run(cmd)

    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    tmp = lib_path + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, lib_path)
    return lib_path


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--sanitize", action="store_true",
                    help="host-side ASan/UBSan build under _build/asan/ (not the package library)")
    args = ap.parse_args(argv)
    path = build(args.jobs, args.verbose, sanitize=args.sanitize)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
