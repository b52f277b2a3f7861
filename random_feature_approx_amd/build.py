"""Build the gfx950 FAVOR+ library (libfavor.so) in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only, in parallel, and linked
into one shared library next to this file.  Packed-fp32 VALU instructions are
disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfavor.so")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the FAVOR+ library needs the ROCm toolchain")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc(), *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libfavor.so.  Returns its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(_compile, srcs, objs))
    tmp = LIB + ".tmp"
    # --no-undefined: a kernel whose launch stub the host pass did not emit
    # fails here rather than at load time
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_host_sanitized(outdir: str) -> str:
    """Host-only build of every source, instrumented with AddressSanitizer and
    UndefinedBehaviorSanitizer, and the argument-checking driver
    tests/abi_check.c linked against it.  The device code is compiled as
    usual (the host objects register it) but never runs: the driver only
    makes calls that are rejected before anything is launched.  Returns the
    path of the driver executable (outdir/abi_check)."""
    os.makedirs(outdir, exist_ok=True)
    # each sanitizer flag goes to the host compilation only
    san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", f]
    srcs = sources()
    objs = [os.path.join(outdir, os.path.basename(s)[:-4] + ".o") for s in srcs]

    def compile_one(src, obj):
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++20", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"host build failed for {os.path.basename(src)}:\n{r.stderr}")

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(compile_one, srcs, objs))
    lib = os.path.join(outdir, "libfavor_host_san.so")
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *san, *objs, "-o", lib],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host link failed:\n{r.stderr}")
    root = os.path.dirname(HERE)
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    exe = os.path.join(outdir, "abi_check")
    cmd = [clang, "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(root, "include"), os.path.join(root, "tests", "abi_check.c"),
           lib, f"-Wl,-rpath,{outdir}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"driver build failed:\n{r.stderr}")
    return exe


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
