"""Build the gfx950 HIP library ``libh3conv.so`` in-tree with hipcc.

Every ``csrc/*.hip`` file is compiled to an object in parallel, then linked
into one shared library next to this file.  The build always runs when
called, also where a built library exists; loaders only load what exists.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libh3conv.so")
BUILD_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", CSRC, "-I", INCLUDE,
    "-Wall", "-Wshadow", "-Wno-unused-function", "-Wno-unused-variable",
]


# Host code instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
# (device code unchanged): `python build.py --sanitize` builds
# libh3conv_san.so beside the library, for host-only checks of the C-ABI shim
# (load it with clang's ASan runtime preloaded).
SAN_LIB = os.path.join(HERE, "libh3conv_san.so")
SAN_FLAGS = ["-g", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + (".san.o" if sanitize else ".o"))
    cmd = [HIPCC, *FLAGS, *(SAN_FLAGS if sanitize else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose: bool = True, sanitize: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda p: _compile(p, sanitize), srcs))
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    if sanitize:
        cmd[1:1] = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out, file=sys.stderr)
    return out


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
