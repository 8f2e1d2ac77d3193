"""Build libpkv.so for gfx950 with hipcc (in-tree, next to this file).

    python -m paged_kv_cache_137_amd.build

Each HIP source compiles to an object in _build/ in parallel, and the objects
are linked into a shared library, which atomically replaces the old one.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpkv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are disabled throughout: hipcc would otherwise form
# v_pk_* fp32 ops from ordinary float code.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # The host pass does not know the packed-fp32 target feature and says so: harmless.
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops' is not a recognized" not in ln]
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    if lines and os.environ.get("PKV_BUILD_VERBOSE"):
        print("\n".join(lines), file=sys.stderr)


def build_library(jobs: int | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), 8)
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _run([HIPCC, *CFLAGS, "-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    tmp = LIB + f".tmp{os.getpid()}"
    # --no-undefined: a kernel whose host stub went missing fails the build, not the load.
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library())
