"""Build libwq.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Each .hip translation unit is compiled to an object in parallel, then linked
into weight_only_bit_wq_amd/libwq.so.  Flags: -O3, C++17, gfx950 only,
packed-fp32 instructions disabled (-packed-fp32-ops), no fast-math.

The measurement kernels of csrc_ceilings/ (streaming read, MFMA-only loops;
not part of the library) go into libwq_ceilings.so, which only bench.py
loads.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libwq.so")
CEIL_SRC = os.path.join(HERE, "csrc_ceilings")
CEIL_LIB = os.path.join(HERE, "libwq_ceilings.so")
ARCH = "gfx950"
# -amdgpu-atomic-optimizer-strategy=None: the kernels' atomics are single-lane
# tickets and counters; the optimizer would rewrite each into a wave-wide
# scan that reads the result at once, waiting out the round trip that the
# split-K kernels issue early precisely to hide it.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-Wall"]


def _hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.isabs(c) and os.path.exists(c):
            return c
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def _link(objs: list, lib: str):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-o", tmp] + objs
    subprocess.check_call(cmd)
    os.replace(tmp, lib)


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    ceil_srcs = sorted(glob.glob(os.path.join(CEIL_SRC, "*.hip")))
    jobs = jobs or min(16, os.cpu_count() or 4)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs + ceil_srcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], CEIL_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
