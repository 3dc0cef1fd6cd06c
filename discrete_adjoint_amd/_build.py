"""Build libdadj.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdadj.so")
SOURCES = ["erk_grad_f64_dopri5.hip", "erk_grad_f64_tsit5.hip", "erk_grad_f32_dopri5.hip",
           "erk_grad_f32_tsit5.hip", "sens.hip", "erk.hip", "ros2.hip", "l96.hip", "api.hip",
           "sort.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# -ffp-contract=off: only the explicit fma() calls fuse; the arithmetic order is
# the one written in the sources.  Packed fp32 instructions are disabled.
CFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-ffp-contract=off", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE,
          "-Wno-unused-parameter"]


def _obj_dir() -> str:
    d = os.path.join(HERE, "_build")
    os.makedirs(d, exist_ok=True)
    return d


def _compile(src: str, extra=(), tag: str = "") -> str:
    obj = os.path.join(_obj_dir(), os.path.splitext(src)[0] + tag + ".o")
    subprocess.run([HIPCC, *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj], check=True)
    return obj


def build(jobs: int = 8, out: str = LIB, extra=()) -> str:
    """Compile every source and link libdadj.so (or `out`, with extra compiler
    flags such as -D build options); returns its path."""
    tag = "" if out == LIB else "_" + os.path.basename(out).replace(".", "_")
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, tag), SOURCES))
    tmp = out + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs],
                   check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
