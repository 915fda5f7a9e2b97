"""Build libmoe.so and libmoe_measure.so (HIP, gfx950) in-tree with hipcc.

    python -m moe_layer_forward_amd.build

Every .hip file directly under csrc/ is compiled to an object in parallel and
linked into moe_layer_forward_amd/libmoe.so (the layer); the files under
csrc/measure/ make moe_layer_forward_amd/libmoe_measure.so (measurement
helpers, not part of the layer).  Packed-fp32 instruction selection is
switched off for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
MEASURE_LIB = os.path.join(PKG, "libmoe_measure.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str) -> str:
    rel = os.path.relpath(src, CSRC).replace(os.sep, "_")
    obj = os.path.join(BUILD, rel + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {out} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int | None = None) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    msrcs = sorted(glob.glob(os.path.join(CSRC, "measure", "*.hip")))
    jobs = jobs or min(8, os.cpu_count() or 4, len(srcs) + len(msrcs))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs + msrcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], MEASURE_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
