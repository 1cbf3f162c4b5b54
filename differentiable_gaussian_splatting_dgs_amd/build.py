"""Build libgs.so (the HIP rasterizer library) and libgs_measure.so (the two
calibration kernels a benchmark times beside it) for gfx950 with hipcc.

Usage: python -m differentiable_gaussian_splatting_dgs_amd.build [--force]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgs.so")
MEASURE_LIB = os.path.join(PKG, "libgs_measure.so")
OBJDIR = os.path.join(PKG, "_build")
SOURCES = ["api.hip", "preprocess.hip", "binning.hip", "render.hip", "preprocess_bwd.hip", "train.hip",
           "densify.hip", "debug.hip"]
MEASURE_SOURCES = ["calibrate.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # never emit packed FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(force=True, verbose=False):
    """Compile every HIP source and link both libraries.  Always rebuilds when force."""
    deps = [os.path.join(CSRC, s) for s in SOURCES + MEASURE_SOURCES] + [
        os.path.join(CSRC, "gs_internal.h"), os.path.join(INCLUDE, "gs.h"), os.path.join(INCLUDE, "gs_measure.h")]
    if (not force and all(os.path.exists(x) for x in (LIB, MEASURE_LIB)) and
            min(os.path.getmtime(LIB), os.path.getmtime(MEASURE_LIB)) >= max(os.path.getmtime(d) for d in deps)):
        return LIB
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + MEASURE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in MEASURE_SOURCES], MEASURE_LIB)
    if verbose:
        print("built", LIB, "and", MEASURE_LIB)
    return LIB


if __name__ == "__main__":
    build(force="--force" in sys.argv or True, verbose=True)
