"""Binding of libgs_measure.so (include/gs_measure.h): the HBM copy and fp32 FMA
calibration kernels a benchmark times to quote this GPU's delivered rates
beside its published peaks.  Argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os

import torch

from .gs import GsError, _p, _stream

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgs_measure.so")
SYMBOLS = ["gs_stream_copy", "gs_fma_loop"]
FMA_LOOP_THREADS, FMA_LOOP_FLOPS_PER_ITER = 256, 128

_lib = None


def load_library(path=LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise GsError(f"{path} is not built: run `python -m differentiable_gaussian_splatting_dgs_amd.build`")
    lib = C.CDLL(path)
    lib.gs_stream_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]
    lib.gs_fma_loop.argtypes = [C.c_int32, C.c_int32, C.c_float, C.c_float, C.c_void_p, C.c_void_p]
    for name in SYMBOLS:
        getattr(lib, name).restype = C.c_int
    _lib = lib
    return lib


def gs_stream_copy(src, dst):
    """dst <- src (float32, numel a multiple of 4) with the non-temporal 16-byte copy kernel."""
    if src.numel() != dst.numel():
        raise GsError("gs_stream_copy: src and dst differ in size")
    rc = load_library().gs_stream_copy(_p(src, torch.float32, "src"), _p(dst, torch.float32, "dst"), src.numel(),
                                       _stream())
    if rc != 0:
        raise GsError(f"gs_stream_copy failed ({rc})")


def gs_fma_loop(blocks, iters, a, b, out):
    """The fp32 FMA loop kernel: blocks * 256 * iters * 128 flops; out holds blocks * 256 floats."""
    if out.numel() < blocks * FMA_LOOP_THREADS:
        raise GsError("gs_fma_loop: out holds fewer than blocks * 256 floats")
    rc = load_library().gs_fma_loop(blocks, iters, a, b, _p(out, torch.float32, "out"), _stream())
    if rc != 0:
        raise GsError(f"gs_fma_loop failed ({rc})")
