"""CPU-side checks of the C ABI: libgs.so loads, exports every function that
include/gs.h declares, the binding wraps each under the same name, and the
host-only calls (no device work) behave."""
import ctypes as C
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gs.h")
MEASURE_HEADER = os.path.join(ROOT, "include", "gs_measure.h")


def header_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gs_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_path():
    names = header_functions()
    for required in ("gs_preprocess", "gs_bin_sort", "gs_render_fwd", "gs_render_bwd", "gs_preprocess_bwd",
                     "gs_image_loss", "gs_densify_accum", "gs_adam_step"):
        assert required in names


def test_library_exports_every_header_symbol():
    from differentiable_gaussian_splatting_dgs_amd import gs
    lib = gs.load_library()
    for name in header_functions():
        assert hasattr(lib, name), name
    assert sorted(gs.SYMBOLS) == header_functions()
    for name in header_functions():
        assert callable(getattr(gs, name, None)) or name in ("gs_error_string", "gs_version"), name


def test_measure_library_exports_its_header():
    """The calibration kernels live in their own library, not in the rasterizer's."""
    from differentiable_gaussian_splatting_dgs_amd import gs, measure
    mlib = measure.load_library()
    names = header_functions(MEASURE_HEADER)
    assert names == sorted(measure.SYMBOLS) == ["gs_fma_loop", "gs_stream_copy"]
    for name in names:
        assert hasattr(mlib, name) and callable(getattr(measure, name)), name
        assert name not in header_functions()
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", gs.LIB_PATH], capture_output=True, text=True).stdout
    assert "gs_stream_copy" not in out and "gs_fma_loop" not in out


def test_bin_status_word():
    """The binding reads gs_bin_sort's status word: bit 1 (failed sort) raises, bit 0
    (overflow) asks for a retry, 0 means the lists are valid."""
    from differentiable_gaussian_splatting_dgs_amd import gs
    assert gs.check_bin_status(0) is False
    assert gs.check_bin_status(1) is True
    for word in (2, 3):
        with pytest.raises(gs.GsError, match="gave up"):
            gs.check_bin_status(word)
    with pytest.raises(gs.GsError, match="unknown"):
        gs.check_bin_status(4)
    lib = gs.load_library()
    prev = gs.gs_debug_sort_wait_limit(-1)
    assert prev == 1 << 22
    assert gs.gs_debug_sort_wait_limit(0) == prev
    assert gs.gs_debug_sort_wait_limit(prev) == 0
    assert lib.gs_debug_sort_wait_limit(-1) == prev


def test_host_only_calls():
    from differentiable_gaussian_splatting_dgs_amd import gs, scenes
    lib = gs.load_library()
    assert lib.gs_version() == 1
    assert lib.gs_error_string(0) == b"ok"
    assert lib.gs_error_string(-5) == b"size exceeds kernel indexing limits"
    cam = scenes.Camera.identity(1920, 1080, 1500.0)
    assert gs.gs_tile_grid(cam) == (120, 68)
    b1 = gs.gs_bin_workspace_size(1000, cam, 10000)
    b2 = gs.gs_bin_workspace_size(1000, cam, 20000)
    assert b2 > b1 > 0 and b1 % 256 == 0
    with pytest.raises(gs.GsError):
        gs.gs_bin_workspace_size(-1, cam, 10)
    with pytest.raises(gs.GsError):
        gs.gs_bin_workspace_size(10, cam, 1 << 31)


def test_product_path_does_not_import_oracle():
    """The binding and the HIP sources never reference the oracle."""
    pkg = os.path.join(ROOT, "differentiable_gaussian_splatting_dgs_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src.lower() or f == "scenes.py" and "oracle" in src, f


def test_scene_generators_deterministic():
    from differentiable_gaussian_splatting_dgs_amd import scenes
    a, b = scenes.tiny(), scenes.tiny()
    for k in ("means", "log_scales", "quats", "opacity_logits", "sh"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
        assert getattr(a, k).dtype == np.float32
    assert a.means.shape == (256, 3) and a.sh.shape == (256, 1, 3) and a.dL_dimage.shape == (3, 64, 64)
    assert np.allclose(np.linalg.norm(a.quats, axis=1), 1, atol=1e-6)
    s = scenes.ball100k()
    assert s.sh.shape == (100_000, 16, 3) and s.loss == "l2" and s.target.shape == (3, 800, 800)
    r = np.linalg.norm(s.means - np.array([0, 0, 4], np.float32), axis=1)
    assert r.max() <= 1.5 + 1e-5


def test_views_and_densify_host_checks():
    """Host-side sizes and argument checks of the batched-view and densify calls (no device work)."""
    from differentiable_gaussian_splatting_dgs_amd import gs, scenes
    lib = gs.load_library()
    cam = scenes.Camera.identity(1920, 1080, 1500.0)
    cams = scenes.orbit_cameras(cam, 4, (0.0, 0.0, 6.0))
    # a batch bins views x n records: its workspace is the single-view one for that many Gaussians
    assert gs.gs_bin_workspace_size_views(1000, cams, 50000) == gs.gs_bin_workspace_size(4000, cam, 50000)
    with pytest.raises(gs.GsError):
        gs.camera_array([])
    with pytest.raises(gs.GsError):
        gs.camera_array([cam] * 9)
    b = C.c_size_t()
    arr, v = gs.camera_array([cam, scenes.Camera.identity(1280, 720, 1000.0)])
    assert lib.gs_bin_workspace_size_views(100, arr, v, 1000, C.byref(b)) == -1   # views of different sizes
    arr9 = (gs.GsCamera * 9)(*([gs.camera_struct(cam)] * 9))
    assert lib.gs_bin_workspace_size_views(100, arr9, 9, 1000, C.byref(b)) == -1   # more than GS_MAX_VIEWS
    # densify workspace
    w1, w2 = gs.gs_densify_workspace_size(1000), gs.gs_densify_workspace_size(2000)
    assert w2 > w1 > 0 and w1 % 256 == 0 and gs.gs_densify_workspace_size(0) == 0
    with pytest.raises(gs.GsError):
        gs.gs_densify_workspace_size(-1)
    # the readings' defaults reach the library as the thresholds the comparisons use
    st = gs.DensifyParams(1.5).struct()
    assert abs(st.prune_logit - math.log(0.005 / 0.995)) < 1e-6
    assert abs(st.split_log_gap - math.log(2.0)) < 1e-7 and abs(st.split_shrink - math.log(1.6)) < 1e-7
    assert abs(gs.DensifyParams.threshold_for(1080) - 1.62) < 1e-9
    # checks that return before any launch
    assert lib.gs_opacity_reset(10, 0.0, None, None, None, None) == -1
    assert lib.gs_opacity_reset(10, 1.5, None, None, None, None) == -1
    assert lib.gs_opacity_reset(0, 0.3, None, None, None, None) == 0
    fake = C.c_void_p(1 << 20)  # never dereferenced: every call below fails its checks first
    inp, out = gs.GsGaussianSet(), gs.GsGaussianSet()
    assert lib.gs_densify(C.byref(st), 10, 4, C.byref(inp), 20, C.byref(out), fake, fake, None, fake, 1 << 20,
                          None) == -1  # SH degree 4
    assert lib.gs_densify(C.byref(st), 10, 3, C.byref(inp), 20, C.byref(out), fake, fake, None, fake, 0,
                          None) == -3  # workspace too small


def test_nonfinite_and_measurement_host_checks():
    """Argument checks of the debug and measurement calls, answered on the host (no device work)."""
    import ctypes as C
    from differentiable_gaussian_splatting_dgs_amd import gs
    lib = gs.load_library()
    fake = C.c_void_p(1 << 20)  # never dereferenced: every call below fails its host checks
    assert lib.gs_count_nonfinite(fake, -1, fake, None) == -1
    assert lib.gs_count_nonfinite(fake, 4, None, None) == -1
    assert lib.gs_count_nonfinite(None, 4, fake, None) == -1
    from differentiable_gaussian_splatting_dgs_amd import measure
    mlib = measure.load_library()
    assert mlib.gs_stream_copy(fake, fake, 6, None) == -1
    assert mlib.gs_stream_copy(C.c_void_p((1 << 20) + 4), fake, 8, None) == -2
    assert mlib.gs_fma_loop(0, 1, 1.0, 0.0, fake, None) == -1
    assert mlib.gs_fma_loop(4, -1, 1.0, 0.0, fake, None) == -1
