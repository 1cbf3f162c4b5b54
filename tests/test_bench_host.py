"""Host logic of bench.py that needs no GPU: the single-GPU guard, argument
checks, the stage-roofline arithmetic and the host description."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_unknown_workload_is_refused():
    r = _run("--workload", "no-such-scene")
    assert r.returncode == 2
    assert "invalid choice" in r.stderr


def test_unknown_extra_is_refused():
    r = _run("--extras", "record16,no-such-field")
    assert r.returncode == 2
    assert "unknown extras" in r.stderr


def test_workloads_are_the_scene_generators():
    from differentiable_gaussian_splatting_dgs_amd import scenes
    assert set(bench.WORKLOADS) == set(scenes.WORKLOADS)


PEAKS = dict(hbm_gbs=dict(measured=4000.0), fp32_tflops=dict(measured=100.0))


def test_blend_flops_use_the_scope_figures():
    """20 flops per evaluated forward pair; 72 per walked backward pair that blends, 16 per one that does not."""
    f, b = bench.blend_flops(1000, 600, 200)
    assert f == 20 * 1000
    assert b == 72 * 200 + 16 * 400


def test_raster_roofline_fraction_is_bound_over_time():
    r = bench.raster_roofline(1_000_000, 5e6, 3, 3e8, 3e8, 1e8, 1.0, PEAKS)
    # the fraction is the summed stage bounds over the measured time
    assert r["frac"] == pytest.approx(r["t_min_sum_us"] * 1e-6 / 1e-3, rel=1e-3)
    # measured peaks are below the published ones, so the bound against them is larger
    assert r["t_min_sum_us_measured_peaks"] > r["t_min_sum_us"]
    assert set(r["t_min_us"]) == {"preprocess", "bin_sort", "render_fwd", "render_bwd", "preprocess_bwd"}
    assert all(v > 0 for v in r["t_min_us"].values())


def test_raster_roofline_scales_with_the_work():
    a = bench.raster_roofline(1_000_000, 5e6, 3, 3e8, 3e8, 1e8, 1.0, PEAKS)
    b = bench.raster_roofline(2_000_000, 1e7, 3, 6e8, 6e8, 2e8, 1.0, PEAKS)
    for k in a["t_min_us"]:
        assert b["t_min_us"][k] == pytest.approx(2 * a["t_min_us"][k], rel=2e-3), k
    # a lower SH degree reads fewer parameter bytes
    c = bench.raster_roofline(1_000_000, 5e6, 0, 3e8, 3e8, 1e8, 1.0, PEAKS)
    assert c["t_min_us"]["preprocess"] < a["t_min_us"]["preprocess"]
    assert c["t_min_us"]["render_fwd"] == a["t_min_us"]["render_fwd"]


def test_raster_roofline_with_the_colour_jacobian():
    """With the colour-direction Jacobian the preprocess writes 36 more bytes per Gaussian and the
    2D->3D backward reads them instead of the SH coefficients (192 bytes at degree 3)."""
    a = bench.raster_roofline(1_000_000, 5e6, 3, 3e8, 3e8, 1e8, 1.0, PEAKS)
    j = bench.raster_roofline(1_000_000, 5e6, 3, 3e8, 3e8, 1e8, 1.0, PEAKS, colorjac=True)
    hbm = bench.PEAK_HBM_GBS * 1e3  # bytes per us
    assert (j["t_min_us"]["preprocess"] - a["t_min_us"]["preprocess"]) * hbm == pytest.approx(36e6, rel=2e-3)
    assert (a["t_min_us"]["preprocess_bwd"] - j["t_min_us"]["preprocess_bwd"]) * hbm == pytest.approx(156e6, rel=2e-3)


def test_host_cpu_description():
    h = bench.host_cpu()
    assert isinstance(h["cpu_model"], str) and h["cpu_model"]
    assert isinstance(h["nproc"], int) and h["nproc"] >= 1
