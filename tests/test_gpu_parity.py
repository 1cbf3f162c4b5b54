"""Parity of the HIP path (called through the C ABI) with the CPU oracle.

Stage-wise: preprocess, binning (bit-exact), forward, 2D and 3D gradients;
on the workload shapes (tiny, 100k@800^2 with L2 loss, 1M@1080p, 3M@4K,
all pixels composited by the oracle) plus random small scenes with SH
degrees 1 and 2 and two scenes either side of the backward's 1024-tile split.
"""
import numpy as np
import pytest

from gpu_cases import CASES, PARAM_KEYS, guard_2d, guard_chain, log, rel_l2, run_case

pytestmark = pytest.mark.gpu

NAMES = list(CASES)


def case(name):
    fn, stride = CASES[name]
    return run_case(name, fn, tile_stride=stride)


@pytest.mark.parametrize("name", NAMES)
def test_preprocess(name):
    c = case(name)
    g, pre = c["gpu"], c["pre"]
    sp = g["splats"]
    valid = pre["valid"] > 0
    vis = pre["tiles_touched"] > 0
    # integer outputs bit-exact
    assert np.array_equal(g["tt"], pre["tiles_touched"]), np.nonzero(g["tt"] != pre["tiles_touched"])[0][:10]
    rect_o = pre["rect"][:, [0, 1, 2, 3]]
    assert np.array_equal(g["rect"][vis].astype(np.int32), rect_o[vis])
    assert np.array_equal(g["depth"][valid], pre["depth"][valid].astype(np.float32))
    # 2D mean: float32 value + float32 residual reproduce the float64 mean
    u = sp[:, 0].astype(np.float64) + sp[:, 2]
    v = sp[:, 1].astype(np.float64) + sp[:, 3]
    assert np.abs(u[valid] - pre["uv"][valid, 0]).max() <= 1e-9 * max(1.0, np.abs(pre["uv"][valid, 0]).max())
    assert np.abs(v[valid] - pre["uv"][valid, 1]).max() <= 1e-9 * max(1.0, np.abs(pre["uv"][valid, 1]).max())
    # conic from the scaled Cholesky factor: conic = (2 / log2 e) L L^T
    k = 2.0 / np.log2(np.e)
    l00, l10, l11 = (sp[:, i].astype(np.float64) for i in (4, 5, 6))
    A, B, C = k * l00 * l00, k * l00 * l10, k * (l10 * l10 + l11 * l11)
    co = pre["conic"]
    scale = np.sqrt(co[:, 0] * co[:, 2])
    # each factor entry is one float32 rounding of the float64 value: per-component
    # relative error of a few 1e-7
    for got, ref in ((A, co[:, 0]), (B, co[:, 1]), (C, co[:, 2])):
        err = (np.abs(got - ref) / (np.abs(ref) + 1e-9 * scale))[valid]
        assert err.max() <= 1e-6, err.max()
    assert np.abs(sp[valid, 7] - pre["opacity"][valid]).max() <= 1e-7
    assert np.abs(sp[valid, 8:11] - pre["rgb"][valid]).max() <= 1e-6
    # clamp mask exact unless the raw colour is within float32 rounding of zero
    assert (g["clamp"][valid] != pre["clamp"][valid]).sum() == 0
    log(f"[{name}] preprocess ok, visible={vis.sum()}")


@pytest.mark.parametrize("name", NAMES)
def test_binning_bit_exact(name):
    from oracle import oracle as O
    c = case(name)
    g, sc = c["gpu"], c["scene"]
    assert g["overflow"] == 0
    # the oracle bins the GPU's own preprocess outputs
    rect = g["rect"].astype(np.int32)
    pl, rg = O.bin_gaussians(sc.cam, rect, g["tt"], g["depth"].astype(np.float64))
    assert g["K"] == len(pl) == int(g["tt"].astype(np.int64).sum())
    # an empty tile's range is any [b, b); the library writes [0, 0)
    rg = np.where((rg[:, 1] == rg[:, 0])[:, None], 0, rg)
    assert np.array_equal(g["ranges"].astype(np.int64), rg)
    assert np.array_equal(g["point_list"].astype(np.int64), pl.astype(np.int64))
    log(f"[{name}] binning bit-exact K={g['K']}")


@pytest.mark.parametrize("name", NAMES)
def test_forward(name):
    c = case(name)
    g, fwd, m = c["gpu"], c["fwd"], c["pixmask"]
    ok = m & ~c["amb"]
    n_amb = int((c["amb"] & m).sum())
    assert n_amb <= max(2, 1e-3 * m.sum()), (n_amb, m.sum())
    err = np.abs(g["image"] - fwd["image"])[:, ok]
    assert err.max() <= 1e-5, (err.max(), np.unravel_index(np.argmax(np.abs(g["image"] - fwd["image"]) * ok), g["image"].shape))
    assert np.abs(g["final_T"] - fwd["final_T"])[ok].max() <= 1e-5
    bad = (g["n_contrib"] != fwd["n_contrib"]) & ok
    assert bad.sum() == 0, (bad.sum(), np.argwhere(bad)[:5])
    log(f"[{name}] forward max err {err.max():.2e}, ambiguous {n_amb} of {m.sum()}")


@pytest.mark.parametrize("name", NAMES)
def test_pair_counts(name):
    """The GPU pair counter (the bench's pairs/s numerator) against the oracle: per pixel on
    every pixel the oracle composited, outside ambiguous ones, the evaluated count (P_fwd's
    share) and n_contrib (P_bwd's) are equal; the totals differ only through ambiguous pixels."""
    c = case(name)
    g, fwd, m = c["gpu"], c["fwd"], c["pixmask"]
    ok = m & ~c["amb"]
    bad = (g["evaluated"] != fwd["evaluated"]) & ok
    assert bad.sum() == 0, (bad.sum(), np.argwhere(bad)[:5])
    assert np.array_equal(g["n_contrib"][ok], fwd["n_contrib"][ok])
    # totals over the composited pixels; an ambiguous pixel can move them by at most its list length
    amb = c["amb"] & m
    slack = int(fwd["evaluated"][amb].sum() + g["evaluated"][amb].sum()) + 16
    assert abs(int(g["evaluated"][m].sum()) - int(fwd["evaluated"][m].sum())) <= slack
    assert abs(int(g["n_contrib"][m].astype(np.int64).sum()) - int(fwd["n_contrib"][m].sum())) <= slack
    if m.all():
        assert abs(int(g["counts"][0]) - int(fwd["counts"][0])) <= slack
        assert abs(int(g["counts"][1]) - int(fwd["counts"][1])) <= slack
        assert abs(int(g["counts"][2]) - int(fwd["counts"][2])) <= slack
    assert int(g["counts"][0]) == int(g["evaluated"].astype(np.int64).sum())
    assert int(g["counts"][1]) == int(g["n_contrib"].astype(np.int64).sum())
    log(f"[{name}] pair counts ok: P_fwd {int(g['counts'][0])}, P_bwd {int(g['counts'][1])}, "
        f"ambiguous pixels {int(amb.sum())}")


@pytest.mark.parametrize("name", NAMES)
def test_backward_2d(name):
    c = case(name)
    g2, o2 = c["gpu"]["grad2d"], c["g2o"]
    vis = c["pre"]["tiles_touched"] > 0
    pairs = [("dxy", g2[:, 0:2]), ("dconic", g2[:, 2:5]), ("dopacity", g2[:, 5]), ("drgb", g2[:, 6:9])]
    for key, got in pairs:
        e = rel_l2(got[vis], o2[key][vis])
        assert e <= 1e-3, (key, e)
    assert np.all(g2[:, 9:] == 0)
    assert np.all(g2[~vis] == 0)
    guard_2d(g2, o2, name)
    log(f"[{name}] 2D grads ok")


@pytest.mark.parametrize("name", NAMES)
def test_backward_3d(name):
    c = case(name)
    g3, o3 = c["gpu"]["g3d"], c["g3o"]
    errs = {}
    for k in PARAM_KEYS:
        errs[k] = rel_l2(g3[k], o3[k])
        assert np.isfinite(g3[k]).all(), k
    log(f"[{name}] 3D grad rel L2: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert e <= 1e-3, (k, e)
    sc = c["scene"]
    guard_chain(sc.cam, sc.sh_degree, sc.params(), c["gpu"]["tt"], c["gpu"]["grad2d"], g3, name)
