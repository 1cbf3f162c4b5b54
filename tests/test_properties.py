"""Property tests over tiny random scenes (hypothesis), on the oracle (CPU) and
on the HIP path (GPU):

  * the result does not depend on the order the Gaussians are given in (the
    depth sort decides the compositing order; depths are drawn continuous, so
    the index tie-break never decides),
  * a Gaussian of (numerically) zero opacity changes nothing: its alpha is below
    the 1/255 skip threshold at every pixel.  Two forms: one added to the scene
    (the preprocess culls it), and a zero-opacity record put into every tile's
    list at a random position, which the blends must walk past,
  * the binned list has exactly sum(tiles_touched) entries.

Images are compared bit for bit (both sides composite the same pairs in the
same order).  Oracle gradients are bit-exact too (every Gaussian's gradient is
accumulated over pixels in image order whatever its input position); GPU
gradients are summed with float atomics in an order that can change with the
input order, so they are compared within 1e-5 relative L2.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, assume, given, settings, strategies as st

from differentiable_gaussian_splatting_dgs_amd import scenes

PARAM_KEYS = ("means", "log_scales", "quats", "opacity_logits", "sh")
_scene_args = dict(seed=st.integers(0, 2**31 - 1), n=st.integers(1, 24), deg=st.sampled_from([0, 1, 3]))
_cpu_settings = settings(max_examples=12, deadline=None, database=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
_gpu_settings = settings(max_examples=8, deadline=None, database=None, suppress_health_check=[HealthCheck.function_scoped_fixture])


def _scene(seed, n, deg):
    return scenes.random_small(seed, n=n, width=40, height=36, f=44.0, sh_degree=deg, scale_mu=-2.0)


def _permuted(sc, perm):
    p = {k: np.ascontiguousarray(v[perm]) for k, v in sc.params().items()}
    return p


def _with_transparent(sc, rng):
    """The scene plus one Gaussian of opacity sigmoid(-40) ~ 4e-18 placed in view."""
    p = {k: np.asarray(v) for k, v in sc.params().items()}
    extra = dict(means=np.array([[rng.uniform(-0.3, 0.3), rng.uniform(-0.3, 0.3), rng.uniform(2.0, 3.0)]]),
                 log_scales=np.full((1, 3), -1.5), quats=np.array([[1.0, 0.0, 0.0, 0.0]]),
                 opacity_logits=np.array([-40.0]), sh=np.ones((1,) + p["sh"].shape[1:]))
    return {k: np.ascontiguousarray(np.concatenate([p[k], extra[k].astype(np.float32)]), dtype=np.float32)
            for k in p}


def _distinct_depths(O, sc):
    pre = O.preprocess(sc.cam, sc.sh_degree, sc.params())
    d = np.asarray(pre["depth"], np.float64)[np.asarray(pre["tiles_touched"]) > 0]
    return len(np.unique(d.astype(np.float32))) == len(d)


# ---------------------------------------------------------------- oracle (CPU)

@given(**_scene_args, perm_seed=st.integers(0, 2**31 - 1))
@_cpu_settings
def test_oracle_input_order(oracle, seed, n, deg, perm_seed):
    sc = _scene(seed, n, deg)
    assume(_distinct_depths(oracle, sc))
    perm = np.random.default_rng(perm_seed).permutation(n)
    dL = np.asarray(sc.dL_dimage, np.float64)
    a = oracle.render(sc.cam, deg, sc.params(), dL_dimage=dL)
    b = oracle.render(sc.cam, deg, _permuted(sc, perm), dL_dimage=dL)
    assert np.array_equal(a["image"], b["image"])
    assert np.array_equal(a["n_contrib"] > 0, b["n_contrib"] > 0)
    for k in PARAM_KEYS:
        assert np.array_equal(a["g3d"][k][perm], b["g3d"][k]), k


@given(**_scene_args, extra_seed=st.integers(0, 2**31 - 1))
@_cpu_settings
def test_oracle_transparent_gaussian_changes_nothing(oracle, seed, n, deg, extra_seed):
    sc = _scene(seed, n, deg)
    dL = np.asarray(sc.dL_dimage, np.float64)
    a = oracle.render(sc.cam, deg, sc.params(), dL_dimage=dL)
    b = oracle.render(sc.cam, deg, _with_transparent(sc, np.random.default_rng(extra_seed)), dL_dimage=dL)
    assert np.array_equal(a["image"], b["image"])
    assert np.array_equal(a["final_T"], b["final_T"])
    for k in PARAM_KEYS:
        assert np.array_equal(a["g3d"][k], b["g3d"][k][:n]), k
        assert not np.any(b["g3d"][k][n:]), k


def _inject_zero(point_list, ranges, extra, rng):
    """Every tile's list with Gaussian `extra` inserted at a random position.
    Returns the new lists, ranges and each tile's insertion position."""
    pl, rg, pos = [], np.zeros_like(ranges), np.zeros(len(ranges), np.int64)
    k = 0
    for t in range(len(ranges)):
        lst = list(point_list[ranges[t, 0]:ranges[t, 1]])
        at = int(rng.integers(0, len(lst) + 1))
        lst.insert(at, extra)
        rg[t] = (k, k + len(lst))
        pos[t] = at
        k += len(lst)
        pl.extend(lst)
    return np.array(pl, np.int32), rg, pos


def _shifted_n_contrib(n_contrib, pos, width, height):
    """n_contrib once every tile's list holds one more entry at pos[tile]: positions
    at or after the insertion move up by one."""
    ntx = (width + 15) // 16
    ty, tx = np.meshgrid(np.arange(height) // 16, np.arange(width) // 16, indexing="ij")
    p = pos[ty * ntx + tx]
    return np.where((n_contrib > 0) & (p < n_contrib), n_contrib + 1, n_contrib)


def _zero_record(rng, cam):
    """A projected Gaussian of opacity 0 somewhere on the image (mean, conic, colour)."""
    uv = np.array([[rng.uniform(0, cam.width), rng.uniform(0, cam.height)]])
    conic = np.array([[0.02, 0.005, 0.03]])
    return uv, conic, np.zeros(1), np.array([[0.7, 0.2, 0.9]])


@given(**_scene_args, extra_seed=st.integers(0, 2**31 - 1))
@_cpu_settings
def test_oracle_zero_opacity_entry_in_lists_changes_nothing(oracle, seed, n, deg, extra_seed):
    sc = _scene(seed, n, deg)
    rng = np.random.default_rng(extra_seed)
    dL = np.asarray(sc.dL_dimage, np.float64)
    r = oracle.render(sc.cam, deg, sc.params(), backward=False)
    pre = r["pre"]
    uv, conic, op, rgb = _zero_record(rng, sc.cam)
    pre2 = dict(pre, uv=np.concatenate([pre["uv"], uv]), conic=np.concatenate([pre["conic"], conic]),
                opacity=np.concatenate([pre["opacity"], op]), rgb=np.concatenate([pre["rgb"], rgb]))
    pl2, rg2, pos = _inject_zero(r["point_list"], r["ranges"], n, rng)
    f1 = oracle.render_fwd(sc.cam, pre, r["point_list"], r["ranges"])
    f2 = oracle.render_fwd(sc.cam, pre2, pl2, rg2)
    assert np.array_equal(f1["image"], f2["image"])
    assert np.array_equal(f1["final_T"], f2["final_T"])
    assert np.array_equal(f2["n_contrib"], _shifted_n_contrib(f1["n_contrib"], pos, sc.cam.width, sc.cam.height))
    assert f2["counts"][2] == f1["counts"][2]
    g1 = oracle.render_bwd(sc.cam, pre, r["point_list"], r["ranges"], dL)
    g2 = oracle.render_bwd(sc.cam, pre2, pl2, rg2, dL)
    for k in g1:
        assert np.array_equal(g1[k], g2[k][:n]), k
        assert not np.any(g2[k][n:]), k


@given(**_scene_args)
@_cpu_settings
def test_oracle_list_length_is_tiles_touched(oracle, seed, n, deg):
    sc = _scene(seed, n, deg)
    r = oracle.render(sc.cam, deg, sc.params(), backward=False)
    assert len(r["point_list"]) == int(np.sum(r["pre"]["tiles_touched"]))


# ---------------------------------------------------------------- HIP path (GPU)

def _gpu_run(cam, deg, params, dL):
    import torch
    from differentiable_gaussian_splatting_dgs_amd import gs
    p = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in params.items()}
    r = gs.Rasterizer(cam, p["means"].shape[0], deg)
    img = r.forward(p, check=True).clone()
    g = r.backward(p, torch.from_numpy(np.ascontiguousarray(dL, dtype=np.float32)).cuda())
    torch.cuda.synchronize()
    return dict(image=img.cpu().numpy(), K=int(r.num_keys.item()), tt=r.tiles_touched.cpu().numpy(),
                g3d={k: v.cpu().numpy() for k, v in g.items()})


def _rel_l2(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / nb if nb > 0 else np.linalg.norm(a)


@pytest.mark.gpu
@given(**_scene_args, perm_seed=st.integers(0, 2**31 - 1))
@_gpu_settings
def test_gpu_input_order(oracle, seed, n, deg, perm_seed):
    sc = _scene(seed, n, deg)
    assume(_distinct_depths(oracle, sc))
    perm = np.random.default_rng(perm_seed).permutation(n)
    a = _gpu_run(sc.cam, deg, sc.params(), sc.dL_dimage)
    b = _gpu_run(sc.cam, deg, _permuted(sc, perm), sc.dL_dimage)
    assert np.array_equal(a["image"], b["image"])
    assert a["K"] == b["K"]
    for k in PARAM_KEYS:
        assert _rel_l2(b["g3d"][k], a["g3d"][k][perm]) <= 1e-5, k


@pytest.mark.gpu
@given(**_scene_args, extra_seed=st.integers(0, 2**31 - 1))
@_gpu_settings
def test_gpu_transparent_gaussian_changes_nothing(seed, n, deg, extra_seed):
    sc = _scene(seed, n, deg)
    a = _gpu_run(sc.cam, deg, sc.params(), sc.dL_dimage)
    b = _gpu_run(sc.cam, deg, _with_transparent(sc, np.random.default_rng(extra_seed)), sc.dL_dimage)
    assert np.array_equal(a["image"], b["image"])
    assert b["tt"][n] == 0
    for k in PARAM_KEYS:
        assert _rel_l2(b["g3d"][k][:n], a["g3d"][k]) <= 1e-5, k
        assert not np.any(b["g3d"][k][n:]), k


@pytest.mark.gpu
@given(**_scene_args, extra_seed=st.integers(0, 2**31 - 1))
@_gpu_settings
def test_gpu_zero_opacity_entry_in_lists_changes_nothing(seed, n, deg, extra_seed):
    """The blend kernels walk past a zero-opacity record placed in every tile's list:
    image and final_T bit-identical, n_contrib shifted by the insertion, the other
    Gaussians' 2D gradients unchanged (within atomic order) and none for it."""
    import torch
    from differentiable_gaussian_splatting_dgs_amd import gs
    sc = _scene(seed, n, deg)
    rng = np.random.default_rng(extra_seed)
    p = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in sc.params().items()}
    r = gs.Rasterizer(sc.cam, n, deg)
    r.forward(p, check=True)
    dL = torch.from_numpy(np.ascontiguousarray(sc.dL_dimage, dtype=np.float32)).cuda()
    g_a = r.backward_2d(dL).clone()
    torch.cuda.synchronize()
    K = int(r.num_keys.item())
    uv, conic, _, rgb = _zero_record(rng, sc.cam)
    # the record in the library's layout: mean, zero residual, a Cholesky factor, opacity 0, colour
    extra = torch.zeros((1, gs.SPLAT_STRIDE), dtype=torch.float32, device="cuda")
    extra[0, 0:2] = torch.from_numpy(uv[0].astype(np.float32))
    extra[0, 4:7] = torch.tensor([0.1, 0.01, 0.12])
    extra[0, 8:11] = torch.from_numpy(rgb[0].astype(np.float32))
    splats2 = torch.cat([r.splats, extra]).contiguous()
    pl = r.point_list[:K].cpu().numpy()
    rg = r.tile_ranges.cpu().numpy().astype(np.int64)
    pl2, rg2, pos = _inject_zero(pl, rg, n, rng)
    pl2_d = torch.from_numpy(pl2).cuda()
    rg2_d = torch.from_numpy(rg2.astype(np.int32)).cuda()
    img2 = torch.empty_like(r.image)
    T2 = torch.empty_like(r.final_T)
    nc2 = torch.empty_like(r.n_contrib)
    contrib2 = torch.empty(len(pl2), dtype=torch.uint8, device="cuda")
    order2 = torch.empty_like(r.tile_order)
    st = r.settings
    gs.gs_render_fwd(sc.cam, st, n + 1, rg2_d, pl2_d, splats2, img2, T2, nc2, contrib2, order2)
    g_b = torch.empty((n + 1, gs.GRAD2D_STRIDE), dtype=torch.float32, device="cuda")
    gs.gs_render_bwd(sc.cam, st, n + 1, rg2_d, pl2_d, splats2, T2, nc2, contrib2, dL, g_b, False, order2[1])
    torch.cuda.synchronize()
    assert torch.equal(img2, r.image)
    assert torch.equal(T2, r.final_T)
    want_nc = _shifted_n_contrib(r.n_contrib.cpu().numpy(), pos, sc.cam.width, sc.cam.height)
    assert np.array_equal(nc2.cpu().numpy(), want_nc)
    assert _rel_l2(g_b[:n].cpu().numpy(), g_a.cpu().numpy()) <= 1e-5
    assert not torch.any(g_b[n:])


@pytest.mark.gpu
@given(**_scene_args)
@_gpu_settings
def test_gpu_list_length_is_tiles_touched(seed, n, deg):
    sc = _scene(seed, n, deg)
    a = _gpu_run(sc.cam, deg, sc.params(), sc.dL_dimage)
    assert a["K"] == int(np.sum(a["tt"]))
