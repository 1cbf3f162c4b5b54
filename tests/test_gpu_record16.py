"""Parity of the 16-bit splat record path (gs_preprocess_h16 and the _h16 blends)
with the CPU oracle reading the same record (oracle.record16).

Contract (Gaussian Splatting backward CUDA page (lshu.cn), sections 5 and 7:
16-bit intermediates, FP16 rendering path, FP32 gradient sums):
  * the record: the mean words are the float32 record's u, v; every binary16
    word is numpy's float16 rounding of the float32 record's value; rect,
    tiles_touched, depth and the clamp mask equal gs_preprocess's bit for bit.
  * against the oracle's record of its own float64 projection, the decoded
    values agree exactly except where the two float32 values straddle a
    binary16 rounding boundary (a one-ulp difference; such Gaussians are counted,
    must be rare, and their tiles are left out of the image and gradient checks).
  * the blends, the pair counts and the gradients are held to the float32
    path's bars against the oracle rendering from the rounded record: image
    within 1e-5 and n_contrib exact outside ambiguous pixels, 2D gradients within
    1e-3 relative L2 and element-wise within 1e-3 of their term sizes, 3D
    gradients within 1e-3 relative L2.
"""
import numpy as np
import pytest

from gpu_cases import CASES, PARAM_KEYS, guard_2d, log, rel_l2, to_dev

pytestmark = pytest.mark.gpu

NAMES = ["tiny", "random_sh1", "random_sh2", "tiles1023", "tiles1024", "ball100k", "clusters1m", "plane3m"]
_CACHE = {}
S2 = 0.5 / np.log(2.0)  # s^2: L L^T = s^2 conic


def _halves(words):
    """[n, k] float32 storage of binary16 pairs -> [n, 2k] float64 (low half first)."""
    h = np.ascontiguousarray(words).view(np.uint32)
    lo = (h & 0xFFFF).astype(np.uint16).view(np.float16)
    hi = (h >> 16).astype(np.uint16).view(np.float16)
    return np.stack([lo, hi], -1).reshape(len(h), -1).astype(np.float64)


def run16(name):
    if name in _CACHE:
        return _CACHE[name]
    import torch
    from differentiable_gaussian_splatting_dgs_amd import gs
    from oracle import oracle as O
    sc = CASES[name][0]()
    log(f"[{name}] record16: n={sc.n} {sc.cam.width}x{sc.cam.height} deg={sc.sh_degree}")
    p = to_dev(sc.params())
    r = gs.Rasterizer(sc.cam, sc.n, sc.sh_degree, record16=True)
    r.forward(p, check=True)
    counts, ev_px = r.count_pairs(per_pixel=True)
    # the float32 record of the same scene, for the record check
    r32 = gs.Rasterizer(sc.cam, sc.n, sc.sh_degree, key_capacity=r.key_capacity)
    r32.preprocess(p)
    torch.cuda.synchronize()
    K = int(r.num_keys.item())
    g = dict(rec=r.splats.cpu().numpy(), rec32=r32.splats.cpu().numpy(), depth=r.depth.cpu().numpy(),
             depth32=r32.depth.cpu().numpy(), rect=r.rect.cpu().numpy(), rect32=r32.rect.cpu().numpy(),
             tt=r.tiles_touched.cpu().numpy(), tt32=r32.tiles_touched.cpu().numpy(), clamp=r.clamp.cpu().numpy(),
             clamp32=r32.clamp.cpu().numpy(), K=K, point_list=r.point_list[:K].cpu().numpy(),
             ranges=r.tile_ranges.cpu().numpy(), image=r.image.cpu().numpy(), final_T=r.final_T.cpu().numpy(),
             n_contrib=r.n_contrib.cpu().numpy(), counts=counts.cpu().numpy(), evaluated=ev_px.cpu().numpy())
    del r32
    log(f"[{name}] gpu forward done K={K}")

    s = O.Settings()
    pre = O.preprocess(sc.cam, sc.sh_degree, sc.params(), s)
    pre16 = O.record16(pre)
    pl, rg = O.bin_gaussians(sc.cam, pre["rect"], pre["tiles_touched"], O.depth_key(pre["depth"]), s)

    # Gaussians whose record differs from the oracle's (a one-ulp binary16 difference where the
    # two float32 values straddle a rounding boundary): their tiles are left out
    rec = g["rec"]
    h = _halves(rec[:, 2:6])
    l00, l10, l11, op16, rgb16 = h[:, 0], h[:, 1], h[:, 2], h[:, 3], h[:, 4:7]
    conic_g = np.stack([l00 * l00, l00 * l10, l10 * l10 + l11 * l11], 1) / S2
    co = pre16["conic"]
    scale = np.sqrt(np.abs(co[:, 0] * co[:, 2])) + 1e-300
    valid = pre["valid"] > 0
    diff = (np.abs(conic_g - co).max(1) > 1e-12 * scale) | (op16 != pre16["opacity"]) | \
           np.any(rgb16 != pre16["rgb"], 1) | np.any(rec[:, :2].astype(np.float64) != pre16["uv"], 1)
    diff &= valid
    ntx, nty = (sc.cam.width + 15) // 16, (sc.cam.height + 15) // 16
    tmask = np.ones((nty, ntx), np.uint8)
    for i in np.nonzero(diff)[0]:
        x0, y0, x1, y1 = pre["rect"][i]
        tmask[y0:y1, x0:x1] = 0
    pixmask = np.repeat(np.repeat(tmask, 16, 0), 16, 1)[: sc.cam.height, : sc.cam.width] > 0
    log(f"[{name}] records differing from the oracle's: {int(diff.sum())} of {int(valid.sum())}; "
        f"tiles left out {int((tmask == 0).sum())} of {tmask.size}")

    full = tmask.all()
    fwd = O.render_fwd(sc.cam, pre16, pl, rg, s, tile_mask=None if full else tmask.ravel())
    amb = (fwd["ambiguous"] & 3) > 0
    amb_grad = fwd["ambiguous"] > 0
    if sc.dL_dimage is not None:
        dL = np.asarray(sc.dL_dimage, np.float64)
    else:
        _, dL = O.loss(sc.loss, fwd["image"], sc.target)
    dL = dL * (pixmask & ~amb_grad)[None]
    g3 = r.backward(p, torch.from_numpy(dL.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    g["grad2d"] = r.grad2d.cpu().numpy()
    g["g3d"] = {k: v.cpu().numpy() for k, v in g3.items()}
    g2o = O.render_bwd(sc.cam, pre16, pl, rg, dL, s, tile_mask=None if full else tmask.ravel(), with_abs=True)
    g3o = O.preprocess_bwd(sc.cam, sc.sh_degree, sc.params(), pre["tiles_touched"], g2o, s)
    log(f"[{name}] oracle done")
    res = dict(scene=sc, gpu=g, pre=pre, pre16=pre16, pl=pl, rg=rg, fwd=fwd, amb=amb, pixmask=pixmask,
               diff=diff, g2o=g2o, g3o=g3o)
    _CACHE[name] = res
    del r
    torch.cuda.empty_cache()
    return res


@pytest.mark.parametrize("name", NAMES)
def test_record16_record(name):
    c = run16(name)
    g = c["gpu"]
    # binning inputs and the clamp mask are those of the float32 preprocess, bit for bit
    for k in ("depth", "rect", "tt", "clamp"):
        assert np.array_equal(g[k], g[k + "32"]), k
    rec, r32 = g["rec"], g["rec32"]
    assert np.array_equal(rec[:, :2], r32[:, :2])
    h = _halves(rec[:, 2:6])
    want = r32[:, [4, 5, 6, 7, 8, 9, 10]].astype(np.float16).astype(np.float64)
    assert np.array_equal(h[:, :7], want)
    assert np.all(h[:, 7] == 0)
    # culled Gaussians: an all-zero record
    culled = c["pre"]["valid"] == 0
    assert np.all(rec[culled].view(np.uint32) == 0)
    nd, nv = int(c["diff"].sum()), int((c["pre"]["valid"] > 0).sum())
    assert nd <= max(3, 1e-4 * nv), (nd, nv)
    log(f"[{name}] record ok; {nd} of {nv} differ from the oracle's by a rounding-boundary ulp")


@pytest.mark.parametrize("name", NAMES)
def test_record16_binning_and_forward(name):
    c = run16(name)
    g, fwd, m = c["gpu"], c["fwd"], c["pixmask"]
    assert g["K"] == len(c["pl"])
    assert np.array_equal(g["point_list"].astype(np.int64), c["pl"].astype(np.int64))
    ok = m & ~c["amb"]
    n_amb = int((c["amb"] & m).sum())
    assert n_amb <= max(2, 1e-3 * m.sum()), (n_amb, m.sum())
    err = np.abs(g["image"] - fwd["image"])[:, ok]
    assert err.max() <= 1e-5, err.max()
    assert np.abs(g["final_T"] - fwd["final_T"])[ok].max() <= 1e-5
    bad = (g["n_contrib"] != fwd["n_contrib"]) & ok
    assert bad.sum() == 0, (bad.sum(), np.argwhere(bad)[:5])
    bad = (g["evaluated"] != fwd["evaluated"]) & ok
    assert bad.sum() == 0, (bad.sum(), np.argwhere(bad)[:5])
    assert int(g["counts"][0]) == int(g["evaluated"].astype(np.int64).sum())
    assert int(g["counts"][1]) == int(g["n_contrib"].astype(np.int64).sum())
    log(f"[{name}] record16 forward max err {err.max():.2e}, ambiguous {n_amb}, pixels checked {int(ok.sum())}")


@pytest.mark.parametrize("name", NAMES)
def test_record16_backward(name):
    c = run16(name)
    g2, o2 = c["gpu"]["grad2d"], c["g2o"]
    vis = c["pre"]["tiles_touched"] > 0
    for key, got in (("dxy", g2[:, 0:2]), ("dconic", g2[:, 2:5]), ("dopacity", g2[:, 5]), ("drgb", g2[:, 6:9])):
        e = rel_l2(got[vis], o2[key][vis])
        assert e <= 1e-3, (key, e)
    guard_2d(g2, o2, name + " record16")
    g3, o3 = c["gpu"]["g3d"], c["g3o"]
    errs = {k: rel_l2(g3[k], o3[k]) for k in PARAM_KEYS}
    log(f"[{name}] record16 3D grad rel L2: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert np.isfinite(g3[k]).all(), k
        assert e <= 1e-3, (k, e)


def test_record16_argument_checks():
    import torch
    from differentiable_gaussian_splatting_dgs_amd import gs, scenes
    sc = scenes.tiny()
    p = to_dev(sc.params())
    r = gs.Rasterizer(sc.cam, sc.n, sc.sh_degree, record16=True)
    r.forward(p)
    # an 8-byte-aligned record is accepted, a 4-byte-aligned one is not
    buf = torch.zeros(sc.n * gs.SPLAT16_STRIDE + 2, dtype=torch.float32, device="cuda")
    with pytest.raises(gs.GsError, match="gs_preprocess_h16"):
        gs.gs_preprocess_h16(sc.cam, r.settings, sc.sh_degree, p["means"], p["log_scales"], p["quats"],
                             p["opacity_logits"], p["sh"], buf[1:1 + sc.n * gs.SPLAT16_STRIDE], r.depth, r.rect,
                             r.tiles_touched, r.clamp)
    with pytest.raises(gs.GsError, match="gs_render_fwd_h16"):
        gs.gs_render_fwd_h16(sc.cam, r.settings, sc.n, r.tile_ranges, r.point_list,
                             buf[1:1 + sc.n * gs.SPLAT16_STRIDE], r.image, r.final_T, r.n_contrib, r.contrib)
    with pytest.raises(gs.GsError):
        r.render_loss(torch.zeros_like(r.image), "l1", torch.zeros_like(r.image),
                      torch.zeros(1 + r.ntiles, dtype=torch.float64, device="cuda"))
    torch.cuda.synchronize()


def test_record16_empty_and_all_culled():
    """No Gaussians, and Gaussians that are all culled: empty lists, the background, zero gradients."""
    import torch
    from differentiable_gaussian_splatting_dgs_amd import gs, scenes
    cam = scenes.Camera.identity(40, 24, 30.0)
    r = gs.Rasterizer(cam, 0, 0, key_capacity=16, record16=True)
    p = {k: torch.zeros((0,) + s, device="cuda") for k, s in
         dict(means=(3,), log_scales=(3,), quats=(4,), opacity_logits=(), sh=(1, 3)).items()}
    r.forward(p)
    torch.cuda.synchronize()
    assert int(r.num_keys.item()) == 0 and int(r.overflow.item()) == 0
    assert torch.all(r.image == 0) and torch.all(r.final_T == 1) and torch.all(r.n_contrib == 0)
    sc = scenes.random_small(31, n=100, width=33, height=17)
    sc.means[:50, 2] = 0.1          # inside the near plane
    sc.means[50:, 2] = -3.0         # behind the camera
    p = to_dev(sc.params())
    r = gs.Rasterizer(sc.cam, sc.n, sc.sh_degree, record16=True)
    r.forward(p)
    g3 = r.backward(p, torch.ones_like(r.image))
    torch.cuda.synchronize()
    assert int(r.num_keys.item()) == 0
    assert torch.all(r.image == 0)
    assert torch.all(r.splats.view(torch.int32) == 0)
    for k, v in g3.items():
        assert torch.all(v == 0), k
