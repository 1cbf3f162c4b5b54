"""Shared machinery of the GPU parity tests: run the HIP path through the C ABI
and the CPU oracle on the same seeded scene, and keep both results.

The comparison protocol (stage-wise, then end to end):
  * preprocess: GPU float32 outputs against the oracle's float64 values;
    tiles_touched, rect and the float32 depth key bit-exact.
  * binning: the oracle bins the GPU's own depth/rect/tiles_touched; point
    lists, tile ranges and K must match bit for bit.
  * forward: image within 1e-5 max-abs and n_contrib exact, outside pixels
    the oracle flags as ambiguous (some pair's opacity*G within a relative
    1e-5 of alpha_min, or T(1 - alpha) within 1e-5 of T_min, where both
    branches are correct results of float32 arithmetic).
  * backward: both sides get the same upstream gradient, zeroed at ambiguous
    pixels (and outside the sampled tiles when a tile subset is used); every
    3D gradient tensor within 1e-3 relative L2.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from differentiable_gaussian_splatting_dgs_amd import scenes  # noqa: E402

PARAM_KEYS = ("means", "log_scales", "quats", "opacity_logits", "sh")
_CACHE = {}


def log(*a):
    print(*a, flush=True)


def to_dev(p):
    import torch
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in p.items()}


def rowwise_errors(got, ref):
    """Per-Gaussian (row) error of a gradient tensor: the row's error norm over its
    reference norm plus a floor of 1e-4 of the tensor's RMS row norm (rows whose
    reference is that small carry no meaningful relative error)."""
    got = np.asarray(got, np.float64).reshape(len(got), -1)
    ref = np.asarray(ref, np.float64).reshape(len(ref), -1)
    rn = np.linalg.norm(ref, axis=1)
    rms = np.sqrt(np.mean(rn * rn)) if len(rn) else 0.0
    return np.linalg.norm(got - ref, axis=1) / (rn + 1e-4 * rms + 1e-30)


def grad2d_rows(g2):
    """The oracle's 2D gradients as [N, 9] in the library's record order."""
    return np.column_stack([g2["dxy"], g2["dconic"], g2["dopacity"][:, None], g2["drgb"]])


def grad2d_dict(rec):
    """The library's 2D gradient records [N, 12] as the oracle's dict."""
    rec = np.asarray(rec, np.float64)
    return dict(dxy=rec[:, 0:2], dconic=rec[:, 2:5], dopacity=rec[:, 5].copy(), drgb=rec[:, 6:9])


def guard_2d(got_rec, g2o, name, bound=1e-3):
    """Element-wise guard of the 2D gradients: every component of every Gaussian within `bound` of
    the sum of the absolute sizes of its terms (the oracle's `abs`), which bounds the rounding of a
    float32 evaluation and summation of the same terms in any order."""
    got = np.asarray(got_rec, np.float64)[:, :9]
    ref, a = grad2d_rows(g2o), g2o["abs"]
    zero = a == 0
    assert not np.any(got[zero]), (name, int(np.count_nonzero(got[zero])))
    r = np.where(zero, 0.0, np.abs(got - ref) / np.where(zero, 1.0, a))
    if r.size:
        worst = np.unravel_index(np.argmax(r), r.shape)
        log(f"    {name}: 2D error / term sizes: median {np.median(r[~zero]):.1e}, "
            f"p99.99 {np.quantile(r[~zero], 0.9999):.1e}, max {r.max():.1e} (Gaussian {worst[0]}, component {worst[1]})")
        assert r.max() <= bound, (name, float(r.max()), int((r > bound).sum()), worst)


def guard_chain(cam, deg, params, tiles_touched, got_rec, got3, name, bound=1e-2):
    """Element-wise guard of the 2D -> 3D backward alone: the oracle's chain fed the GPU's own 2D
    gradients against the GPU's 3D gradients, row by row (rowwise_errors).  The kernel recomputes
    the 2D covariance and its inverse in float32, so a nearly singular one carries relative errors
    of its condition number times 6e-8 (up to a few 1e-3 on 1M-Gaussian scenes); a mistake in the
    chain shows as an error of order one."""
    from oracle import oracle as O
    o3 = O.preprocess_bwd(cam, deg, params, tiles_touched, grad2d_dict(got_rec))
    vis = np.asarray(tiles_touched) > 0
    for k in o3:
        e = rowwise_errors(np.asarray(got3[k])[vis], o3[k][vis])
        if e.size:
            log(f"    {name} {k}: chain row error median {np.median(e):.1e}, p99.99 {np.quantile(e, 0.9999):.1e}, "
                f"max {e.max():.1e}")
            assert e.max() <= bound, (name, k, float(e.max()), int((e > bound).sum()))


def rel_l2(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / nb if nb > 0 else np.linalg.norm(a)


def gpu_forward(scene, key_capacity=None):
    import torch
    from differentiable_gaussian_splatting_dgs_amd import gs
    p = to_dev(scene.params())
    r = gs.Rasterizer(scene.cam, scene.n, scene.sh_degree, key_capacity=key_capacity)
    r.forward(p, check=True)
    torch.cuda.synchronize()
    return r, p


def run_case(name, scene_fn, tile_stride=1, seed=0):
    """Everything the parity tests compare, computed once per scene."""
    if name in _CACHE:
        return _CACHE[name]
    import torch
    from oracle import oracle as O
    t0 = time.time()
    sc = scene_fn()
    log(f"[{name}] scene n={sc.n} {sc.cam.width}x{sc.cam.height} deg={sc.sh_degree} ({time.time() - t0:.1f}s)")
    r, p = gpu_forward(sc)
    K = int(r.num_keys.item())
    g = dict(splats=r.splats.cpu().numpy(), depth=r.depth.cpu().numpy(), rect=r.rect.cpu().numpy(),
             tt=r.tiles_touched.cpu().numpy(), clamp=r.clamp.cpu().numpy(), K=K,
             overflow=int(r.overflow.item()), point_list=r.point_list[:K].cpu().numpy(),
             ranges=r.tile_ranges.cpu().numpy(), image=r.image.cpu().numpy(), final_T=r.final_T.cpu().numpy(),
             n_contrib=r.n_contrib.cpu().numpy())
    counts, ev_px = r.count_pairs(per_pixel=True)
    torch.cuda.synchronize()
    g["counts"] = counts.cpu().numpy()
    g["evaluated"] = ev_px.cpu().numpy()
    log(f"[{name}] gpu forward done K={K} ({time.time() - t0:.1f}s)")

    s = O.Settings()
    pre = O.preprocess(sc.cam, sc.sh_degree, sc.params(), s)
    dk = O.depth_key(pre["depth"])
    pl, rg = O.bin_gaussians(sc.cam, pre["rect"], pre["tiles_touched"], dk, s)
    ntx = (sc.cam.width + 15) // 16
    nty = (sc.cam.height + 15) // 16
    tmask = np.zeros(ntx * nty, np.uint8)
    tmask[np.random.default_rng(seed).permutation(ntx * nty)[: max(1, (ntx * nty) // tile_stride)]] = 1
    if tile_stride == 1:
        tmask[:] = 1
    fwd = O.render_fwd(sc.cam, pre, pl, rg, s, tile_mask=None if tile_stride == 1 else tmask)
    log(f"[{name}] oracle forward done ({time.time() - t0:.1f}s)")
    pixmask = np.repeat(np.repeat(tmask.reshape(nty, ntx), 16, 0), 16, 1)[: sc.cam.height, : sc.cam.width] > 0
    amb = (fwd["ambiguous"] & 3) > 0        # skip or stop within rounding: the image may differ there
    amb_grad = fwd["ambiguous"] > 0         # also the 0.99 clamp: the gradient may differ there

    # upstream gradient: given, or from the scene's loss on each side's own image
    if sc.dL_dimage is not None:
        dL = np.asarray(sc.dL_dimage, np.float64)
    else:
        _, dL = O.loss(sc.loss, fwd["image"], sc.target)
    dL = dL * (pixmask & ~amb_grad)[None]
    dL_dev = torch.from_numpy(dL.astype(np.float32)).cuda()
    g3 = r.backward(p, dL_dev)
    torch.cuda.synchronize()
    g["grad2d"] = r.grad2d.cpu().numpy()
    g["g3d"] = {k: v.cpu().numpy() for k, v in g3.items()}
    log(f"[{name}] gpu backward done ({time.time() - t0:.1f}s)")
    g2o = O.render_bwd(sc.cam, pre, pl, rg, dL, s, tile_mask=None if tile_stride == 1 else tmask, with_abs=True)
    g3o = O.preprocess_bwd(sc.cam, sc.sh_degree, sc.params(), pre["tiles_touched"], g2o, s)
    log(f"[{name}] oracle backward done ({time.time() - t0:.1f}s)")
    res = dict(scene=sc, gpu=g, pre=pre, pl=pl, rg=rg, fwd=fwd, amb=amb, pixmask=pixmask, tmask=tmask,
               g2o=g2o, g3o=g3o, dL=dL)
    _CACHE[name] = res
    del r
    torch.cuda.empty_cache()
    return res


CASES = {
    # name: (scene factory, tile_stride for the oracle's pixel walk)
    "tiny": (scenes.tiny, 1),
    "random_sh1": (lambda: scenes.random_small(21, n=300, width=61, height=45, sh_degree=1, scale_mu=-2.0), 1),
    "random_sh2": (lambda: scenes.random_small(22, n=500, width=100, height=77, sh_degree=2, scale_mu=-2.2), 1),
    # either side of the backward's two-waves-per-tile threshold: 33 x 31 = 1023 tiles, 32 x 32 = 1024
    "tiles1023": (lambda: scenes.random_small(23, n=4000, width=528, height=496, f=420.0, sh_degree=3), 1),
    "tiles1024": (lambda: scenes.random_small(24, n=4000, width=512, height=512, f=420.0, sh_degree=3), 1),
    "ball100k": (scenes.ball100k, 1),
    "clusters1m": (scenes.clusters1m, 1),
    "plane3m": (scenes.plane3m, 1),
}
