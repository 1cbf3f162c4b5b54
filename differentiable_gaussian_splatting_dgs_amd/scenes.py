"""Seeded synthetic scenes for the tile rasterizer.

This module only draws random numbers. It holds none of the rasterizer's
arithmetic (no projection, no spherical-harmonic evaluation, no blending), so
the HIP path and the CPU oracle can both consume its output without sharing
any of the method's code.

Every scene is drawn from ``numpy.random.default_rng(seed)`` in float64 with a
fixed draw order, then cast to float32. The camera is the identity world to
camera transform, with the principal point at the image centre.

Parameter layout (what a rasterizer user hands over):

* ``means``           [N, 3]  world-space centres
* ``log_scales``      [N, 3]  per-axis log standard deviations
* ``quats``           [N, 4]  rotation quaternions (w, x, y, z), unit length
* ``opacity_logits``  [N]     pre-sigmoid opacity
* ``sh``              [N, K, 3] spherical-harmonic colour coefficients,
                               K = (degree + 1)^2, index l*l + l + m

The five named workloads follow the rasterizer configurations of the method
(tiny 256-Gaussian view, 100k at 800x800, 1M at 1080p, 3M at 4K, and a
training step on the 1M scene).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

SQRT_PI = math.sqrt(math.pi)


@dataclasses.dataclass
class Camera:
    width: int
    height: int
    fx: float
    fy: float
    cx: float
    cy: float
    R: np.ndarray  # [3,3] world -> camera rotation, row-major
    t: np.ndarray  # [3] world -> camera translation

    @staticmethod
    def identity(width, height, f):
        return Camera(width, height, float(f), float(f), width / 2.0, height / 2.0,
                      np.eye(3), np.zeros(3))


@dataclasses.dataclass
class Scene:
    name: str
    cam: Camera
    sh_degree: int
    means: np.ndarray
    log_scales: np.ndarray
    quats: np.ndarray
    opacity_logits: np.ndarray
    sh: np.ndarray
    # exactly one of these drives the backward pass
    dL_dimage: Optional[np.ndarray] = None      # [3, H, W] upstream gradient
    target: Optional[np.ndarray] = None         # [3, H, W] loss target
    loss: Optional[str] = None                  # "l1" | "l2" | None
    adam_lr: Optional[dict] = None

    @property
    def n(self):
        return int(self.means.shape[0])

    def params(self):
        return dict(means=self.means, log_scales=self.log_scales, quats=self.quats,
                    opacity_logits=self.opacity_logits, sh=self.sh)


def _unit_rows(rng, n, d):
    q = rng.standard_normal((n, d))
    return q / np.linalg.norm(q, axis=1, keepdims=True)


def _f32(*arrs):
    return [np.ascontiguousarray(a, dtype=np.float32) for a in arrs]


def _sh3(rng, n):
    """SH degree-3 coefficients: DC uniform on [0,1], higher bands N(0, 0.05)."""
    sh = np.empty((n, 16, 3))
    sh[:, 0, :] = rng.uniform(0.0, 1.0, (n, 3))
    sh[:, 1:, :] = rng.normal(0.0, 0.05, (n, 15, 3))
    return sh


def _in_view_xy(rng, z, cam):
    """x, y uniform inside the view frustum at depth z (identity camera)."""
    x = rng.uniform(-cam.cx / cam.fx, (cam.width - cam.cx) / cam.fx, z.shape) * z
    y = rng.uniform(-cam.cy / cam.fy, (cam.height - cam.cy) / cam.fy, z.shape) * z
    return x, y


def tiny(seed=0, n=256, size=64, f=64.0):
    """256 Gaussians, 64x64 view, SH degree 0, colours uniform on [0, 1].

    With SH degree 0 the colour is the DC coefficient times the degree-0 basis
    constant plus one half, so a DC coefficient uniform on [-sqrt(pi), sqrt(pi)]
    gives colours uniform on [0, 1].
    """
    rng = np.random.default_rng(seed)
    cam = Camera.identity(size, size, f)
    means = np.column_stack([rng.uniform(-1, 1, n), rng.uniform(-1, 1, n), rng.uniform(2, 4, n)])
    log_scales = rng.normal(-2.5, 0.4, (n, 3))
    quats = _unit_rows(rng, n, 4)
    opac = rng.normal(0.0, 1.0, n)
    sh = rng.uniform(-SQRT_PI, SQRT_PI, (n, 1, 3))
    dL = rng.standard_normal((3, size, size))
    m, s, q, o, c, g = _f32(means, log_scales, quats, opac, sh, dL)
    return Scene("tiny", cam, 0, m, s, q, o, c, dL_dimage=g)


def ball100k(seed=1, n=100_000, size=800, f=1100.0):
    """100k Gaussians uniform in a radius-1.5 ball centred 4 units ahead, L2 loss."""
    rng = np.random.default_rng(seed)
    cam = Camera.identity(size, size, f)
    d = _unit_rows(rng, n, 3)
    r = 1.5 * rng.uniform(0, 1, n) ** (1.0 / 3.0)
    means = d * r[:, None] + np.array([0.0, 0.0, 4.0])
    log_scales = rng.normal(-4.0, 0.5, (n, 3))
    quats = _unit_rows(rng, n, 4)
    opac = rng.normal(0.0, 1.5, n)
    sh = _sh3(rng, n)
    target = rng.uniform(0, 1, (3, size, size))
    m, s, q, o, c, t = _f32(means, log_scales, quats, opac, sh, target)
    return Scene("ball100k", cam, 3, m, s, q, o, c, target=t, loss="l2")


def _clusters_shell(rng, n, cam, n_clusters=64, frac_shell=0.3):
    n_shell = int(round(frac_shell * n))
    n_cl = n - n_shell
    cz = rng.uniform(3.0, 9.0, n_clusters)
    cx, cy = _in_view_xy(rng, cz, cam)
    centres = np.column_stack([cx, cy, cz])
    # random orientation per cluster from the QR factor of a Gaussian matrix
    rots = np.empty((n_clusters, 3, 3))
    for k in range(n_clusters):
        qm, rm = np.linalg.qr(rng.standard_normal((3, 3)))
        rots[k] = qm * np.sign(np.diag(rm))[None, :]
    stds = rng.uniform(0.05, 0.6, (n_clusters, 3))
    labels = rng.integers(0, n_clusters, n_cl)
    local = rng.standard_normal((n_cl, 3)) * stds[labels]
    pts_cl = np.einsum("nij,nj->ni", rots[labels], local) + centres[labels]
    d = _unit_rows(rng, n_shell, 3)
    rad = 2.5 + rng.normal(0.0, 0.03, n_shell)
    pts_sh = d * rad[:, None] + np.array([0.0, 0.0, 6.0])
    return np.concatenate([pts_cl, pts_sh], axis=0)


def clusters1m(seed=2, n=1_000_000, width=1920, height=1080, f=1500.0, training=False):
    """1M Gaussians at 1080p: 64 anisotropic clusters plus 30% on a noisy shell.

    With ``training`` the last draw is an L1 target instead of dL/dpixel and
    the Adam learning rates of the training step are attached.
    """
    rng = np.random.default_rng(seed)
    cam = Camera.identity(width, height, f)
    means = _clusters_shell(rng, n, cam)
    log_scales = rng.normal(-4.5, 0.6, (n, 3))
    quats = _unit_rows(rng, n, 4)
    opac = rng.normal(0.5, 1.5, n)
    sh = _sh3(rng, n)
    last = rng.standard_normal((3, height, width)) if not training else rng.uniform(0, 1, (3, height, width))
    m, s, q, o, c, g = _f32(means, log_scales, quats, opac, sh, last)
    if training:
        return Scene("train1m", cam, 3, m, s, q, o, c, target=g, loss="l1", adam_lr=dict(ADAM_LR))
    return Scene("clusters1m", cam, 3, m, s, q, o, c, dL_dimage=g)


def plane3m(seed=3, n=3_000_000, width=3840, height=2160, f=3000.0):
    """3M Gaussians at 4K: half on a thin tilted plane at z=8, half uniform in the frustum z in [1, 20]."""
    rng = np.random.default_rng(seed)
    cam = Camera.identity(width, height, f)
    n_pl = n // 2
    n_fr = n - n_pl
    hx = 1.1 * 8.0 * (width / 2.0) / f
    hy = 1.1 * 8.0 * (height / 2.0) / f
    px = rng.uniform(-hx, hx, n_pl)
    py = rng.uniform(-hy, hy, n_pl)
    pz = 8.0 + 0.1 * px + rng.normal(0.0, 0.01, n_pl)
    fz = rng.uniform(1.0, 20.0, n_fr)
    fx_, fy_ = _in_view_xy(rng, fz, cam)
    means = np.concatenate([np.column_stack([px, py, pz]), np.column_stack([fx_, fy_, fz])])
    log_scales = rng.normal(-5.0, 0.7, (n, 3))
    quats = _unit_rows(rng, n, 4)
    opac = rng.normal(1.0, 1.0, n)
    sh = _sh3(rng, n)
    dL = rng.standard_normal((3, height, width))
    m, s, q, o, c, g = _f32(means, log_scales, quats, opac, sh, dL)
    return Scene("plane3m", cam, 3, m, s, q, o, c, dL_dimage=g)


# Adam learning rates of the training step, per parameter group.
ADAM_LR = dict(means=1.6e-4, log_scales=5e-3, quats=1e-3, opacity_logits=5e-2,
               sh_dc=2.5e-3, sh_rest=1.25e-4)


def training1m(seed=2, **kw):
    return clusters1m(seed=seed, training=True, **kw)


WORKLOADS = {
    "tiny": tiny,
    "ball100k": ball100k,
    "clusters1m": clusters1m,
    "plane3m": plane3m,
    "train1m": training1m,
}


def make(name, **kw):
    return WORKLOADS[name](**kw)


def random_small(seed, n=48, width=48, height=40, f=50.0, sh_degree=3, scale_mu=-2.3):
    """A small random scene with an arbitrary SH degree, for property tests."""
    rng = np.random.default_rng(seed)
    cam = Camera.identity(width, height, f)
    means = np.column_stack([rng.uniform(-0.8, 0.8, n), rng.uniform(-0.7, 0.7, n), rng.uniform(1.8, 3.5, n)])
    log_scales = rng.normal(scale_mu, 0.4, (n, 3))
    quats = _unit_rows(rng, n, 4) * rng.uniform(0.5, 2.0, (n, 1))   # deliberately not unit
    opac = rng.normal(0.3, 1.2, n)
    k = (sh_degree + 1) ** 2
    sh = np.empty((n, k, 3))
    sh[:, 0, :] = rng.uniform(-1.0, 1.0, (n, 3))
    if k > 1:
        sh[:, 1:, :] = rng.normal(0.0, 0.3, (n, k - 1, 3))
    dL = rng.standard_normal((3, height, width))
    m, s, q, o, c, g = _f32(means, log_scales, quats, opac, sh, dL)
    return Scene(f"random{seed}", cam, sh_degree, m, s, q, o, c, dL_dimage=g)


def densify_case(seed, n, sh_degree=3, with_moments=True):
    """Inputs of a densification step: a Gaussian set after some training views.

    Parameters as in the scenes above (log-scales spread so both isotropic and
    elongated Gaussians occur), Adam moments, and the densification statistic:
    count = views that saw the Gaussian (0-4), accum = a sum of per-view gradient
    norms (exponential, so a tail of large mean gradients exists).  Returns a dict
    with the five groups, 'exp_avg' / 'exp_avg_sq' (dicts) or None, 'densify_accum'
    float32 [n] and 'densify_count' int32 [n].
    """
    rng = np.random.default_rng(seed)
    K = (sh_degree + 1) ** 2
    means = rng.normal(0.0, 1.0, (n, 3))
    log_scales = rng.normal(-3.5, 0.3, (n, 1)) + rng.normal(0.0, 0.6, (n, 3))
    quats = _unit_rows(rng, n, 4)
    opacity = rng.normal(-1.0, 2.5, n)
    sh = rng.normal(0.0, 0.3, (n, K, 3))
    count = rng.integers(0, 5, n)
    accum = rng.exponential(1.0, n) * count
    out = dict(means=means, log_scales=log_scales, quats=quats, opacity_logits=opacity, sh=sh)
    out = {k: np.ascontiguousarray(v, dtype=np.float32) for k, v in out.items()}
    out["densify_accum"] = accum.astype(np.float32)
    out["densify_count"] = count.astype(np.int32)
    out["exp_avg"] = out["exp_avg_sq"] = None
    if with_moments:
        out["exp_avg"] = {k: rng.normal(0.0, 1e-3, np.shape(out[k])).astype(np.float32)
                          for k in ("means", "log_scales", "quats", "opacity_logits", "sh")}
        out["exp_avg_sq"] = {k: rng.uniform(0.0, 1e-5, np.shape(out[k])).astype(np.float32)
                             for k in ("means", "log_scales", "quats", "opacity_logits", "sh")}
    return out


def orbit_cameras(cam, views, centre, step_deg=8.0):
    """A batch of `views` cameras with cam's intrinsics on a horizontal arc around
    `centre`: view v is cam turned by (v - (views - 1) / 2) step_deg about the
    vertical axis through centre, so every view looks at the scene the way cam
    does (for an odd count the middle view is cam itself)."""
    c = np.asarray(centre, dtype=np.float64)
    R0, t0 = np.asarray(cam.R, np.float64), np.asarray(cam.t, np.float64)
    pos0 = -R0.T @ t0  # camera centre in world coordinates
    out = []
    for v in range(views):
        th = math.radians((v - (views - 1) / 2.0) * step_deg)
        Ry = np.array([[math.cos(th), 0.0, math.sin(th)], [0.0, 1.0, 0.0], [-math.sin(th), 0.0, math.cos(th)]])
        pos = c + Ry @ (pos0 - c)
        R = R0 @ Ry.T
        out.append(Camera(cam.width, cam.height, cam.fx, cam.fy, cam.cx, cam.cy, R, -R @ pos))
    return out
