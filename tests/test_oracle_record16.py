"""Pins of the oracle's 16-bit splat record (orc_round_binary16, orc_record16).

The record stores the 2D mean in float32 and the conic (through its scaled
Cholesky factor), the opacity and the colour in IEEE 754 binary16 (Gaussian
Splatting backward CUDA page (lshu.cn), section 5: some intermediates kept as
16-bit floats; section 7: FP16 on the rendering path, FP32 gradient sums).

- The rounding is checked against numpy's float16 conversion, an independent
  implementation of the same IEEE definition, on every finite binary16 value,
  on every midpoint between neighbours (the ties), just either side of them,
  across the subnormal range and at overflow.
- The record's conic is pinned by a closed form (covariances whose Cholesky
  factor is exactly representable come back unchanged, and an axis-aligned
  covariance keeps B = 0) and by the element-wise rounding bound that the
  factor form implies.
- The cost of the relaxation, the change of the oracle's own image when it
  reads the rounded record, is reported and held to a first-order bound.
"""
import math

import numpy as np
import pytest

from differentiable_gaussian_splatting_dgs_amd import scenes

U16 = 2.0 ** -11          # unit roundoff of binary16
U = U16 + 2.0 ** -24      # rounding to float32 first, then to binary16


def _finite_f16():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    h = codes.view(np.float16)
    return np.unique(h[np.isfinite(h)].astype(np.float64))


def test_round_binary16_matches_numpy(oracle):
    vals = _finite_f16()                                  # every finite binary16 value, sorted
    mids = 0.5 * (vals[:-1] + vals[1:])                   # every tie (exact in double)
    nudge = np.concatenate([np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)])
    rng = np.random.default_rng(7)
    rand = np.exp(rng.uniform(np.log(1e-9), np.log(7e4), 200000)) * rng.choice([-1.0, 1.0], 200000)
    edge = np.array([65504.0, 65519.999, 65520.0, 65536.0, 1e6, -65520.0, 2.0 ** -24, 2.0 ** -25,
                     3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 0.0, -0.0])
    x = np.concatenate([vals, mids, nudge, rand, edge])
    got = oracle.round_binary16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    # ties go to the even significand: 1 + 2^-11 lies between 1 and 1 + 2^-10
    assert oracle.round_binary16(np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11])).tolist() == [1.0, 1 + 2.0 ** -9]
    assert np.isnan(oracle.round_binary16(np.array([np.nan]))[0])


def _pre_from_cov(cov, uv=None, opacity=None, rgb=None):
    n = cov.shape[0]
    return dict(uv=np.zeros((n, 2)) if uv is None else uv, cov2d=cov,
                opacity=np.full(n, 0.5) if opacity is None else opacity,
                rgb=np.full((n, 3), 0.25) if rgb is None else rgb, valid=np.ones(n, np.uint8))


def test_record16_exact_factor_round_trips(oracle):
    """A conic whose scaled Cholesky factor is made of binary16 numbers comes back as itself."""
    s2 = 0.5 / math.log(2.0)
    Ls = [(0.75, -0.125, 0.5), (1.5, 0.0, 0.046875), (0.0625, 0.25, 0.375), (0.5, -0.5, 0.5)]
    cov, conic = [], []
    for l00, l10, l11 in Ls:
        A = np.array([[l00 * l00, l00 * l10], [l00 * l10, l10 * l10 + l11 * l11]]) / s2
        S = np.linalg.inv(A)
        cov.append([S[0, 0], S[0, 1], S[1, 1]])
        conic.append([A[0, 0], A[0, 1], A[1, 1]])
    r = oracle.record16(_pre_from_cov(np.array(cov)))
    np.testing.assert_allclose(r["conic"], np.array(conic), rtol=1e-13, atol=0)
    # axis-aligned covariance: the factor has L10 = 0, so B stays exactly 0
    r = oracle.record16(_pre_from_cov(np.array([[4.0, 0.0, 9.0], [0.3, 0.0, 0.3]])))
    assert np.all(r["conic"][:, 1] == 0.0)
    np.testing.assert_allclose(r["conic"][:, 0], 1 / np.array([4.0, 0.3]), rtol=2 * U)
    np.testing.assert_allclose(r["conic"][:, 2], 1 / np.array([9.0, 0.3]), rtol=2 * U)


def test_record16_values_and_bounds(oracle):
    """Opacity and colour are float32-then-binary16 roundings; the conic is within
    the factor form's rounding bound, element by element; the mean is float32."""
    rng = np.random.default_rng(11)
    n = 4000
    # 2D covariances with eigenvalues 0.3..2000 px^2 at random angles (factor entries in binary16's normal range)
    lam = np.exp(rng.uniform(np.log(0.3), np.log(2000.0), (n, 2)))
    th = rng.uniform(0, np.pi, n)
    c, s = np.cos(th), np.sin(th)
    a = lam[:, 0] * c * c + lam[:, 1] * s * s
    b = (lam[:, 0] - lam[:, 1]) * c * s
    d = lam[:, 0] * s * s + lam[:, 1] * c * c
    cov = np.stack([a, b, d], 1)
    uv = rng.uniform(0, 3840, (n, 2))
    op = rng.uniform(1 / 255, 0.999, n)
    rgb = rng.uniform(0, 1.5, (n, 3))
    r = oracle.record16(_pre_from_cov(cov, uv, op, rgb))
    assert np.array_equal(r["uv"], uv.astype(np.float32).astype(np.float64))
    assert np.array_equal(r["opacity"], op.astype(np.float32).astype(np.float16).astype(np.float64))
    assert np.array_equal(r["rgb"], rgb.astype(np.float32).astype(np.float16).astype(np.float64))
    det = a * d - b * b
    A, B, C = d / det, -b / det, a / det
    s2 = 0.5 / math.log(2.0)
    l00, l10, l11 = np.sqrt(A * s2), B * np.sqrt(s2 / A), np.sqrt(s2 / d)
    # each stored factor entry is within U |l| + 2^-25 of l (2^-25: half the subnormal spacing)
    e00, e10, e11 = (U * np.abs(x) + 2.0 ** -25 for x in (l00, l10, l11))
    a00, a10, a11 = np.abs(l00), np.abs(l10), np.abs(l11)
    slack = 1 + 1e-9
    assert np.all(np.abs(r["conic"][:, 0] - A) <= slack * ((a00 + e00) ** 2 - a00 ** 2) / s2)
    assert np.all(np.abs(r["conic"][:, 1] - B) <= slack * ((a00 + e00) * (a10 + e10) - a00 * a10) / s2)
    assert np.all(np.abs(r["conic"][:, 2] - C) <=
                  slack * ((a10 + e10) ** 2 - a10 ** 2 + (a11 + e11) ** 2 - a11 ** 2) / s2)
    # and the rounding does happen: the conic is not the exact one
    assert np.mean(r["conic"][:, 0] != A) > 0.9
    # culled Gaussians have a zero record
    pre = _pre_from_cov(cov[:3], uv[:3], op[:3], rgb[:3])
    pre["valid"] = np.array([1, 0, 1], np.uint8)
    r = oracle.record16(pre)
    assert np.all(r["conic"][1] == 0) and r["opacity"][1] == 0 and np.all(r["uv"][1] == 0)


@pytest.mark.parametrize("which", ["tiny", "ball"])
def test_record16_image_change_is_bounded(oracle, which):
    """The oracle's image from the rounded record against its full-precision image.

    With the element-wise conic bound above (relative tol on A, B and C away from
    binary16's subnormal range, which these scenes' factors do not reach) and |B| <
    sqrt(A C), a pair's exponent moves by |d power| <= tol (1 + kappa) |power|, kappa the
    conic's condition number, and |power| <= ln(opacity / alpha_min) <= ln 255 for every
    blended pair.  So alpha moves by a relative amount of at most e = u + tol (1 + kappa)
    ln 255 (first order; opacity rounding u), and a pixel whose skip and stop decisions
    do not change moves by at most (e + u) times the largest colour, since
    sum_k T_k alpha_k <= 1 (colour rounding u).  Pixels where a decision changes are
    counted and must be rare."""
    sc = scenes.tiny() if which == "tiny" else scenes.ball100k(n=4000, size=160, f=220.0)
    s = oracle.Settings()
    params = {k: np.asarray(v, np.float64) for k, v in sc.params().items()}
    pre = oracle.preprocess(sc.cam, sc.sh_degree, params, s)
    pl, rg = oracle.bin_gaussians(sc.cam, pre["rect"], pre["tiles_touched"], oracle.depth_key(pre["depth"]), s)
    full = oracle.render_fwd(sc.cam, pre, pl, rg, s)
    half = oracle.render_fwd(sc.cam, oracle.record16(pre), pl, rg, s)
    v = pre["valid"] != 0
    a, b, c = pre["cov2d"][v].T
    tr, det = a + c, a * c - b * b
    disc = np.sqrt(np.maximum(tr * tr / 4 - det, 0))
    kappa = float(np.max((tr / 2 + disc) / (tr / 2 - disc)))
    tol = 2 * U + U * U
    e = U + tol * (1 + kappa) * math.log(255.0)
    cmax = float(pre["rgb"].max())
    bound = 1.01 * (e + U) * cmax
    same = half["hash"] == full["hash"]
    err = np.abs(half["image"] - full["image"]).max(axis=0)
    print(f"{which}: kappa_max {kappa:.1f}; max |image(record16) - image| on {same.mean():.4f} of pixels "
          f"{err[same].max():.3e} (bound {bound:.3e}); all pixels {err.max():.3e}")
    assert err[same].max() <= bound
    assert err[same].max() > 0
    assert same.mean() >= 0.97
