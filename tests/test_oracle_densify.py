"""Pins of the oracle's densification, pruning and opacity reset.

The rules come from the 3DGS training notes (notes.huajishe.fun), D.1-D.3
and E.1 steps 4-6; the numbers those passages leave out are parameters.
Each pin checks the oracle against something other than itself: hand-worked
decisions at the exact boundaries of every rule, the eigendecomposition of
Sigma (numpy eigh on a covariance built with scipy's rotation), invariants of
the output multiset, and scipy's logistic function.
"""
import json
import math
import os

import numpy as np
import pytest

PAGE = {k: v["value"] for k, v in json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                                               "page_constants.json"))).items()}
GROUPS = ("means", "log_scales", "quats", "opacity_logits", "sh")


def _sigma(ls, q):
    from scipy.spatial.transform import Rotation
    R = Rotation.from_quat([q[1], q[2], q[3], q[0]]).as_matrix()
    S = np.diag(np.exp(ls))
    return R @ S @ S @ R.T


def _params(rng, n, K=16):
    return dict(means=rng.normal(size=(n, 3)), log_scales=rng.normal(-2, 0.7, size=(n, 3)),
                quats=rng.normal(size=(n, 4)), opacity_logits=rng.normal(size=n), sh=rng.normal(size=(n, K, 3)))


def _moments(rng, p):
    return {k: (rng.normal(size=np.shape(v)), rng.uniform(0.1, 1, size=np.shape(v))) for k, v in p.items()}


def test_decisions_at_the_boundaries(oracle):
    O = oracle
    dp = O.DensifyParams(grad_threshold=0.25, prune_logit=-2.0, split_log_gap=0.5, split_shrink=math.log(1.6),
                         split_offset=1.0, clone_offset=0.125)
    rng = np.random.default_rng(1)
    p = _params(rng, 8)
    # (opacity logit, accum, count, log-scales) and the action each must take
    cases = [(-2.5, 9.0, 1, (0.0, 1.0, 0.0), 0),    # below the opacity floor: removed even though densified
             (-2.0, 0.0, 1, (0.0, 0.0, 0.0), 1),    # exactly at the floor: kept (the test is strict)
             (0.0, 5.0, 0, (0.0, 0.0, 0.0), 1),     # never seen in a view: no mean gradient, kept
             (0.0, 1.0, 4, (0.0, 0.5, 0.0), 3),     # mean gradient exactly at the threshold, gap exactly at it: split
             (0.0, 0.99, 4, (0.0, 2.0, 0.0), 1),    # mean gradient just below: kept
             (0.0, 3.0, 2, (0.1, 0.2, 0.3), 2),     # densified, nearly isotropic: cloned
             (0.0, 1.0, 1, (-1.0, 0.5, 0.5), 3),    # split; the longest axis is the first of the tie (axis 1)
             (-1.9, 1.0, 1, (0.0, 0.0, 0.0), 2)]    # densified, exactly isotropic: cloned
    for i, (lo, ac, ct, ls, _) in enumerate(cases):
        p["opacity_logits"][i] = lo
        p["log_scales"][i] = ls
    accum = np.array([c[1] for c in cases])
    count = np.array([c[2] for c in cases], np.int32)
    mom = _moments(rng, p)
    action, out, om = O.densify_apply(p, accum, count, dp, mom)
    assert action.tolist() == [c[4] for c in cases]
    # each Gaussian is replaced in order by 0, 1 or 2 outputs
    src = [1, 2, 3, 3, 4, 5, 5, 6, 6, 7, 7]
    fresh = [False, False, True, True, False, False, True, True, True, False, True]
    assert out["means"].shape[0] == len(src)
    for o, (i, f) in enumerate(zip(src, fresh)):
        assert np.array_equal(out["quats"][o], p["quats"][i])
        assert out["opacity_logits"][o] == p["opacity_logits"][i]
        assert np.array_equal(out["sh"][o], p["sh"][i])
        for k in GROUPS:
            for mv in (0, 1):
                want = np.zeros_like(mom[k][mv][i]) if f else mom[k][mv][i]
                assert np.array_equal(om[k][mv][o], want), (o, k, mv)
    # kept Gaussians and cloned originals are unchanged
    for o, i in ((0, 1), (1, 2), (4, 4), (5, 5), (9, 7)):
        assert np.array_equal(out["means"][o], p["means"][i])
        assert np.array_equal(out["log_scales"][o], p["log_scales"][i])
    # split children shrink every axis; the axis of case 6 is axis 1 (first maximum)
    for o, i in ((2, 3), (3, 3), (7, 6), (8, 6)):
        assert np.allclose(out["log_scales"][o], p["log_scales"][i] - np.float32(math.log(1.6)), rtol=0, atol=1e-15)
    d6 = out["means"][7] - p["means"][6]
    Sig = _sigma(p["log_scales"][6], p["quats"][6])
    w, V = np.linalg.eigh(Sig)
    # the two largest eigenvalues tie: the displacement lies in their plane, and is R's column 1
    from scipy.spatial.transform import Rotation
    q = p["quats"][6]
    e1 = Rotation.from_quat([q[1], q[2], q[3], q[0]]).as_matrix()[:, 1]
    assert np.allclose(d6, math.exp(0.5) * e1, rtol=0, atol=1e-12)


def test_split_follows_the_principal_axis(oracle):
    O = oracle
    rng = np.random.default_rng(2)
    n = 200
    p = _params(rng, n)
    dp = O.DensifyParams(grad_threshold=0.0, prune_logit=-1e30, split_log_gap=0.0, split_shrink=math.log(1.6),
                         split_offset=1.0, clone_offset=0.0)
    action, out, _ = O.densify_apply(p, np.ones(n), np.ones(n, np.int32), dp)
    assert (action == 3).all() and out["means"].shape[0] == 2 * n
    phi2 = math.exp(2 * float(np.float32(math.log(1.6))))
    for i in range(n):
        Sig = _sigma(p["log_scales"][i], p["quats"][i])
        w, V = np.linalg.eigh(Sig)
        a, b = out["means"][2 * i] - p["means"][i], out["means"][2 * i + 1] - p["means"][i]
        assert np.allclose(a, -b, rtol=0, atol=1e-15)                       # symmetric about the parent
        assert abs(np.linalg.norm(a) - math.sqrt(w[-1])) < 1e-12 * math.sqrt(w[-1])   # one sd of the long axis
        assert abs(abs(a @ V[:, -1]) - np.linalg.norm(a)) < 1e-12 * np.linalg.norm(a)  # along it
        for c in (2 * i, 2 * i + 1):                                          # each child: Sigma / phi^2
            Sc = _sigma(out["log_scales"][c], out["quats"][c])
            assert np.allclose(Sc * phi2, Sig, rtol=1e-12, atol=1e-14 * np.abs(Sig).max())


def test_clone_is_an_offset_copy(oracle):
    O = oracle
    rng = np.random.default_rng(3)
    n = 100
    p = _params(rng, n)
    dp = O.DensifyParams(grad_threshold=0.0, prune_logit=-1e30, split_log_gap=1e30, split_shrink=0.5,
                         split_offset=1.0, clone_offset=0.25)
    action, out, _ = O.densify_apply(p, np.ones(n), np.ones(n, np.int32), dp)
    assert (action == 2).all()
    for i in range(n):
        assert np.array_equal(out["means"][2 * i], p["means"][i])
        d = out["means"][2 * i + 1] - p["means"][i]
        w, V = np.linalg.eigh(_sigma(p["log_scales"][i], p["quats"][i]))
        assert abs(np.linalg.norm(d) - 0.25 * math.sqrt(w[-1])) < 1e-12
        assert abs(abs(d @ V[:, -1]) - np.linalg.norm(d)) < 1e-11
        for k in ("log_scales", "quats", "sh"):
            assert np.array_equal(out[k][2 * i + 1], p[k][i])


def test_output_multiset(oracle):
    """Removed rows vanish, kept rows appear once, densified rows twice."""
    O = oracle
    rng = np.random.default_rng(4)
    n = 2000
    p = _params(rng, n, K=9)
    accum = rng.exponential(1.0, n)
    count = rng.integers(0, 4, n).astype(np.int32)
    dp = O.DensifyParams(grad_threshold=0.8, prune_logit=-1.0, split_log_gap=0.9, split_shrink=math.log(1.6),
                         split_offset=1.0, clone_offset=0.1)
    action, out, _ = O.densify_apply(p, accum, count, dp)
    assert set(np.unique(action).tolist()) == {0, 1, 2, 3}
    mult = np.array([0, 1, 2, 2])[action]
    assert out["sh"].shape[0] == mult.sum()
    # the SH rows are distinct random vectors, so each output row names its source
    key = {p["sh"][i].tobytes(): i for i in range(n)}
    seen = np.zeros(n, np.int64)
    last = -1
    for r in out["sh"]:
        i = key[r.tobytes()]
        assert i >= last           # outputs follow the input order
        last = i
        seen[i] += 1
    assert np.array_equal(seen, mult)
    assert np.all(p["opacity_logits"][action == 0] < np.float32(-1.0))
    assert np.all(p["opacity_logits"][action != 0] >= np.float32(-1.0))


def test_opacity_reset_closed_form(oracle):
    from scipy.special import expit
    O = oracle
    x = np.linspace(-12, 12, 97)
    f = PAGE["opacity_reset_factor"]
    y = O.opacity_reset(x, f)
    assert np.allclose(expit(y), f * expit(x), rtol=1e-13, atol=0)
    # factor 1 is the identity, up to the cancellation in 1 - sigma (about 1e-16 e^|x|)
    assert np.all(np.abs(O.opacity_reset(x, 1.0) - x) <= 1e-15 * np.exp(np.abs(x)) + 1e-15)
    assert np.all(np.diff(y) > 0)
