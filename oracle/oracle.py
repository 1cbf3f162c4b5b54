"""ctypes harness around the C oracle (gs_oracle.c).

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path (the HIP library
and its binding) never does, and this module imports nothing from it.

Everything is float64.  Scene parameters arrive as float32 arrays and are
widened once; all arithmetic happens in the C oracle in double precision.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gs_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force=False):
    """Compile the oracle with gcc (plain C99, no fused multiply-add contraction)."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    subprocess.check_call(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                           "-shared", "-Wall", "-o", tmp, SRC, "-lm"])
    os.replace(tmp, LIB)
    return LIB


_lib = None


class _Cam(C.Structure):
    _fields_ = [("fx", C.c_double), ("fy", C.c_double), ("cx", C.c_double), ("cy", C.c_double),
                ("width", C.c_int32), ("height", C.c_int32), ("R", C.c_double * 9), ("t", C.c_double * 3)]


class _Set(C.Structure):
    _fields_ = [("near_z", C.c_double), ("alpha_min", C.c_double), ("alpha_max", C.c_double),
                ("T_min", C.c_double), ("dilation", C.c_double), ("bg", C.c_double * 3), ("tile", C.c_int32)]


@dataclass
class Settings:
    near_z: float = 0.2
    alpha_min: float = 1.0 / 255.0
    alpha_max: float = 0.99
    T_min: float = 1e-4
    dilation: float = 0.3
    bg: tuple = (0.0, 0.0, 0.0)
    tile: int = 16


def lib():
    global _lib
    if _lib is None:
        build()
        _lib = C.CDLL(LIB)
        _lib.orc_bin.restype = C.c_int64
        _lib.orc_loss.restype = C.c_double
    return _lib


def _p(a, ctype=C.c_double):
    return a.ctypes.data_as(C.POINTER(ctype))


def _d(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def cam_struct(cam):
    c = _Cam()
    c.fx, c.fy, c.cx, c.cy = cam.fx, cam.fy, cam.cx, cam.cy
    c.width, c.height = cam.width, cam.height
    for i, v in enumerate(np.asarray(cam.R, dtype=np.float64).reshape(-1)):
        c.R[i] = v
    for i, v in enumerate(np.asarray(cam.t, dtype=np.float64).reshape(-1)):
        c.t[i] = v
    return c


def set_struct(s: Settings):
    o = _Set()
    o.near_z, o.alpha_min, o.alpha_max, o.T_min, o.dilation = s.near_z, s.alpha_min, s.alpha_max, s.T_min, s.dilation
    for i in range(3):
        o.bg[i] = s.bg[i]
    o.tile = s.tile
    return o


def sh_basis(deg, d):
    """Real SH values Y[K] and their gradients dY[K,3] at direction d (oracle routine)."""
    K = (deg + 1) ** 2
    Y = np.zeros(16)
    g = np.zeros(48)
    lib().orc_sh_basis(C.c_int(deg), _p(_d(d)), _p(Y), _p(g))
    return Y[:K].copy(), g.reshape(16, 3)[:K].copy()


def quat_to_rot(q):
    R = np.zeros(9)
    lib().orc_quat_to_rot(_p(_d(q)), _p(R))
    return R.reshape(3, 3)


def preprocess(cam, deg, params, s: Settings = None):
    s = s or Settings()
    means, ls, qs, op, sh = (_d(params[k]) for k in ("means", "log_scales", "quats", "opacity_logits", "sh"))
    N = means.shape[0]
    out = dict(uv=np.zeros((N, 2)), depth=np.zeros(N), conic=np.zeros((N, 3)), cov2d=np.zeros((N, 3)),
               opacity=np.zeros(N), rgb=np.zeros((N, 3)), clamp=np.zeros(N, np.uint8), ext=np.zeros((N, 2)),
               rect=np.zeros((N, 4), np.int32), tiles_touched=np.zeros(N, np.int32), valid=np.zeros(N, np.uint8))
    lib().orc_preprocess(C.byref(cam_struct(cam)), C.byref(set_struct(s)), C.c_int(N), C.c_int(deg),
                         _p(means), _p(ls), _p(qs), _p(op), _p(sh),
                         _p(out["uv"]), _p(out["depth"]), _p(out["conic"]), _p(out["cov2d"]), _p(out["opacity"]),
                         _p(out["rgb"]), _p(out["clamp"], C.c_uint8), _p(out["ext"]), _p(out["rect"], C.c_int),
                         _p(out["tiles_touched"], C.c_int), _p(out["valid"], C.c_uint8))
    return out


def depth_key(depth):
    """The sort key is the float32 depth (ties broken by Gaussian index)."""
    return np.asarray(depth, dtype=np.float32).astype(np.float64)


def bin_gaussians(cam, rect, tiles_touched, depth_k, s: Settings = None):
    s = s or Settings()
    rect = np.ascontiguousarray(rect, dtype=np.int32)
    tt = np.ascontiguousarray(tiles_touched, dtype=np.int32)
    dk = _d(depth_k)
    N = rect.shape[0]
    ntx = (cam.width + s.tile - 1) // s.tile
    nty = (cam.height + s.tile - 1) // s.tile
    ranges = np.zeros((ntx * nty, 2), np.int64)
    cap = int(tt.astype(np.int64).sum())
    pl = np.zeros(max(cap, 1), np.int32)
    K = lib().orc_bin(C.c_int(N), C.c_int(cam.width), C.c_int(cam.height), C.c_int(s.tile),
                      _p(rect, C.c_int), _p(tt, C.c_int), _p(dk), _p(pl, C.c_int), C.c_int64(cap),
                      _p(ranges, C.c_int64))
    assert K == cap
    return pl[:K].copy(), ranges


def global_list(valid, depth_k):
    """All non-culled Gaussians in (depth key, index) order: the brute-force list."""
    idx = np.nonzero(np.asarray(valid) != 0)[0]
    order = np.lexsort((idx, np.asarray(depth_k)[idx]))
    pl = idx[order].astype(np.int32)
    return pl, np.array([[0, len(pl)]], np.int64)


def _tmask(tile_mask):
    if tile_mask is None:
        return None, None
    m = np.ascontiguousarray(tile_mask, dtype=np.uint8)
    return m, _p(m, C.c_uint8)


def render_fwd(cam, pre, point_list, ranges, s: Settings = None, brute=False, amb_rel=1e-5, tile_mask=None):
    s = s or Settings()
    tm, tmp = _tmask(tile_mask)
    W, H = cam.width, cam.height
    out = dict(image=np.zeros((3, H, W)), final_T=np.zeros((H, W)), n_contrib=np.zeros((H, W), np.int32),
               wsum=np.zeros((H, W)), ambiguous=np.zeros((H, W), np.uint8), hash=np.zeros((H, W), np.uint64),
               counts=np.zeros(3, np.int64), evaluated=np.zeros((H, W), np.int64))
    pl = np.ascontiguousarray(point_list, dtype=np.int32)
    rg = np.ascontiguousarray(ranges, dtype=np.int64)
    lib().orc_render_fwd(C.byref(cam_struct(cam)), C.byref(set_struct(s)), C.c_int(1 if brute else 0),
                         _p(pl, C.c_int), _p(rg, C.c_int64), _p(_d(pre["uv"])), _p(_d(pre["conic"])),
                         _p(_d(pre["opacity"])), _p(_d(pre["rgb"])), _p(out["image"]), _p(out["final_T"]),
                         _p(out["n_contrib"], C.c_int), _p(out["wsum"]), _p(out["ambiguous"], C.c_uint8),
                         C.c_double(amb_rel), _p(out["hash"], C.c_uint64), _p(out["counts"], C.c_int64), tmp,
                         _p(out["evaluated"], C.c_int64))
    return out


def render_bwd(cam, pre, point_list, ranges, dL_dimage, s: Settings = None, brute=False, tile_mask=None,
               with_abs=False):
    """2D gradients; with_abs also returns abs [N, 9]: per Gaussian and component (du, dv, dA, dB,
    dC, dopacity, dr, dg, db) the sum of the absolute sizes of the terms added, a scale for the
    rounding error of a float32 evaluation of the same sums."""
    s = s or Settings()
    tm, tmp = _tmask(tile_mask)
    N = pre["uv"].shape[0]
    out = dict(dxy=np.zeros((N, 2)), dconic=np.zeros((N, 3)), dopacity=np.zeros(N), drgb=np.zeros((N, 3)))
    if with_abs:
        out["abs"] = np.zeros((N, 9))
    pl = np.ascontiguousarray(point_list, dtype=np.int32)
    rg = np.ascontiguousarray(ranges, dtype=np.int64)
    lib().orc_render_bwd(C.byref(cam_struct(cam)), C.byref(set_struct(s)), C.c_int(1 if brute else 0),
                         _p(pl, C.c_int), _p(rg, C.c_int64), _p(_d(pre["uv"])), _p(_d(pre["conic"])),
                         _p(_d(pre["opacity"])), _p(_d(pre["rgb"])), _p(_d(dL_dimage)),
                         _p(out["dxy"]), _p(out["dconic"]), _p(out["dopacity"]), _p(out["drgb"]), C.c_int(N), tmp,
                         _p(out["abs"]) if with_abs else None)
    return out


def preprocess_bwd(cam, deg, params, tiles_touched, g2d, s: Settings = None):
    s = s or Settings()
    means, ls, qs, op, sh = (_d(params[k]) for k in ("means", "log_scales", "quats", "opacity_logits", "sh"))
    N = means.shape[0]
    K = (deg + 1) ** 2
    out = dict(means=np.zeros((N, 3)), log_scales=np.zeros((N, 3)), quats=np.zeros((N, 4)),
               opacity_logits=np.zeros(N), sh=np.zeros((N, K, 3)))
    tt = np.ascontiguousarray(tiles_touched, dtype=np.int32)
    lib().orc_preprocess_bwd(C.byref(cam_struct(cam)), C.byref(set_struct(s)), C.c_int(N), C.c_int(deg),
                             _p(means), _p(ls), _p(qs), _p(op), _p(sh), _p(tt, C.c_int),
                             _p(_d(g2d["dxy"])), _p(_d(g2d["dconic"])), _p(_d(g2d["dopacity"])),
                             _p(_d(g2d["drgb"])), _p(out["means"]), _p(out["log_scales"]), _p(out["quats"]),
                             _p(out["opacity_logits"]), _p(out["sh"]))
    return out


def loss(mode, pred, target):
    """mode 'l1' or 'l2'; returns (L, dL/dpred)."""
    pred = _d(pred)
    g = np.zeros_like(pred)
    L = lib().orc_loss(C.c_int(1 if mode == "l1" else 2), C.c_int64(pred.size), _p(pred), _p(_d(target)), _p(g))
    return L, g


def densify(tiles_touched, dxy, accum, count):
    accum = _d(accum).copy()
    count = np.ascontiguousarray(count, dtype=np.int32).copy()
    lib().orc_densify(C.c_int(len(accum)), _p(np.ascontiguousarray(tiles_touched, dtype=np.int32), C.c_int),
                      _p(_d(dxy)), _p(accum), _p(count, C.c_int))
    return accum, count


def adam(p, g, m, v, lr, step, b1=0.9, b2=0.999, eps=1e-8):
    p, m, v = _d(p).copy(), _d(m).copy(), _d(v).copy()
    lib().orc_adam(C.c_int64(p.size), _p(p), _p(_d(g)), _p(m), _p(v), C.c_double(lr), C.c_double(b1),
                   C.c_double(b2), C.c_double(eps), C.c_int(step))
    return p, m, v


def quat_renorm(q):
    q = _d(q).copy()
    lib().orc_quat_renorm(C.c_int(q.shape[0]), _p(q))
    return q


def render(cam, deg, params, s: Settings = None, dL_dimage=None, brute=False, amb_rel=1e-5, backward=True):
    """Full oracle pipeline: preprocess, bin, forward and (optionally) backward."""
    s = s or Settings()
    pre = preprocess(cam, deg, params, s)
    dk = depth_key(pre["depth"])
    if brute:
        pl, rg = global_list(pre["valid"], dk)
    else:
        pl, rg = bin_gaussians(cam, pre["rect"], pre["tiles_touched"], dk, s)
    fwd = render_fwd(cam, pre, pl, rg, s, brute=brute, amb_rel=amb_rel)
    res = dict(pre=pre, point_list=pl, ranges=rg, **fwd)
    if backward and dL_dimage is not None:
        g2d = render_bwd(cam, pre, pl, rg, dL_dimage, s, brute=brute)
        g3d = preprocess_bwd(cam, deg, params, pre["tiles_touched"], g2d, s)
        res["g2d"] = g2d
        res["g3d"] = g3d
    return res


def render_views(cams, deg, params, dL_dimages, s: Settings = None, mask_ambiguous=True):
    """A batch of views ([P4] E.1 steps 1-2: render every view of the batch; the
    batch's loss is the sum of the views' losses, so its gradient is the sum of
    the views' gradients).  dL_dimages [views, 3, H, W].  With mask_ambiguous the
    upstream gradient is zeroed at each view's ambiguous pixels (as in the
    single-view parity tests).  Returns the per-view forward results and the 3D
    gradients summed over the views."""
    s = s or Settings()
    per_view, total = [], None
    for cam, dL in zip(cams, dL_dimages):
        o = render(cam, deg, params, s, backward=False)
        dL = np.asarray(dL, np.float64)
        if mask_ambiguous:
            dL = dL * ((o["ambiguous"] & 3) == 0)[None]
        g2d = render_bwd(cam, o["pre"], o["point_list"], o["ranges"], dL, s)
        g3d = preprocess_bwd(cam, deg, params, o["pre"]["tiles_touched"], g2d, s)
        o["g2d"], o["g3d"], o["dL_used"] = g2d, g3d, dL
        per_view.append(o)
        total = {k: v.copy() for k, v in g3d.items()} if total is None else {k: total[k] + g3d[k] for k in total}
    return per_view, total


@dataclass
class DensifyParams:
    """The numbers [P4] D.1-D.3 leave out (see orc_densify_apply).  Values are
    rounded to float32, as the HIP library receives them."""
    grad_threshold: float
    prune_logit: float
    split_log_gap: float
    split_shrink: float
    split_offset: float
    clone_offset: float

    def array(self):
        return np.array([np.float32(x) for x in (self.grad_threshold, self.prune_logit, self.split_log_gap,
                                                 self.split_shrink, self.split_offset, self.clone_offset)],
                        dtype=np.float64)


GROUPS = ("means", "log_scales", "quats", "opacity_logits", "sh")


def densify_apply(params, accum, count, dp: DensifyParams, moments=None):
    """Densify and prune ([P4] D.1-D.3, E.1 steps 4-5).  params: the five groups;
    moments: None or dict group -> (m, v).  Returns (action, out_params, out_moments)
    with out arrays of the exact output count."""
    p = {k: _d(params[k]) for k in GROUPS}
    N = p["means"].shape[0]
    K = p["sh"].reshape(N, -1).shape[1] // 3 if N else 1
    width = {"means": 3, "log_scales": 3, "quats": 4, "opacity_logits": 1, "sh": 3 * K}
    outs = {k: np.zeros((2 * N, width[k])) for k in GROUPS}
    action = np.zeros(N, np.uint8)
    PP = C.POINTER(C.c_double)
    mom_in = mom_out = None
    keep = []
    if moments is not None:
        ins = [_d(moments[k][0]) for k in GROUPS] + [_d(moments[k][1]) for k in GROUPS]
        outs_m = [np.zeros((2 * N, width[k])) for k in GROUPS] + [np.zeros((2 * N, width[k])) for k in GROUPS]
        keep = ins + outs_m
        mom_in = (PP * 10)(*[_p(a) for a in ins])
        mom_out = (PP * 10)(*[_p(a) for a in outs_m])
    prm = dp.array()
    n_out = lib().orc_densify_apply(
        C.c_int(N), C.c_int(K), _p(prm), _p(p["means"]), _p(p["log_scales"]), _p(p["quats"]),
        _p(p["opacity_logits"]), _p(p["sh"]), _p(_d(accum)), _p(np.ascontiguousarray(count, dtype=np.int32), C.c_int),
        mom_in, _p(outs["means"]), _p(outs["log_scales"]), _p(outs["quats"]), _p(outs["opacity_logits"]),
        _p(outs["sh"]), mom_out, _p(action, C.c_uint8))
    out_params = {k: outs[k][:n_out].copy() for k in GROUPS}
    out_params["opacity_logits"] = out_params["opacity_logits"].reshape(n_out)
    out_params["sh"] = out_params["sh"].reshape(n_out, K, 3)
    out_moments = None
    if moments is not None:
        out_moments = {}
        for gi, k in enumerate(GROUPS):
            m, v = keep[10 + gi][:n_out].copy(), keep[15 + gi][:n_out].copy()
            if k == "opacity_logits":
                m, v = m.reshape(n_out), v.reshape(n_out)
            elif k == "sh":
                m, v = m.reshape(n_out, K, 3), v.reshape(n_out, K, 3)
            out_moments[k] = (m, v)
    return action, out_params, out_moments


def opacity_reset(logits, factor):
    """[P4] E.1 step 6: sigma <- factor sigma, as a logit."""
    x = _d(logits).copy()
    lib().orc_opacity_reset(C.c_int(x.size), C.c_double(factor), _p(x))
    return x


def round_binary16(x):
    """The nearest IEEE 754 binary16 values (ties to even; |x| >= 65520 to inf), as float64."""
    x = _d(x)
    out = np.zeros_like(x)
    lib().orc_round_binary16_array(C.c_int64(x.size), _p(x), _p(out))
    return out


def record16(pre):
    """The 2D quantities the blends read from 16-bit splat records ([P3] sections 5
    and 7): float32 mean; conic (through its scaled Cholesky factor), opacity and
    colour rounded to float32 and then to binary16.  Returns a copy of `pre` with
    uv, conic, opacity and rgb replaced; rect, tiles_touched, depth and the cull
    flags stay those of the full-precision projection."""
    N = pre["uv"].shape[0]
    out = dict(pre)
    out.update(uv=np.zeros((N, 2)), conic=np.zeros((N, 3)), opacity=np.zeros(N), rgb=np.zeros((N, 3)))
    valid = np.ascontiguousarray(pre["valid"], dtype=np.uint8)
    lib().orc_record16(C.c_int(N), _p(_d(pre["uv"])), _p(_d(pre["cov2d"])), _p(_d(pre["opacity"])),
                       _p(_d(pre["rgb"])), _p(valid, C.c_uint8), _p(out["uv"]), _p(out["conic"]),
                       _p(out["opacity"]), _p(out["rgb"]))
    return out
