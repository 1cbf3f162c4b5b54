"""The training step at its own configuration (1M Gaussians, 1920x1080, SH 3,
L1 loss against a random target) through the calls the benchmark times, against
the oracle running the same step:

  * gs_render_fwd_loss: forward with the L1 loss fused in (image and dL/dimage),
    which also clears the 2D-gradient buffer;
  * gs_render_bwd with accumulate = 1;
  * gs_preprocess_bwd_adam: the fused 2D->3D backward, densification statistic
    and Adam step (per-group learning rates, quaternion renormalisation).

Training notes (notes.huajishe.fun) E.1 (render, L1 loss, backpropagate,
accumulate the position-gradient statistic, optimizer step) and C.2 (Adam with
per-parameter learning rates).

Where a pixel's L1 sign or a blend decision is ambiguous (both outcomes are
correct float results) the two sides could differentiate different functions,
so both take the GPU's sign and the upstream gradient is zeroed at ambiguous
pixels, as in the other parity tests.  The Adam moments start at zero, so at
step 1 the first moment is (1 - beta1) g: the GPU's 3D gradient is recovered
from it and held to the per-tensor 1e-3 relative L2 bar and the per-Gaussian
row guard; the second moment, the updated parameters and the statistic are
compared element by element.
"""
import numpy as np
import pytest

from gpu_cases import PARAM_KEYS, guard_2d, guard_chain, log, rel_l2, to_dev
from differentiable_gaussian_splatting_dgs_amd import scenes

pytestmark = pytest.mark.gpu

# the Adam hyper-parameters as the library receives them (float32)
B1, B2, EPS = (float(np.float32(x)) for x in (0.9, 0.999, 1e-8))


def _loop_bars(cam, deg, params, tt, g2o, g3o, s):
    """Per-tensor relative L2 bars of a training-loop check: 1e-3, or the error a float32 evaluation
    of the same gradients can carry, whichever is larger.  Each 2D gradient component is a sum of
    per-pixel terms (the oracle's `abs` holds their absolute sizes); rounding each term to float32
    moves it by a few units of 2^-24 of its size, so the model perturbs every component by
    4 * 2^-24 of its terms' size with random signs and takes the 3D chain of that perturbation
    (linear for fixed parameters), the largest of four draws.  Early iterations give a model far
    under 1e-3; after thousands of iterations towards one target the gradients are sums of terms
    that cancel (the mean gradients by a factor of thousands), and the model rises above it."""
    from oracle import oracle as O
    from gpu_cases import grad2d_dict
    a = np.asarray(g2o["abs"], np.float64)
    rng = np.random.default_rng(0)
    bars = {k: 1e-3 for k in PARAM_KEYS}
    for _ in range(4):
        d = 4.0 * 2.0 ** -24 * a * rng.choice([-1.0, 1.0], a.shape)
        d3 = O.preprocess_bwd(cam, deg, params, tt, grad2d_dict(d), s)
        for k in PARAM_KEYS:
            bars[k] = max(bars[k], float(np.linalg.norm(d3[k]) / max(np.linalg.norm(g3o[k]), 1e-300)))
    return bars


def _oracle_adam(O, params, g3, lr, deg):
    """The oracle's step-1 Adam on every group, SH band 0 and the higher bands at their own rates,
    then the quaternion renormalisation."""
    out, mom = {}, {}
    for k in PARAM_KEYS:
        p = np.asarray(params[k], np.float64)
        g = np.asarray(g3[k], np.float64)
        if k == "sh":
            P, G = p.reshape(len(p), -1).copy(), g.reshape(len(g), -1)
            M, V = np.zeros_like(P), np.zeros_like(P)
            for cb, ce, key in ((0, 3, "sh_dc"), (3, P.shape[1], "sh_rest")):
                if ce > cb:
                    P[:, cb:ce], M[:, cb:ce], V[:, cb:ce] = O.adam(P[:, cb:ce], G[:, cb:ce], np.zeros_like(P[:, cb:ce]),
                                                                   np.zeros_like(P[:, cb:ce]), lr[key], 1, B1, B2, EPS)
            out[k], mom[k] = P.reshape(p.shape), (M.reshape(p.shape), V.reshape(p.shape))
        else:
            pp, mm, vv = O.adam(p, g, np.zeros_like(p), np.zeros_like(p), lr[k], 1, B1, B2, EPS)
            out[k], mom[k] = pp, (mm, vv)
    out["quats"] = O.quat_renorm(out["quats"])
    return out, mom


def test_train1m_step_matches_oracle():
    import torch
    from differentiable_gaussian_splatting_dgs_amd import gs
    from oracle import oracle as O
    sc = scenes.training1m()
    n, deg = sc.n, sc.sh_degree
    lr = dict(scenes.ADAM_LR)
    log(f"[train1m] n={n} {sc.cam.width}x{sc.cam.height}")
    p = to_dev(sc.params())
    r = gs.Rasterizer(sc.cam, n, deg)
    r.forward(p, check=True)  # sizes the lists
    target = torch.from_numpy(sc.target).cuda()
    dL = torch.empty_like(target)
    loss = torch.zeros(1 + r.ntiles, dtype=torch.float64, device="cuda")
    r.preprocess(p)
    r.bin()
    r.render_loss(target, "l1", dL, loss, clear_grad2d=True)
    torch.cuda.synchronize()
    assert int(r.overflow.item()) == 0
    img = r.image.cpu().numpy()
    sign = dL.cpu().numpy()
    tt = r.tiles_touched.cpu().numpy()
    log("[train1m] gpu forward + L1 done")

    s = O.Settings()
    pre = O.preprocess(sc.cam, deg, sc.params(), s)
    pl, rg = O.bin_gaussians(sc.cam, pre["rect"], pre["tiles_touched"], O.depth_key(pre["depth"]), s)
    fwd = O.render_fwd(sc.cam, pre, pl, rg, s)
    amb = (fwd["ambiguous"] & 3) > 0
    amb_grad = fwd["ambiguous"] > 0  # the 0.99 clamp too: only the gradient depends on it
    log(f"[train1m] oracle forward done, ambiguous pixels {int(amb.sum())}")
    assert amb.sum() <= 1e-3 * amb.size
    assert np.abs(img - fwd["image"])[:, ~amb].max() <= 1e-5
    # the fused loss: sign(image - target) with sign(0) = 0, and the loss itself
    L_o, dL_o = O.loss("l1", fwd["image"], sc.target)
    sure = np.abs(fwd["image"] - sc.target) > 1e-5
    assert np.array_equal(sign[sure & ~amb[None]], dL_o[sure & ~amb[None]])
    assert abs(float(loss[0]) - L_o) <= 1e-5 * L_o
    dL_used = sign * (~amb_grad)[None]

    # backward through the timed calls, from the masked sign
    dL.copy_(torch.from_numpy(dL_used.astype(np.float32)))
    r.backward_2d(dL, accumulate=True)
    m = {k: torch.zeros_like(v) for k, v in p.items()}
    v = {k: torch.zeros_like(x) for k, x in p.items()}
    acc = torch.zeros(n, dtype=torch.float32, device="cuda")
    cnt = torch.zeros(n, dtype=torch.int32, device="cuda")
    gs.gs_preprocess_bwd_adam(r.cam, r.settings, deg, p, r.tiles_touched, r.clamp, r.grad2d, m, v, lr, 1,
                              densify_accum=acc, densify_count=cnt)
    torch.cuda.synchronize()
    log("[train1m] gpu backward + fused tail done")

    g2o = O.render_bwd(sc.cam, pre, pl, rg, dL_used, s, with_abs=True)
    g3o = O.preprocess_bwd(sc.cam, deg, sc.params(), pre["tiles_touched"], g2o, s)
    log("[train1m] oracle backward done")

    vis = tt > 0
    g2 = r.grad2d.cpu().numpy()
    guard_2d(g2, g2o, "train1m")
    # the GPU's 3D gradient, from the first moment (zero before the step): (1 - beta1) g
    g_gpu = {k: m[k].cpu().numpy().astype(np.float64) / (1 - B1) for k in PARAM_KEYS}
    for k in PARAM_KEYS:
        e = rel_l2(g_gpu[k], g3o[k])
        log(f"[train1m] {k}: gradient rel L2 {e:.2e}")
        assert e <= 1e-3, (k, e)
    guard_chain(sc.cam, deg, sc.params(), tt, g2, g_gpu, "train1m")
    # the densification statistic from the GPU's own 2D gradients
    assert np.array_equal(cnt.cpu().numpy(), vis.astype(np.int32))
    acc_o = np.where(vis, np.linalg.norm(g2[:, 0:2].astype(np.float64), axis=1), 0.0)
    assert np.all(np.abs(acc.cpu().numpy() - acc_o) <= 1e-6 * acc_o + 1e-30)
    # Adam step 1 from the GPU's own gradients: the update's arithmetic
    po, mo = _oracle_adam(O, sc.params(), g_gpu, lr, deg)
    for k in PARAM_KEYS:
        pg = p[k].cpu().numpy().astype(np.float64)
        lr_k = np.full(pg.shape, lr[k] if k != "sh" else lr["sh_rest"])
        if k == "sh":
            lr_k[:, 0, :] = lr["sh_dc"]
        ulp = np.spacing(np.abs(po[k]).astype(np.float32)).astype(np.float64)
        d = np.abs(pg - po[k])
        assert np.all(d <= 1e-4 * lr_k + 8 * ulp), (k, float(d.max()))
        gv = v[k].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(gv - mo[k][1]) <= 1e-5 * mo[k][1] + 1e-30), k
        log(f"[train1m] {k}: updated parameters max diff {d.max():.2e}")


def _host(d):
    return {k: v.detach().cpu().numpy().copy() for k, v in d.items()}


def test_training_loop_across_densify_and_reset():
    """The training loop over iterations ([P4] E.1 steps 1-6) with the interval and factor the notes
    print: densify and prune every 100 iterations (N changes and the Rasterizer is rebuilt), reset
    every opacity to 0.3 of itself every 3000.  The loop runs 3001 iterations through gs.Trainer.
    At chosen iterations -- the first two, the densifications at 100 and 3000 and the iterations
    right after them (the first at the new N), and the reset at 3000 -- the oracle recomputes the
    iteration from the GPU state before it, stage by stage: image, loss sign, 3D gradients, the
    Adam update from the GPU's gradients, the statistic, the densification from the GPU's
    updated state, and the reset.  The 3D gradients meet 1e-3 relative L2 per tensor, or the
    float32 error model of _loop_bars where the state's gradients are sums of cancelling terms;
    every 2D component stays within 1e-3 of its terms' size and every chain row within the
    chain guard."""
    import json
    import os
    import torch
    from differentiable_gaussian_splatting_dgs_amd import gs
    from oracle import oracle as O
    page = {k: v["value"] for k, v in json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                                                   "page_constants.json"))).items()}
    d_int, r_int, r_fac = int(page["densify_interval"]), int(page["opacity_reset_interval"]), page["opacity_reset_factor"]
    sc = scenes.random_small(80, n=300, width=96, height=80, f=70.0, sh_degree=1, scale_mu=-2.2)
    deg = sc.sh_degree
    target = np.random.default_rng(80).uniform(0, 1, (3, sc.cam.height, sc.cam.width)).astype(np.float32)
    lr = dict(scenes.ADAM_LR)
    dp = gs.DensifyParams(grad_threshold=1.5)
    tr = gs.Trainer(sc.cam, to_dev(sc.params()), deg, torch.from_numpy(target).cuda(), lr, densify=dp,
                    densify_interval=d_int, reset_interval=r_int, reset_factor=r_fac)
    checks = {1, 2, d_int, d_int + 1, r_int, r_int + 1}
    s = O.Settings()
    n_checked = 0

    def checked_step():
        t = tr.t + 1
        pre = dict(p=_host(tr.p), m=_host(tr.m), v=_host(tr.v), acc=tr.accum.cpu().numpy().copy(),
                   cnt=tr.count.cpu().numpy().copy())
        n = tr.n
        params = {k: pre["p"][k] for k in PARAM_KEYS}
        o = O.render(sc.cam, deg, params, s, backward=False)
        amb = (o["ambiguous"] & 3) > 0
        amb_grad = o["ambiguous"] > 0
        seen = {}

        def hook(dL):
            img = tr.rast.image.cpu().numpy()
            assert np.abs(img - o["image"])[:, ~amb].max() <= 1e-5, t
            sign = dL.cpu().numpy()
            sure = (np.abs(o["image"] - target) > 1e-5) & ~amb[None]
            _, dL_o = O.loss("l1", o["image"], target)
            assert np.array_equal(sign[sure], dL_o[sure]), t
            seen["dL"] = sign * (~amb_grad)[None]
            dL.copy_(torch.from_numpy(seen["dL"].astype(np.float32)))

        grads = {k: torch.empty_like(v) for k, v in tr.p.items()}

        def after(trainer):
            seen["post"] = dict(p=_host(trainer.p), m=_host(trainer.m), v=_host(trainer.v),
                                acc=trainer.accum.cpu().numpy().copy(), cnt=trainer.count.cpu().numpy().copy())
            seen["g"] = _host(grads)
            seen["g2"] = trainer.rast.grad2d.cpu().numpy().copy()
            seen["tt"] = trainer.rast.tiles_touched.cpu().numpy().copy()

        tr.step(dL_hook=hook, grads=grads, after_update=after)
        torch.cuda.synchronize()
        g2o = O.render_bwd(sc.cam, o["pre"], o["point_list"], o["ranges"], seen["dL"], s, with_abs=True)
        g3o = O.preprocess_bwd(sc.cam, deg, params, o["pre"]["tiles_touched"], g2o, s)
        vis = o["pre"]["tiles_touched"] > 0
        assert np.array_equal(seen["tt"], o["pre"]["tiles_touched"]), t
        if os.environ.get("GS_DUMP_LOOP"):
            np.savez(os.path.join(os.environ["GS_DUMP_LOOP"], f"loop_t{t}.npz"), dL=seen["dL"], g2=seen["g2"],
                     tt=seen["tt"], **{"p_" + k: v for k, v in params.items()},
                     **{"g_" + k: v for k, v in seen["g"].items()})
        guard_2d(seen["g2"], g2o, f"t={t}")
        guard_chain(sc.cam, deg, params, seen["tt"], seen["g2"], seen["g"], f"t={t}")
        bars = _loop_bars(sc.cam, deg, params, o["pre"]["tiles_touched"], g2o, g3o, s)
        for k in PARAM_KEYS:
            e = rel_l2(seen["g"][k], g3o[k])
            assert e <= bars[k], (t, k, e, bars[k])
        log(f"t={t}: relative L2 bars {', '.join(f'{k} {v:.1e}' for k, v in bars.items())}")
        # Adam at iteration t from the GPU's own gradients: the update's arithmetic alone
        post = seen["post"]
        for k in PARAM_KEYS:
            P, G = pre["p"][k].astype(np.float64), seen["g"][k].astype(np.float64)
            M, V = pre["m"][k].astype(np.float64), pre["v"][k].astype(np.float64)
            if k == "sh":
                P, G, M, V = (x.reshape(n, -1) for x in (P, G, M, V))
                cols = ((0, 3, "sh_dc"), (3, P.shape[1], "sh_rest"))
            else:
                cols = ((None, None, k),)
            Po, Mo, Vo, LR = P.copy(), M.copy(), V.copy(), np.zeros_like(P)
            for cb, ce, key in cols:
                sl = (slice(None), slice(cb, ce)) if cb is not None else (Ellipsis,)
                Po[sl], Mo[sl], Vo[sl] = O.adam(P[sl], G[sl], M[sl], V[sl], lr[key], t, B1, B2, EPS)
                LR[sl] = lr[key]
            if k == "quats":
                Po = O.quat_renorm(Po)
            # float32 rounding of the moments (a few roundings of each term), of the parameter (a few
            # ulps) and of the update (1e-4 of its learning rate: a wrong rate, step or bias
            # correction moves it by the order of the rate itself)
            gp = post["p"][k].reshape(Po.shape).astype(np.float64)
            ulp = np.spacing(np.abs(Po).astype(np.float32)).astype(np.float64)
            assert np.all(np.abs(gp - Po) <= 1e-4 * LR + 8 * ulp), (t, k, float(np.abs(gp - Po).max()))
            gm = post["m"][k].reshape(Mo.shape).astype(np.float64)
            assert np.all(np.abs(gm - Mo) <= 1e-6 * (0.9 * np.abs(M) + 0.1 * np.abs(G)) + 1e-30), (t, k)
            gv = post["v"][k].reshape(Vo.shape).astype(np.float64)
            assert np.all(np.abs(gv - Vo) <= 1e-6 * Vo + 1e-30), (t, k)
        # densification statistic
        cnt_o = pre["cnt"] + vis
        assert np.array_equal(post["cnt"], cnt_o), t
        acc_o = pre["acc"] + np.where(vis, np.linalg.norm(seen["g2"][:, 0:2].astype(np.float64), axis=1), 0.0)
        assert np.all(np.abs(post["acc"] - acc_o) <= 1e-6 * acc_o + 1e-30), t
        if t % d_int == 0:
            moments = {k: (post["m"][k], post["v"][k]) for k in PARAM_KEYS}
            st = dp.struct()
            odp = O.DensifyParams(st.grad_threshold, st.prune_logit, st.split_log_gap, st.split_shrink,
                                  st.split_offset, st.clone_offset)
            oa, op, om = O.densify_apply({k: post["p"][k] for k in PARAM_KEYS}, post["acc"], post["cnt"], odp,
                                         moments)
            assert np.array_equal(tr.last_action.cpu().numpy(), oa), t
            assert tr.n == op["means"].shape[0], t
            after_d = _host(tr.p)
            if t % r_int == 0:
                op = dict(op, opacity_logits=O.opacity_reset(op["opacity_logits"], r_fac))
                assert float(tr.m["opacity_logits"].abs().max()) == 0.0
                assert float(tr.v["opacity_logits"].abs().max()) == 0.0
                assert np.all(np.abs(after_d["opacity_logits"] - op["opacity_logits"]) <=
                              16 * 2.0 ** -24 * (1.0 + np.abs(op["opacity_logits"]))), t
            else:
                assert np.array_equal(after_d["opacity_logits"], op["opacity_logits"].astype(np.float32)), t
            for k in ("quats", "sh"):
                assert np.array_equal(after_d[k], op[k].astype(np.float32)), (t, k)
            for k in ("means", "log_scales"):
                assert np.allclose(after_d[k], op[k], rtol=1e-6, atol=1e-6), (t, k)
            if t % r_int != 0:
                for k in PARAM_KEYS:
                    assert np.array_equal(tr.m[k].cpu().numpy(), om[k][0].astype(np.float32)), (t, k)
            assert float(tr.accum.abs().max()) == 0.0 and int(tr.count.abs().max()) == 0
        log(f"[loop] iteration {t} checked, N {n} -> {tr.n}")

    while tr.t < r_int + 1:
        if tr.t + 1 in checks:
            checked_step()
            n_checked += 1
        else:
            tr.step()
    torch.cuda.synchronize()
    kinds = [e[1] for e in tr.events]
    assert kinds.count("densify") == r_int // d_int and kinds.count("reset") == 1
    sizes = [e[2] for e in tr.events if e[1] == "densify"]
    assert any(a != b for a, b in sizes), sizes  # N changed
    assert n_checked == len(checks)
    log(f"[loop] {tr.t} iterations, N {sc.n} -> {tr.n}, densify events {len(sizes)}")
