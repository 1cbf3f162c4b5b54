"""Benchmark of the differentiable tile rasterizer on one MI355X.

One step = the whole hot path on the 1M-Gaussian 1920x1080 cluster-mixture
scene: preprocess, binning + depth sort, forward compositing with the L1 loss
against a random target fused in, reverse-walk backward, 2D->3D backward,
densification statistic and the Adam update of all parameter groups (with
quaternion renormalisation).  Inputs are resident in HBM before timing starts.

Prints one JSON line.  `value` is Gaussian-pixel blend pairs per second over the
whole step: (evaluated forward pairs + walked backward pairs) / step time.
The step runs on one stream by default; --overlap color|sh moves the SH work to a
second stream (see Step).  On MI355X both overlaps are slower than one stream:
the SH passes are HBM-bound and slow the latency-bound projection and binning
they run beside more than they hide.
`fwd_bwd` reports the rasterizer on the same scene and state: preprocess,
binning, forward (with the per-pixel loss gradient the backward starts from),
backward blend and the unfused 2D->3D backward that writes the 3D gradients
(no optimizer).  `densify` times the densify / split / clone / prune pass
(run every 100 training steps, so not part of the step) on the trained state.
`views` times a batched training step over --views orbit views of the same scene.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd rasterize ms/iter & blend pairs/s, 1M Gaussians @1080p; % roofline"
PEAK_FP32_TFLOPS = 157.3   # MI355X published fp32 vector peak
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E

# Algorithmic operations per pair, counted from the method's arithmetic (each
# add, mul, compare, exp and divide is one operation):
#   evaluate alpha:  d (2), d^T conic d (9), exp (1), opacity*G (1), min (1) = 14
#   forward blend:   1 - alpha, T(1 - alpha), stop test, w = alpha T, C += w c (6) = 10
#   backward blend:  T / (1 - alpha) (2), w (1), dL/dc (3), dL/dalpha (9), C_next (6),
#                    dsigma, dG, dpower (3), dconic (5), dmean2D (8), 9 accumulations = 47
FLOPS_EVAL, FLOPS_FWD_BLEND, FLOPS_BWD_BLEND = 14, 10, 47


WORKLOADS = ("train1m", "tiny", "ball100k", "clusters1m", "plane3m")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--views", type=int, default=4,
                    help="views of the batched training step measured beside the main one (1 skips it)")
    ap.add_argument("--overlap", choices=("none", "color", "sh"), default="none",
                    help="work moved to a second stream: none, the SH colour pass (color), or the colour pass and "
                         "the SH half of the Adam tail (sh)")
    ap.add_argument("--cpu-tile-fraction", type=float, default=1.0)
    ap.add_argument("--workload", default="train1m", choices=WORKLOADS,
                    help="train1m (the training step, the default bench line) or tiny / ball100k / clusters1m / "
                         "plane3m: the rasterizer's fwd+bwd alone on that scene")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="run one device copy of this many MiB first (scales HBM byte counters)")
    return ap.parse_args()


def sha_of(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def read_traffic(kernel, launches_per_step=1):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None when
    the summary is missing or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_train1m_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"source_sha256:\s*(\w+)", text)
    src = os.path.join(ROOT, "differentiable_gaussian_splatting_dgs_amd", "csrc", "render.hip")
    if not m_sha or m_sha.group(1) != sha_of(src):
        return None
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    return float(m_b.group(1)) if m_b else None


class Step:
    """All buffers of the training step.  run() enqueues one step.

    Without overlap (the default) a step is the single-stream sequence
    preprocess, bin, fwd+loss, bwd, fused tail.

    overlap="sh" runs the SH work on a second stream: the SH coefficients are
    needed again only by the next step's colour pass, not by its projection and
    binning, so step i's SH update and step i+1's colour pass run while step
    i+1 bins its tiles.  Events keep every read after the write it depends on,
    so each step computes what the single-stream order computes:

      main:  project(i) -> bin(i) -> [wait colour(i)] -> fwd+loss(i) -> bwd(i) -> geometry tail(i)
      side:  [wait geometry tail(i-1)] -> SH tail(i-1) -> colour(i)

    overlap="color" keeps the fused tail on the main stream and moves only the
    colour pass.  finish() enqueues the last SH tail and joins the streams.
    """

    def __init__(self, sc, overlap="none"):
        import torch
        from differentiable_gaussian_splatting_dgs_amd import gs, scenes
        self.gs, self.torch, self.sc = gs, torch, sc
        dev = "cuda"
        self.p = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in sc.params().items()}
        self.target = torch.from_numpy(sc.target).to(dev)
        self.rast = gs.Rasterizer(sc.cam, sc.n, sc.sh_degree)
        self.dL = torch.empty_like(self.target)
        self.loss = torch.zeros(1 + self.rast.ntiles, dtype=torch.float64, device=dev)
        self.m = {k: torch.zeros_like(v) for k, v in self.p.items()}
        self.v = {k: torch.zeros_like(v) for k, v in self.p.items()}
        self.accum = torch.zeros(sc.n, dtype=torch.float32, device=dev)
        self.count = torch.zeros(sc.n, dtype=torch.int32, device=dev)
        lr = scenes.ADAM_LR
        self.lr = dict(lr)
        self.step_no = 0
        # overlap: "none" (one stream), "color" (the colour pass on a second stream) or "sh" (the colour pass
        # and the SH half of the tail on a second stream)
        if overlap is True:
            overlap = "sh"
        elif overlap is False or overlap is None:
            overlap = "none"
        assert overlap in ("none", "color", "sh"), overlap
        self.overlap = overlap if overlap != "none" else None
        self.ev_geom = None
        self.sh_step = 0
        if self.overlap:
            self.stages = ["project", "bin_sort", "render_fwd_loss", "render_bwd",
                           "geometry_tail" if self.overlap == "sh" else "grad3d_densify_adam"]
            self.side = torch.cuda.Stream()  # default priority
            self.view_dir = torch.empty((sc.n, 3), dtype=torch.float32, device=dev)
        else:
            self.stages = ["preprocess", "bin_sort", "render_fwd_loss", "render_bwd", "grad3d_densify_adam"]
        self.g3 = {k: torch.empty_like(v) for k, v in self.p.items()}

    def _sh_tail(self):
        r = self.rast
        self.gs.gs_preprocess_bwd_adam_sh(r.deg, self.p["sh"], r.clamp, r.grad2d, self.view_dir, self.m["sh"],
                                          self.v["sh"], self.lr, self.sh_step)

    def run(self, events=None, check=False):
        gs, torch, r, p = self.gs, self.torch, self.rast, self.p
        self.step_no += 1
        ev = events

        def mark(i):
            if ev is not None:
                ev[i].record()
        if self.overlap:
            main = torch.cuda.current_stream()
            with torch.cuda.stream(self.side):
                if self.ev_geom is not None:
                    self.side.wait_event(self.ev_geom)
                    if self.overlap == "sh":
                        self._sh_tail()
                else:
                    self.side.wait_stream(main)
                gs.gs_shade(r.cam, r.deg, p["means"], p["sh"], r.splats, r.clamp)
                ev_color = torch.cuda.Event()
                ev_color.record(self.side)
            mark(0)
            gs.gs_project(r.cam, r.settings, p, r.splats, r.depth, r.rect, r.tiles_touched)
        else:
            mark(0)
            r.preprocess(p)
        mark(1)
        r.bin()
        if check and int(r.overflow.item()) != 0:
            K = int(r.num_keys.item())
            r._alloc_lists(int(K * 1.25) + 1024)
            r.bin()
        mark(2)
        if self.overlap:
            main.wait_event(ev_color)
        # forward blend with the L1 loss fused in; it also clears the 2D-gradient buffer
        r.render_loss(self.target, "l1", self.dL, self.loss, clear_grad2d=True)
        mark(3)
        r.backward_2d(self.dL, accumulate=True)
        mark(4)
        if self.overlap == "sh":
            gs.gs_preprocess_bwd_adam_geom(r.cam, r.settings, r.deg, p, r.tiles_touched, r.clamp, r.grad2d, self.m,
                                           self.v, self.lr, self.step_no, self.view_dir, densify_accum=self.accum,
                                           densify_count=self.count)
        else:
            gs.gs_preprocess_bwd_adam(r.cam, r.settings, r.deg, p, r.tiles_touched, r.clamp, r.grad2d, self.m,
                                      self.v, self.lr, self.step_no, densify_accum=self.accum,
                                      densify_count=self.count)
        if self.overlap:
            self.ev_geom = torch.cuda.Event()
            self.ev_geom.record(main)
            self.sh_step = self.step_no
        mark(5)

    def finish(self):
        """Enqueue the last step's SH update and make the current stream wait for it."""
        if self.overlap and self.ev_geom is not None:
            torch = self.torch
            if self.overlap == "sh":
                with torch.cuda.stream(self.side):
                    self.side.wait_event(self.ev_geom)
                    self._sh_tail()
            torch.cuda.current_stream().wait_stream(self.side)
            self.ev_geom = None

    def preprocess_bwd(self):
        """The unfused 2D->3D backward with its gradients written out (the rasterizer's own backward)."""
        r, p, g = self.rast, self.p, self.g3
        self.gs.gs_preprocess_bwd(r.cam, r.settings, r.deg, p["means"], p["log_scales"], p["quats"],
                                  p["opacity_logits"], p["sh"], r.tiles_touched, r.clamp, r.grad2d, g["means"],
                                  g["log_scales"], g["quats"], g["opacity_logits"], g["sh"])


def views_measure(sc, views, steps, warmup):
    """A batched training step ([P4] E.1: a batch of views rendered, their L1 losses summed,
    one Adam step): `views` orbit cameras around the train1m scene, each with its own
    random target, through the *_views calls.  Fresh parameters and Adam state, so it
    does not disturb the main measurement."""
    import torch
    from differentiable_gaussian_splatting_dgs_amd import gs, scenes
    dev = "cuda"
    centre = (0.0, 0.0, float(np.median(np.asarray(sc.means[:, 2], np.float64))))
    cams = scenes.orbit_cameras(sc.cam, views, centre, step_deg=8.0)
    rng = np.random.default_rng(11)
    target = torch.from_numpy(rng.uniform(0, 1, (views, 3, sc.cam.height, sc.cam.width)).astype(np.float32)).to(dev)
    p = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in sc.params().items()}
    m = {k: torch.zeros_like(v) for k, v in p.items()}
    v2 = {k: torch.zeros_like(v) for k, v in p.items()}
    acc = torch.zeros(sc.n, dtype=torch.float32, device=dev)
    cnt = torch.zeros(sc.n, dtype=torch.int32, device=dev)
    rv = gs.RasterizerViews(cams, sc.n, sc.sh_degree)
    dL = torch.empty_like(target)
    loss = torch.zeros(1 + rv.ntiles, dtype=torch.float64, device=dev)
    lr = dict(scenes.ADAM_LR)
    stages = ["preprocess", "bin_sort", "render_fwd_loss", "render_bwd", "grad3d_densify_adam"]
    step_no = [0]

    def run(ev=None, check=False):
        step_no[0] += 1

        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        rv.preprocess(p)
        mark(1)
        rv.bin()
        if check and int(rv.overflow.item()) != 0:
            rv._alloc_lists(int(int(rv.num_keys.item()) * 1.25) + 1024)
            rv.bin()
        mark(2)
        rv.render_loss(target, "l1", dL, loss, clear_grad2d=True)
        mark(3)
        rv.backward_2d(dL, accumulate=True)
        mark(4)
        gs.gs_preprocess_bwd_adam_views(cams, rv.settings, sc.sh_degree, p, rv.tiles_touched, rv.clamp, rv.grad2d,
                                        m, v2, lr, step_no[0], densify_accum=acc, densify_count=cnt)
        mark(5)

    run(check=True)
    for _ in range(max(0, warmup - 1)):
        run()
    torch.cuda.synchronize()
    c0 = rv.count_pairs().cpu().numpy()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run(evs[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    assert int(rv.overflow.item()) == 0, "list capacity overflow during the batched timing"
    c1 = rv.count_pairs().cpu().numpy()
    stage_ms = {name: round(float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)])), 4)
                for j, name in enumerate(stages)}
    pairs = float((c0[0] + c1[0]) / 2 + (c0[1] + c1[1]) / 2)
    out = dict(workload=f"train1m x {views} views: {views} orbit cameras 8 degrees apart around the scene, "
                        f"one L1 target each, losses summed, one Adam step",
               views=views, ms_per_step=round(ms, 4), ms_per_view=round(ms / views, 4),
               pairs_per_s=float(pairs / (ms * 1e-3)), keys=int(rv.num_keys.item()), stage_ms=stage_ms)
    del rv, p, m, v2
    torch.cuda.empty_cache()
    return out


def measure_peaks(reps=5):
    """What this GPU delivers on the two binding resources, timed with HIP events:
    HBM with the library's non-temporal copy over 1 GiB (2 GiB of traffic), fp32
    with its FMA loop (8 independent chains per lane, 8 waves per SIMD).  Median
    of `reps` timed calls after one untimed call."""
    import torch
    from differentiable_gaussian_splatting_dgs_amd import gs
    n = 256 << 20
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def timed(fn):
        fn()
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(out))
    t_copy = timed(lambda: gs.gs_stream_copy(src, dst))
    del src, dst
    blocks, iters = 256 * 8, 512
    out = torch.empty(blocks * gs.FMA_LOOP_THREADS, dtype=torch.float32, device="cuda")
    t_fma = timed(lambda: gs.gs_fma_loop(blocks, iters, 1.0000001, 1e-7, out))
    flops = blocks * gs.FMA_LOOP_THREADS * iters * gs.FMA_LOOP_FLOPS_PER_ITER
    return dict(hbm_gbs=dict(spec=PEAK_HBM_GBS, measured=round(8.0 * n / t_copy / 1e9, 1),
                             kernel="gs_stream_copy, 1 GiB"),
                fp32_tflops=dict(spec=PEAK_FP32_TFLOPS, measured=round(flops / t_fma / 1e12, 2),
                                 kernel="gs_fma_loop, 8 chains x 8 waves per SIMD"))


def walked_entries(r):
    """List entries the backward blend walks with at least one flagged quadrant: each
    costs one nine-value reduction and nine float atomics (two entries share one
    atomic instruction).  Counted on the device from the last step's buffers."""
    import torch
    K = int(r.num_keys.item())
    T = r.ntiles
    rng = r.tile_ranges.long()
    H, W = r.n_contrib.shape
    nc = torch.zeros((r.tiles_y * 16, r.tiles_x * 16), dtype=torch.int32, device=r.n_contrib.device)
    nc[:H, :W] = r.n_contrib
    ncmax = nc.view(r.tiles_y, 16, r.tiles_x, 16).amax(dim=(1, 3)).reshape(-1).long()
    tile_of = torch.repeat_interleave(torch.arange(T, device=rng.device), rng[:, 1] - rng[:, 0])
    pos = torch.arange(K, device=rng.device) - rng[tile_of, 0]
    walked = (pos < ncmax[tile_of]) & (r.contrib[:K] != 0)
    return int(walked.sum().item())


def densify_measure(st, reps):
    """gs_densify (densify, split or clone, prune) on the trained state: the parameters, Adam moments
    and the statistic the steps above accumulated.  Out of place, so every repetition does the same
    work.  Algorithmic bytes: every surviving Gaussian's row read once (parameters, moments,
    statistic), a removed one's decision fields (log-scales, opacity, statistic: 24 B), every output
    row written once."""
    gs, torch, sc = st.gs, st.torch, st.sc
    n, K = sc.n, (sc.sh_degree + 1) ** 2
    dp = gs.DensifyParams(gs.DensifyParams.threshold_for(sc.cam.height))
    cap = 2 * n

    def like(t):
        return torch.empty((cap,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)

    inp = dict(st.p, densify_accum=st.accum, densify_count=st.count, exp_avg=st.m, exp_avg_sq=st.v)
    out = {k: like(v) for k, v in st.p.items()}
    out["exp_avg"] = {k: like(v) for k, v in st.m.items()}
    out["exp_avg_sq"] = {k: like(v) for k, v in st.v.items()}
    out["densify_accum"], out["densify_count"] = like(st.accum), like(st.count)
    n_out = torch.zeros(1, dtype=torch.int32, device="cuda")
    ovf = torch.zeros(1, dtype=torch.int32, device="cuda")
    action = torch.empty(n, dtype=torch.uint8, device="cuda")
    wsz = gs.gs_densify_workspace_size(n)
    ws = torch.empty(wsz + 256, dtype=torch.uint8, device="cuda")
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + wsz]
    gs.gs_densify(dp, sc.sh_degree, inp, cap, out, n_out, ovf, ws, action)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record()
        gs.gs_densify(dp, sc.sh_degree, inp, cap, out, n_out, ovf, ws, action)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    acts = np.bincount(action.cpu().numpy(), minlength=4)
    rows = int(n_out.item())
    row_bytes = 4 * (2 * 3 + 4 + 1 + 3 * K) * 3 + 8          # parameters, two moments, statistic
    nbytes = row_bytes * (n - int(acts[0])) + 24 * int(acts[0]) + row_bytes * rows
    gbs = nbytes / (ms * 1e-3) / 1e9
    del out, inp
    return dict(ms=round(ms, 4), n_in=n, n_out=rows,
                actions=dict(removed=int(acts[0]), kept=int(acts[1]), cloned=int(acts[2]), split=int(acts[3])),
                grad_threshold=round(dp.grad_threshold, 4), algorithmic_bytes=int(nbytes),
                roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=round(gbs / PEAK_HBM_GBS, 4)))


def host_cpu():
    """The host the CPU baseline ran on: CPU model (from /proc/cpuinfo) and the number of CPUs."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(cpu_model=model, nproc=os.cpu_count())


def cpu_baseline(sc, frac, seed=0):
    """The oracle on a bounded sample of the same step, scaled to blend pairs/s.

    Sample: full preprocess and binning of all Gaussians; forward, L1 loss and
    backward over a random `frac` of the tiles; 2D->3D backward, densification and
    Adam over the same fraction of the Gaussians.  Each stage's time is scaled by
    its sampled fraction (pixel stages by pairs, per-Gaussian stages by count)."""
    from oracle import oracle as O
    s = O.Settings()
    params = sc.params()
    t = {}
    t0 = time.perf_counter()
    pre = O.preprocess(sc.cam, sc.sh_degree, params, s)
    t["preprocess"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    pl, rg = O.bin_gaussians(sc.cam, pre["rect"], pre["tiles_touched"], O.depth_key(pre["depth"]), s)
    t["bin"] = time.perf_counter() - t0
    ntiles = rg.shape[0]
    rng = np.random.default_rng(seed)
    tmask = np.zeros(ntiles, np.uint8)
    tmask[rng.permutation(ntiles)[: max(1, int(frac * ntiles))]] = 1
    t0 = time.perf_counter()
    fwd = O.render_fwd(sc.cam, pre, pl, rg, s, tile_mask=tmask)
    t["fwd"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    _, dL = O.loss("l1", fwd["image"], sc.target)
    t["loss"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    g2 = O.render_bwd(sc.cam, pre, pl, rg, dL, s, tile_mask=tmask)
    t["bwd"] = time.perf_counter() - t0
    n_s = max(1, int(frac * sc.n))
    sub = {k: v[:n_s] for k, v in params.items()}
    g2s = {k: v[:n_s] for k, v in g2.items()}
    t0 = time.perf_counter()
    g3 = O.preprocess_bwd(sc.cam, sc.sh_degree, sub, pre["tiles_touched"][:n_s], g2s, s)
    t["preprocess_bwd"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.densify(pre["tiles_touched"][:n_s], g2s["dxy"], np.zeros(n_s), np.zeros(n_s, np.int32))
    for k in ("means", "log_scales", "quats", "opacity_logits", "sh"):
        O.adam(sub[k], g3[k], np.zeros(sub[k].shape), np.zeros(sub[k].shape), 1e-3, 1)
    O.quat_renorm(sub["quats"])
    t["densify_adam"] = time.perf_counter() - t0
    pairs_sample = int(fwd["counts"][0] + fwd["counts"][1])
    # fraction of the full step's pairs covered by the tile sample
    pix_frac = float(tmask.mean())
    est = (t["preprocess"] + t["bin"] + (t["fwd"] + t["bwd"]) / pix_frac + t["loss"]
           + (t["preprocess_bwd"] + t["densify_adam"]) * sc.n / n_s)
    work = sum(t.values())
    return dict(est_step_s=est, work_s=work, pairs_sample=pairs_sample, tile_fraction=pix_frac,
                gauss_fraction=n_s / sc.n, stage_s={k: round(v, 3) for k, v in t.items()})


def raster_roofline(N, K, deg, p_fwd, p_bwd, p_blend, raster_ms, peaks):
    """The rasterizer's roofline fraction: the sum over its stages of the least time the binding peak allows
    for the stage's algorithmic bytes (preprocess, binning, 2D->3D backward) or flops (the two blends), over
    the measured fwd+bwd time; against the published peaks and against the measured ones."""
    hbm = PEAK_HBM_GBS * 1e9
    fl = PEAK_FP32_TFLOPS * 1e12
    par = 4.0 * (3 + 3 + 4 + 1 + 3 * (deg + 1) ** 2)                      # parameter bytes per Gaussian
    tmin = dict(
        preprocess=(par + 65.0) * N / hbm,                                 # parameters in, 65 B records out
        bin_sort=(16 * N + 4 * 16 * N + 20 * N + 8 * K + 2 * 16 * K + 4 * K) / hbm,  # keys, 4 depth passes,
                                                                           # emission, 2 tile passes, ranges
        render_fwd=(FLOPS_EVAL * p_fwd + FLOPS_FWD_BLEND * p_blend) / fl,
        render_bwd=(FLOPS_EVAL * p_bwd + FLOPS_BWD_BLEND * p_blend) / fl,
        preprocess_bwd=(2 * par + 41.0) * N / hbm)  # parameters + 36 B 2D gradients + 5 B count/clamp in, grads out
    scale = dict(preprocess=PEAK_HBM_GBS / peaks["hbm_gbs"]["measured"],
                 bin_sort=PEAK_HBM_GBS / peaks["hbm_gbs"]["measured"],
                 render_fwd=PEAK_FP32_TFLOPS / peaks["fp32_tflops"]["measured"],
                 render_bwd=PEAK_FP32_TFLOPS / peaks["fp32_tflops"]["measured"],
                 preprocess_bwd=PEAK_HBM_GBS / peaks["hbm_gbs"]["measured"])
    tmin_meas = sum(v * scale[k] for k, v in tmin.items())
    return dict(t_min_us={k: round(v * 1e6, 2) for k, v in tmin.items()},
                t_min_sum_us=round(sum(tmin.values()) * 1e6, 2),
                frac=round(sum(tmin.values()) / (raster_ms * 1e-3), 4),
                t_min_sum_us_measured_peaks=round(tmin_meas * 1e6, 2),
                frac_of_measured=round(tmin_meas / (raster_ms * 1e-3), 4))


def rasterizer_workload(name, steps, warmup):
    """fwd+bwd of the rasterizer alone on another scene (no optimizer, so the workload does not drift):
    preprocess, binning, forward (with the scene's loss fused in when it has one), backward blend and the
    2D->3D backward.  Prints its own JSON line; the default bench line is the training step on train1m."""
    import torch
    from differentiable_gaussian_splatting_dgs_amd import gs, scenes
    sc = scenes.make(name)
    dev = "cuda"
    p = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in sc.params().items()}
    r = gs.Rasterizer(sc.cam, sc.n, sc.sh_degree)
    g3 = {k: torch.empty_like(v) for k, v in p.items()}
    loss = torch.zeros(1 + r.ntiles, dtype=torch.float64, device=dev)
    if sc.loss:
        target = torch.from_numpy(np.ascontiguousarray(sc.target)).to(dev)
        dL = torch.empty_like(target)
    else:
        target = None
        dL = torch.from_numpy(np.ascontiguousarray(sc.dL_dimage)).to(dev)
    r.forward(p, check=True)                       # sizes the list capacity
    stages = ["preprocess", "bin_sort", "render_fwd", "render_bwd", "preprocess_bwd"]

    def run(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        r.preprocess(p)
        mark(1)
        r.bin()
        mark(2)
        if target is not None:
            r.render_loss(target, sc.loss, dL, loss, clear_grad2d=False)
        else:
            r.render()
        mark(3)
        r.backward_2d(dL)
        mark(4)
        gs.gs_preprocess_bwd(r.cam, r.settings, r.deg, p["means"], p["log_scales"], p["quats"],
                             p["opacity_logits"], p["sh"], r.tiles_touched, r.clamp, r.grad2d, g3["means"],
                             g3["log_scales"], g3["quats"], g3["opacity_logits"], g3["sh"])
        mark(5)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        run(evs[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    assert int(r.overflow.item()) == 0, "list capacity overflow during timing"
    p_fwd, p_bwd, p_blend = (float(x) for x in r.count_pairs().cpu().numpy())
    stage_ms = {n: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)]))
                for j, n in enumerate(stages)}
    ev_ms = float(np.mean([evs[i][0].elapsed_time(evs[i][5]) for i in range(steps)]))
    peaks = measure_peaks()
    K = float(r.num_keys.item())
    out = dict(metric=METRIC, value=(p_fwd + p_bwd) / (ms * 1e-3), unit="blend pairs/s", n_gpus=1, steps=steps,
               warmup=warmup, ms_per_step=round(ms, 4), higher_is_better=True, scaling="weak", vs_baseline=None,
               dtype="f32", data="synthetic",
               config=dict(workload=f"{name}: {sc.n} Gaussians, {sc.cam.width}x{sc.cam.height}, SH {sc.sh_degree}; "
                                    "rasterizer fwd + bwd to the 3D gradients, no optimizer",
                           gaussians=sc.n, width=sc.cam.width, height=sc.cam.height, sh_degree=sc.sh_degree,
                           tile=16, parallelism="single-gpu"),
               event_ms=round(ev_ms, 4), stage_ms={k: round(v, 4) for k, v in stage_ms.items()},
               pairs=dict(fwd_evaluated=p_fwd, bwd_walked=p_bwd, blended=p_blend, keys=int(K)),
               roofline=raster_roofline(sc.n, K, sc.sh_degree, p_fwd, p_bwd, p_blend, ev_ms, peaks), peaks=peaks)
    print(json.dumps(out))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the library runs on a "
              "single MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch
    from differentiable_gaussian_splatting_dgs_amd import scenes
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload != "train1m":
        rasterizer_workload(args.workload, args.steps, args.warmup)
        return
    t_gen = time.time()
    sc = scenes.training1m()
    print(f"# scene {sc.name}: n={sc.n} {sc.cam.width}x{sc.cam.height} ({time.time() - t_gen:.1f}s)", file=sys.stderr,
          flush=True)
    st = Step(sc, overlap=args.overlap)
    if args.copy_calibration_mb:
        src = torch.empty(args.copy_calibration_mb * (1 << 20) // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()
    st.run(check=True)             # sizes the list capacity
    for _ in range(max(0, args.warmup - 1)):
        st.run()
    st.finish()
    torch.cuda.synchronize()
    c0 = st.rast.count_pairs().cpu().numpy()
    nst = len(st.stages)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        st.run(events=evs[i])
    st.finish()                    # the last step's SH update belongs to the timed steps
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert int(st.rast.overflow.item()) == 0, "list capacity overflow during timing"
    c1 = st.rast.count_pairs().cpu().numpy()
    torch.cuda.synchronize()
    # the rasterizer's own 2D->3D backward (gradients written, no Adam), timed on the same state: back-to-back
    # launches behind an untimed one, so the host's per-call cost overlaps the kernels instead of adding idle gaps
    pe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    st.preprocess_bwd()
    pe[0].record()
    for _ in range(args.steps):
        st.preprocess_bwd()
    pe[1].record()
    torch.cuda.synchronize()
    pbwd_ms = float(pe[0].elapsed_time(pe[1])) / args.steps
    entries = walked_entries(st.rast)
    dens = densify_measure(st, max(3, min(args.steps, 10)))
    mv = views_measure(sc, args.views, args.steps, args.warmup) if args.views > 1 else None
    stage_ms = {name: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]))
                for j, name in enumerate(st.stages)}
    step_ev = np.array([evs[i][0].elapsed_time(evs[i][nst]) for i in range(args.steps)])
    peaks = measure_peaks()
    ms = elapsed * 1e3 / args.steps
    counts = (c0.astype(np.float64) + c1) / 2
    p_fwd, p_bwd, p_blend = counts
    pairs = p_fwd + p_bwd
    value = pairs / (ms * 1e-3)
    # the rasterizer, forward + backward down to the 3D gradients (no optimizer; the forward carries the fused
    # per-pixel loss gradient, which the backward needs as its input)
    raster_ms = sum(stage_ms[k] for k in (st.stages[0], "bin_sort", "render_fwd_loss", "render_bwd"))
    raster_ms += pbwd_ms

    raster_roof = raster_roofline(sc.n, float(st.rast.num_keys.item()), sc.sh_degree, p_fwd, p_bwd, p_blend,
                                  raster_ms, peaks)

    # roofline of the dominant kernel (render_bwd: FP32 VALU bound)
    dom = max(("render_fwd_loss", "render_bwd"), key=lambda k: stage_ms[k])
    if dom == "render_bwd":
        flops = FLOPS_EVAL * p_bwd + FLOPS_BWD_BLEND * p_blend
    else:
        flops = FLOPS_EVAL * p_fwd + FLOPS_FWD_BLEND * p_blend
    achieved = flops / (stage_ms[dom] * 1e-3) / 1e12
    traffic = read_traffic(dom)
    roof = dict(kernel=dom, bound="alu", achieved=round(achieved, 3), peak=PEAK_FP32_TFLOPS, unit="TFLOP/s",
                frac=round(achieved / PEAK_FP32_TFLOPS, 4), traffic=traffic,
                flops_per_launch=float(flops), launch_ms=round(stage_ms[dom], 4),
                peak_measured=peaks["fp32_tflops"]["measured"],
                frac_of_measured=round(achieved / peaks["fp32_tflops"]["measured"], 4))

    out = dict(metric=METRIC, value=float(value), unit="blend pairs/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=round(ms, 4), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="f32", data="synthetic",
               config=dict(workload="train1m: 1M Gaussians, 1920x1080, SH3, cluster-mixture scene; "
                                    "fwd + L1 + bwd + densify stat + Adam",
                           gaussians=sc.n, width=sc.cam.width, height=sc.cam.height, sh_degree=sc.sh_degree,
                           tile=16, parallelism="single-gpu"),
               fwd_bwd=dict(ms=round(raster_ms, 4), pairs_per_s=float(pairs / (raster_ms * 1e-3)),
                            stages=f"{st.stages[0]} + bin_sort + render_fwd_loss + render_bwd + preprocess_bwd",
                            preprocess_bwd_ms=round(pbwd_ms, 4), roofline=raster_roof),
               stage_ms={k: round(v, 4) for k, v in stage_ms.items()},
               step_ms_events=dict(p10=round(float(np.percentile(step_ev, 10)), 4),
                                   median=round(float(np.median(step_ev)), 4),
                                   p90=round(float(np.percentile(step_ev, 90)), 4)),
               blend=dict(fwd_pairs_per_s=float(p_fwd / (stage_ms["render_fwd_loss"] * 1e-3)),
                          bwd_pairs_per_s=float(p_bwd / (stage_ms["render_bwd"] * 1e-3)),
                          bwd_walked_entries=entries, bwd_float_atomics=9 * entries,
                          bwd_atomics_per_s=float(9 * entries / (stage_ms["render_bwd"] * 1e-3))),
               peaks=peaks,
               schedule={"none": "one stream",
                         "color": "two streams: the SH colour pass runs on a second stream while the main stream "
                                  "projects and bins; stage_ms are main-stream intervals",
                         "sh": "two streams: the SH colour pass and the previous step's SH Adam update run on a "
                               "second stream while the main stream projects and bins; stage_ms are main-stream "
                               "intervals"}[st.overlap or "none"],
               pairs=dict(fwd_evaluated=float(p_fwd), bwd_walked=float(p_bwd), blended=float(p_blend),
                          keys=int(st.rast.num_keys.item())),
               roofline=roof,
               densify=dens)
    if mv is not None:
        out["views"] = mv
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        cb = cpu_baseline(sc, args.cpu_tile_fraction)
        out["cpu_baseline"] = dict(value=float(pairs / cb["est_step_s"]), unit="blend pairs/s", cores=1,
                                   kind="oracle",
                                   sample=(f"float64 C oracle, single thread, {platform.processor() or 'x86_64'}: "
                                           f"full preprocess+binning, fwd/L1/bwd over {cb['tile_fraction']:.0%} of "
                                           f"tiles, 2D->3D bwd/densify/Adam over {cb['gauss_fraction']:.0%} of "
                                           f"Gaussians; {cb['work_s']:.1f}s of work, stage times scaled to the "
                                           f"full step ({cb['est_step_s']:.1f}s)"),
                                   stage_s=cb["stage_s"], host=host_cpu())
    print(json.dumps(out))


if __name__ == "__main__":
    main()
