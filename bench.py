"""Benchmark of the differentiable tile rasterizer on one MI355X.

The default line is the rasterizer's forward + backward on the 1M-Gaussian
1920x1080 cluster-mixture scene (clusters1m) with an N(0,1) upstream gradient
dL/dpixel: preprocess, binning + depth sort, forward compositing, reverse-walk
backward and the 2D->3D backward that writes the gradients of all five
parameter groups.  No optimizer, so the scene does not drift between steps.
Inputs are resident in HBM before timing starts.  `ms_per_step` is the host
clock over the timed steps (bracketed by device synchronisation); `value` is
Gaussian-pixel blend pairs per second, (evaluated forward pairs + walked
backward pairs) / step time, with both pair counts taken on the GPU.

Beside it, as extra fields of the same line: `train1m` (the full training step
on the same scene: forward with the L1 loss fused in, backward, the fused
2D->3D backward + densification statistic + Adam), `densify` (the densify /
split / clone / prune pass, run every 100 training steps), `views` (a batched
training step over several orbit views) and the CPU oracle's rate on the same
fwd+bwd (`cpu_baseline`).  --workload NAME prints the line of another scene.
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

# Algorithmic work per pair, the scope table's figures (an exp or a divide
# counts as one operation):
#   forward: about 19 flops + 1 exp per evaluated pair                       -> 20
#   backward: about 70 flops + 1 exp + 1 div per walked pair that blends     -> 72
#             about 15 flops + 1 exp per walked pair that does not blend     -> 16
FLOPS_FWD_PAIR = 20
FLOPS_BWD_BLENDED, FLOPS_BWD_SKIPPED = 72, 16

RASTER_WORKLOADS = ("clusters1m", "tiny", "ball100k", "plane3m")
WORKLOADS = RASTER_WORKLOADS + ("train1m",)
STAGES = ("preprocess", "bin_sort", "render_fwd", "render_bwd", "preprocess_bwd")
EXTRAS = ("record16", "train", "densify", "views")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the rasterizer line: no record16, training step, densify or views fields")
    ap.add_argument("--extras", default=",".join(EXTRAS),
                    help="comma-separated extra fields of the clusters1m line, from " + ", ".join(EXTRAS) +
                         " (densify and views need train)")
    ap.add_argument("--views", type=int, default=4,
                    help="views of the batched training step measured beside the main line (1 skips it)")
    ap.add_argument("--workload", default="clusters1m", choices=WORKLOADS,
                    help="clusters1m (the default line: 1M Gaussians at 1080p) or tiny / ball100k / plane3m: the "
                         "rasterizer's fwd+bwd on that scene; train1m: the training step as the line")
    args = ap.parse_args()
    args.extra_set = set() if args.no_extras else {e for e in args.extras.split(",") if e}
    if args.extra_set - set(EXTRAS):
        ap.error(f"unknown extras: {sorted(args.extra_set - set(EXTRAS))}")
    return args


def sha_of(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None when the summary
    is missing or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"source_sha256:\s*(\w+)", text)
    src = os.path.join(ROOT, "differentiable_gaussian_splatting_dgs_amd", "csrc", "render.hip")
    if not m_sha or m_sha.group(1) != sha_of(src):
        return None
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    return float(m_b.group(1)) if m_b else None


def measure_peaks(reps=5):
    """What this GPU delivers on the two binding resources, timed with HIP events:
    HBM with the calibration library's non-temporal copy over 1 GiB (2 GiB of
    traffic), fp32 with its FMA loop (8 independent chains per lane, 8 waves per
    SIMD).  Median of `reps` timed calls after one untimed call."""
    import torch
    from differentiable_gaussian_splatting_dgs_amd import measure
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
    t_copy = timed(lambda: measure.gs_stream_copy(src, dst))
    del src, dst
    blocks, iters = 256 * 8, 512
    out = torch.empty(blocks * measure.FMA_LOOP_THREADS, dtype=torch.float32, device="cuda")
    t_fma = timed(lambda: measure.gs_fma_loop(blocks, iters, 1.0000001, 1e-7, out))
    flops = blocks * measure.FMA_LOOP_THREADS * iters * measure.FMA_LOOP_FLOPS_PER_ITER
    return dict(hbm_gbs=dict(spec=PEAK_HBM_GBS, measured=round(8.0 * n / t_copy / 1e9, 1),
                             kernel="gs_stream_copy, 1 GiB"),
                fp32_tflops=dict(spec=PEAK_FP32_TFLOPS, measured=round(flops / t_fma / 1e12, 2),
                                 kernel="gs_fma_loop, 8 chains x 8 waves per SIMD"))


def blend_flops(p_fwd, p_bwd, p_blend):
    """Algorithmic flops of one forward and one backward blend launch."""
    return (FLOPS_FWD_PAIR * p_fwd,
            FLOPS_BWD_BLENDED * p_blend + FLOPS_BWD_SKIPPED * (p_bwd - p_blend))


def raster_roofline(N, K, deg, p_fwd, p_bwd, p_blend, raster_ms, peaks, colorjac=False):
    """The rasterizer's roofline fraction: the sum over its stages of the least time the binding peak allows
    for the stage's algorithmic bytes (preprocess, binning, 2D->3D backward) or flops (the two blends), over
    the measured fwd+bwd time; against the published peaks and against the measured ones.  colorjac: the
    preprocess also writes the 36-byte colour-direction Jacobian, which the 2D->3D backward reads instead
    of the SH coefficients."""
    hbm = PEAK_HBM_GBS * 1e9
    fl = PEAK_FP32_TFLOPS * 1e12
    sh = 4.0 * 3 * (deg + 1) ** 2
    par = 4.0 * (3 + 3 + 4 + 1) + sh                                      # parameter bytes per Gaussian
    jac = 36.0 if colorjac else 0.0
    f_fwd, f_bwd = blend_flops(p_fwd, p_bwd, p_blend)
    tmin = dict(
        preprocess=(par + 65.0 + jac) * N / hbm,                           # parameters in, 65 B records out
        bin_sort=(16 * N + 4 * 16 * N + 20 * N + 8 * K + 2 * 16 * K + 4 * K) / hbm,  # keys, 4 depth passes,
                                                                           # emission, 2 tile passes, ranges
        render_fwd=f_fwd / fl,
        render_bwd=f_bwd / fl,
        # parameters (without the SH with the Jacobian) + 36 B 2D gradients + 5 B count/clamp in, gradients out
        preprocess_bwd=((par - sh + jac if colorjac else par) + 41.0 + par) * N / hbm)
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


def kernel_roofline(stage_ms, p_fwd, p_bwd, p_blend, peaks, workload):
    """Roofline of the dominant blend kernel: its algorithmic flops per launch over its event-timed
    launch duration, against the fp32 vector peak (the blends are VALU-bound)."""
    f_fwd, f_bwd = blend_flops(p_fwd, p_bwd, p_blend)
    dom = max(("render_fwd", "render_bwd"), key=lambda k: stage_ms[k])
    flops = f_bwd if dom == "render_bwd" else f_fwd
    achieved = flops / (stage_ms[dom] * 1e-3) / 1e12
    return dict(kernel=dom, bound="alu", achieved=round(achieved, 3), peak=PEAK_FP32_TFLOPS, unit="TFLOP/s",
                frac=round(achieved / PEAK_FP32_TFLOPS, 4), traffic=read_traffic(dom, workload),
                flops_per_launch=float(flops), launch_ms=round(stage_ms[dom], 4),
                peak_measured=peaks["fp32_tflops"]["measured"],
                frac_of_measured=round(achieved / peaks["fp32_tflops"]["measured"], 4))


def walked_entries(r):
    """List entries the backward blend walks with at least one flagged quadrant (each
    costs one nine-value reduction and nine float atomics; two entries share one
    atomic instruction) and the flagged quadrants of those entries (each a 64-pixel
    recursion step).  Counted on the device from the last pass's buffers."""
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
    flags = r.contrib[:K].long()
    walked = (pos < ncmax[tile_of]) & (flags != 0)
    quads = ((flags & 1) + ((flags >> 1) & 1) + ((flags >> 2) & 1) + ((flags >> 3) & 1)) * walked
    return int(walked.sum().item()), int(quads.sum().item())


class RasterPass:
    """Buffers of the rasterizer's forward + backward on one scene.  run() enqueues one pass:
    preprocess, bin, forward (with the scene's loss fused in when it has one, else the given
    upstream gradient), backward blend, 2D->3D backward with the gradients written out."""

    def __init__(self, sc, record16=False):
        import torch
        from differentiable_gaussian_splatting_dgs_amd import gs
        self.gs, self.torch, self.sc = gs, torch, sc
        dev = "cuda"
        self.p = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in sc.params().items()}
        self.r = gs.Rasterizer(sc.cam, sc.n, sc.sh_degree, record16=record16)
        self.g3 = {k: torch.empty_like(v) for k, v in self.p.items()}
        self.loss = torch.zeros(1 + self.r.ntiles, dtype=torch.float64, device=dev)
        if sc.loss:
            self.target = torch.from_numpy(np.ascontiguousarray(sc.target)).to(dev)
            self.dL = torch.empty_like(self.target)
        else:
            self.target = None
            self.dL = torch.from_numpy(np.ascontiguousarray(sc.dL_dimage)).to(dev)

    def run(self, ev=None):
        """ev: None, or a list of events (None entries skipped) recorded at the stage boundaries
        0 preprocess 1 bin 2 forward 3 backward blend 4 2D->3D backward 5."""
        gs, r, p, g3 = self.gs, self.r, self.p, self.g3

        def mark(i):
            if ev is not None and ev[i] is not None:
                ev[i].record()
        mark(0)
        r.preprocess(p)
        mark(1)
        r.bin()
        mark(2)
        # the forward also clears the 2D-gradient buffer the backward then accumulates into
        if self.target is not None:
            r.render_loss(self.target, self.sc.loss, self.dL, self.loss, clear_grad2d=True)
        else:
            r.render(clear_grad2d=True)
        mark(3)
        r.backward_2d(self.dL, accumulate=True)
        mark(4)
        r.backward_3d(p, g3)
        mark(5)


def time_passes(run, nstages, steps, warmup, first=None, watch=None, drifts=False):
    """Warm-up, then `steps` timed passes: host clock over all of them (device synchronised on both
    sides).  An event records a stream marker that drains the pipeline (about 5 us of idle GPU
    each), so inside the timed passes events bracket only stage `watch` (the dominant kernel, for
    its launch duration); a second run of `steps` passes with events at every stage boundary gives
    the per-stage times and the per-pass percentiles.  Events are recorded on the stream the kernels
    use.  Returns (host ms per pass, per-stage ms, percentiles, ms of stage `watch` in the timed
    passes).  drifts: each pass changes the state the next one sees (a training step), so a second
    run would measure other work: then the timed passes themselves carry the events at every stage
    boundary."""
    import torch
    if first is not None:
        first()
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    if drifts:
        evs = [[mk() for _ in range(nstages + 1)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            run(evs[i])
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        stage = [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j in range(nstages)]
        step_ev = np.array([e[0].elapsed_time(e[nstages]) for e in evs])
        pct = dict(p10=round(float(np.percentile(step_ev, 10)), 4), median=round(float(np.median(step_ev)), 4),
                   p90=round(float(np.percentile(step_ev, 90)), 4))
        return ms, stage, pct, (stage[watch] if watch is not None else None)
    watched = [[mk() if j in (watch, watch + 1) else None for j in range(nstages + 1)] if watch is not None else None
               for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run(watched[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    watch_ms = (float(np.mean([w[watch].elapsed_time(w[watch + 1]) for w in watched])) if watch is not None
                else None)
    evs = [[mk() for _ in range(nstages + 1)] for _ in range(steps)]
    for i in range(steps):
        run(evs[i])
    torch.cuda.synchronize()
    stage = [float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)])) for j in range(nstages)]
    step_ev = np.array([evs[i][0].elapsed_time(evs[i][nstages]) for i in range(steps)])
    pct = dict(p10=round(float(np.percentile(step_ev, 10)), 4), median=round(float(np.median(step_ev)), 4),
               p90=round(float(np.percentile(step_ev, 90)), 4))
    return ms, stage, pct, watch_ms


def raster_line(name, steps, warmup, peaks):
    """The rasterizer's fwd+bwd on scene `name` as a bench line (without the extras)."""
    from differentiable_gaussian_splatting_dgs_amd import gs, scenes
    t_gen = time.time()
    sc = scenes.make(name)
    print(f"# scene {name}: n={sc.n} {sc.cam.width}x{sc.cam.height} ({time.time() - t_gen:.1f}s)", file=sys.stderr,
          flush=True)
    rp = RasterPass(sc)
    r = rp.r
    ms, stage, pct, bwd_ms = time_passes(rp.run, len(STAGES), steps, warmup,
                                         first=lambda: r.forward(rp.p, check=True), watch=STAGES.index("render_bwd"))
    if gs.check_bin_status(r.overflow.item()):
        raise gs.GsError("list capacity overflow during timing")
    p_fwd, p_bwd, p_blend = (float(x) for x in r.count_pairs().cpu().numpy())
    stage_ms = dict(zip(STAGES, stage))
    timed_ms = dict(stage_ms, render_bwd=bwd_ms)  # the backward blend as timed inside the timed passes
    K = float(r.num_keys.item())
    entries, quads = walked_entries(r)
    line = dict(metric=METRIC, value=(p_fwd + p_bwd) / (ms * 1e-3), unit="blend pairs/s", n_gpus=1, steps=steps,
                warmup=warmup, ms_per_step=round(ms, 4), higher_is_better=True, scaling="weak", vs_baseline=None,
                dtype="f32", data="synthetic",
                config=dict(workload=f"{name}: {sc.n} Gaussians, {sc.cam.width}x{sc.cam.height}, SH {sc.sh_degree}, "
                                     + (f"{sc.loss.upper()} loss" if sc.loss else "N(0,1) dL/dpixel")
                                     + "; rasterizer fwd + bwd to the 3D gradients, no optimizer",
                            gaussians=sc.n, width=sc.cam.width, height=sc.cam.height, sh_degree=sc.sh_degree,
                            tile=16, parallelism="single-gpu"),
                stage_ms={k: round(v, 4) for k, v in stage_ms.items()}, step_ms_events=pct,
                pairs=dict(fwd_evaluated=p_fwd, bwd_walked=p_bwd, blended=p_blend, keys=int(K)),
                blend=dict(fwd_pairs_per_s=p_fwd / (stage_ms["render_fwd"] * 1e-3),
                           bwd_pairs_per_s=p_bwd / (stage_ms["render_bwd"] * 1e-3),
                           bwd_walked_entries=entries, bwd_walked_quadrants=quads, bwd_float_atomics=9 * entries,
                           bwd_atomics_per_s=9 * entries / (stage_ms["render_bwd"] * 1e-3)),
                stage_roofline=raster_roofline(sc.n, K, sc.sh_degree, p_fwd, p_bwd, p_blend, ms, peaks,
                                               colorjac=r.colorjac is not None),
                roofline=kernel_roofline(timed_ms, p_fwd, p_bwd, p_blend, peaks, name),
                peaks=peaks)
    return line, sc


def record16_measure(sc, steps, warmup, ref):
    """The same fwd+bwd pass with 16-bit splat records (24 bytes gathered per list entry instead of
    48; conic factor, opacity and colour in binary16), timed like the main line; ref is the main
    line, for the stage-by-stage comparison."""
    import torch
    from differentiable_gaussian_splatting_dgs_amd import gs
    assert sc.loss is None, "the 16-bit record pass takes a given upstream gradient"
    rp = RasterPass(sc, record16=True)
    r = rp.r
    ms, stage, pct, bwd_ms = time_passes(rp.run, len(STAGES), steps, warmup,
                                         first=lambda: r.forward(rp.p, check=True), watch=STAGES.index("render_bwd"))
    if gs.check_bin_status(r.overflow.item()):
        raise gs.GsError("list capacity overflow during timing")
    p_fwd, p_bwd, p_blend = (float(x) for x in r.count_pairs().cpu().numpy())
    K = float(r.num_keys.item())
    stage_ms = dict(zip(STAGES, stage))
    out = dict(ms_per_step=round(ms, 4), value=(p_fwd + p_bwd) / (ms * 1e-3), unit="blend pairs/s",
               stage_ms={k: round(v, 4) for k, v in stage_ms.items()}, step_ms_events=pct,
               render_bwd_timed_ms=round(bwd_ms, 4),
               pairs=dict(fwd_evaluated=p_fwd, bwd_walked=p_bwd, blended=p_blend, keys=int(K)),
               record_bytes=24, record_bytes_float32=48,
               speedup_vs_float32={k: round(ref["stage_ms"][k] / v, 4) for k, v in stage_ms.items() if v > 0})
    out["speedup_vs_float32"]["step"] = round(ref["ms_per_step"] / ms, 4)
    del rp
    torch.cuda.empty_cache()
    return out


class TrainStep:
    """All buffers of the training step.  run() enqueues one step on one stream: preprocess, bin,
    forward with the L1 loss fused in (which also clears the 2D-gradient buffer), backward blend
    accumulating into it, then the fused 2D->3D backward + densification statistic + Adam."""
    STAGES = ("preprocess", "bin_sort", "render_fwd_loss", "render_bwd", "grad3d_densify_adam")

    def __init__(self, sc):
        import torch
        from differentiable_gaussian_splatting_dgs_amd import gs, scenes
        self.gs, self.torch, self.sc = gs, torch, sc
        dev = "cuda"
        self.p = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in sc.params().items()}
        self.target = torch.from_numpy(sc.target).to(dev)
        # the fused Adam tail reads the SH coefficients anyway: no colour-direction Jacobian
        self.rast = gs.Rasterizer(sc.cam, sc.n, sc.sh_degree, colorjac=False)
        self.dL = torch.empty_like(self.target)
        self.loss = torch.zeros(1 + self.rast.ntiles, dtype=torch.float64, device=dev)
        self.m = {k: torch.zeros_like(v) for k, v in self.p.items()}
        self.v = {k: torch.zeros_like(v) for k, v in self.p.items()}
        self.accum = torch.zeros(sc.n, dtype=torch.float32, device=dev)
        self.count = torch.zeros(sc.n, dtype=torch.int32, device=dev)
        self.lr = dict(scenes.ADAM_LR)
        self.step_no = 0

    def run(self, ev=None, check=False):
        gs, r, p = self.gs, self.rast, self.p
        self.step_no += 1

        def mark(i):
            if ev is not None and ev[i] is not None:
                ev[i].record()
        mark(0)
        r.preprocess(p)
        mark(1)
        r.bin()
        if check and gs.check_bin_status(r.overflow.item()):
            K = int(r.num_keys.item())
            r._alloc_lists(int(K * 1.25) + 1024)
            r.bin()
        mark(2)
        r.render_loss(self.target, "l1", self.dL, self.loss, clear_grad2d=True)
        mark(3)
        r.backward_2d(self.dL, accumulate=True)
        mark(4)
        gs.gs_preprocess_bwd_adam(r.cam, r.settings, r.deg, p, r.tiles_touched, r.clamp, r.grad2d, self.m,
                                  self.v, self.lr, self.step_no, densify_accum=self.accum, densify_count=self.count)
        mark(5)


def train_measure(steps, warmup):
    """The training step on train1m.  The scene is trained against a random target, so its workload
    drifts with the steps: pair counts are taken before and after the timed steps and averaged."""
    from differentiable_gaussian_splatting_dgs_amd import gs, scenes
    sc = scenes.training1m()
    st = TrainStep(sc)
    st.run(check=True)
    for _ in range(max(0, warmup - 1)):
        st.run()
    c0 = st.rast.count_pairs().cpu().numpy()
    ms, stage, pct, _ = time_passes(st.run, len(TrainStep.STAGES), steps, 0, drifts=True)
    if gs.check_bin_status(st.rast.overflow.item()):
        raise gs.GsError("list capacity overflow during timing")
    c1 = st.rast.count_pairs().cpu().numpy()
    p_fwd, p_bwd, p_blend = (c0.astype(np.float64) + c1) / 2
    out = dict(workload="train1m: the clusters1m scene, fwd + L1 loss (fused) + bwd + densification statistic + "
                        "Adam over all parameter groups with quaternion renormalisation",
               ms_per_step=round(ms, 4), pairs_per_s=float((p_fwd + p_bwd) / (ms * 1e-3)),
               stage_ms={k: round(v, 4) for k, v in zip(TrainStep.STAGES, stage)}, step_ms_events=pct,
               pairs=dict(fwd_evaluated=float(p_fwd), bwd_walked=float(p_bwd), blended=float(p_blend),
                          keys=int(st.rast.num_keys.item())))
    return out, st


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


def views_measure(views, steps, warmup):
    """A batched training step (training notes E.1: a batch of views rendered, their L1 losses
    summed, one Adam step): `views` orbit cameras around the train1m scene, each with its own
    random target, through the *_views calls.  Fresh parameters and Adam state."""
    import torch
    from differentiable_gaussian_splatting_dgs_amd import gs, scenes
    sc = scenes.training1m()
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
            if ev is not None and ev[i] is not None:
                ev[i].record()
        mark(0)
        rv.preprocess(p)
        mark(1)
        rv.bin()
        if check and gs.check_bin_status(rv.overflow.item(), "gs_bin_sort_views"):
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
    c0 = rv.count_pairs().cpu().numpy()
    ms, stage, _, _ = time_passes(run, len(stages), steps, 0, drifts=True)
    if gs.check_bin_status(rv.overflow.item(), "gs_bin_sort_views"):
        raise gs.GsError("list capacity overflow during the batched timing")
    c1 = rv.count_pairs().cpu().numpy()
    pairs = float((c0[0] + c1[0]) / 2 + (c0[1] + c1[1]) / 2)
    out = dict(workload=f"train1m x {views} views: {views} orbit cameras 8 degrees apart around the scene, "
                        f"one L1 target each, losses summed, one Adam step",
               views=views, ms_per_step=round(ms, 4), ms_per_view=round(ms / views, 4),
               pairs_per_s=float(pairs / (ms * 1e-3)), keys=int(rv.num_keys.item()),
               stage_ms={k: round(v, 4) for k, v in zip(stages, stage)})
    del rv, p, m, v2
    torch.cuda.empty_cache()
    return out


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


def cpu_baseline(sc, tile_fraction=1.0, seed=0):
    """The oracle on the same fwd+bwd, single-threaded: full preprocess and binning, forward and
    backward over a random `tile_fraction` of the tiles (all of them by default), 2D->3D backward of
    every Gaussian.  Its rate is the oracle's own pair count (evaluated + walked pairs on the tiles it
    composited) over its time, with the per-Gaussian stages counted in full."""
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
    tmask = None
    if tile_fraction < 1.0:
        tmask = np.zeros(ntiles, np.uint8)
        tmask[np.random.default_rng(seed).permutation(ntiles)[: max(1, int(tile_fraction * ntiles))]] = 1
    t0 = time.perf_counter()
    fwd = O.render_fwd(sc.cam, pre, pl, rg, s, tile_mask=tmask)
    t["fwd"] = time.perf_counter() - t0
    if sc.loss:
        t0 = time.perf_counter()
        _, dL = O.loss(sc.loss, fwd["image"], sc.target)
        t["loss"] = time.perf_counter() - t0
    else:
        dL = np.asarray(sc.dL_dimage, np.float64)
    t0 = time.perf_counter()
    g2 = O.render_bwd(sc.cam, pre, pl, rg, dL, s, tile_mask=tmask)
    t["bwd"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.preprocess_bwd(sc.cam, sc.sh_degree, params, pre["tiles_touched"], g2, s)
    t["preprocess_bwd"] = time.perf_counter() - t0
    pairs = float(fwd["counts"][0] + fwd["counts"][1])
    frac = 1.0 if tmask is None else float(tmask.mean())
    pix_s = t["fwd"] + t["bwd"] + t.get("loss", 0.0)
    est = t["preprocess"] + t["bin"] + t["preprocess_bwd"] + pix_s / frac
    return dict(value=pairs / frac / est, est_s=est, work_s=sum(t.values()), pairs=pairs, tile_fraction=frac,
                stage_s={k: round(v, 3) for k, v in t.items()})


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the library runs on a "
              "single MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    peaks = measure_peaks()
    if args.workload == "train1m":
        tr, st = train_measure(args.steps, args.warmup)
        line = dict(metric=METRIC, value=tr["pairs_per_s"], unit="blend pairs/s", n_gpus=1, steps=args.steps,
                    warmup=args.warmup, ms_per_step=tr["ms_per_step"], higher_is_better=True, scaling="weak",
                    vs_baseline=None, dtype="f32", data="synthetic",
                    config=dict(workload=tr["workload"], gaussians=st.sc.n, width=st.sc.cam.width,
                                height=st.sc.cam.height, sh_degree=st.sc.sh_degree, tile=16,
                                parallelism="single-gpu"),
                    train1m=tr, peaks=peaks)
        print(json.dumps(line))
        return
    line, sc = raster_line(args.workload, args.steps, args.warmup, peaks)
    extras = args.extra_set
    if args.workload == "clusters1m" and "record16" in extras:
        print("# 16-bit splat records ...", file=sys.stderr, flush=True)
        line["record16"] = record16_measure(sc, args.steps, args.warmup, line)
    if args.workload == "clusters1m" and "train" in extras:
        print("# training step ...", file=sys.stderr, flush=True)
        tr, st = train_measure(args.steps, args.warmup)
        line["train1m"] = tr
        if "densify" in extras:
            line["densify"] = densify_measure(st, max(3, min(args.steps, 10)))
        del st
        torch.cuda.empty_cache()
        if args.views > 1 and "views" in extras:
            print("# batched views ...", file=sys.stderr, flush=True)
            line["views"] = views_measure(args.views, args.steps, args.warmup)
    if not args.no_cpu_baseline and args.workload != "plane3m":
        print("# cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        cb = cpu_baseline(sc)
        line["cpu_baseline"] = dict(
            value=float(cb["value"]), unit="blend pairs/s", cores=1, kind="oracle",
            sample=(f"float64 C oracle, single thread, on the same {args.workload} fwd+bwd: preprocess, binning, "
                    f"forward and backward over {cb['tile_fraction']:.0%} of the tiles, 2D->3D backward of every "
                    f"Gaussian; {cb['work_s']:.1f}s of work, {cb['pairs']:.4g} oracle-counted pairs"),
            stage_s=cb["stage_s"], host=host_cpu())
    print(json.dumps(line))


if __name__ == "__main__":
    main()
