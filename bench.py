#!/usr/bin/env python3
"""Benchmark of one 3D Gaussian Splatting training step on one MI355X.

A step is one pass of the whole hot path for one orbit view: preprocess -> bin/sort -> forward
blend -> L1 loss -> backward blend -> preprocess backward fused with Adam, over the scene's
Gaussians, with every input already resident in HBM.  Default workload: the 4M-Gaussian gyroid
isosurface at 2048x2048 over the 448-view orbit (views taken in orbit order; targets rendered
beforehand from a second seeded Gaussian set, untimed).  By default each step's preprocess
backward also preprocesses the next view from the parameters it has just updated (one read of
them for both; the first step's view is preprocessed before the loop), so a timed step holds one
preprocess, as the plain sequence does; --separate-preprocess runs it as a call of its own.

Prints ONE JSON line on stdout (progress goes to stderr):
  value        Gaussian-pixel blends per second over the timed steps (sum of n_examined, the
               list entries each pixel's forward walk examines, / wall time)
  ms_per_step  wall time per step
  roofline     the dominant kernel (the longest single-kernel phase of the step: the fused image
               pass k_blend_step by default) against its roof, from HIP events on the launch
               stream: the method's flops (or bytes) per launch / time against the fp32 vector
               peak (or 8 TB/s), with the HBM bytes the counters measured for it
               (COUNTER_TRAFFIC) and, for the image pass, the issue rate of all its VALU
               instructions against the SIMDs' limit (COUNTER_VALU)
  cpu_baseline the CPU oracle on a bounded sample of the same step (see cpu_baseline())
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "ms per fwd+bwd+Adam step and Gaussian-pixel blends/s, 4M Gaussians @2048^2"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(phase, N, R, K, P, T, n_vis, batch=1):
    """Bytes the method itself must move per launch (reads + writes), by phase; with batch > 1
    the preprocess backward's mean over the batch's views (the first writes the accumulator, the
    middle ones read and write it, the last reads it and runs Adam)."""
    if phase == "preprocess":          # params in; 48-B record + tiles + depth key + tile rect out
        return N * (4 * R + 64)
    if phase == "forward":             # per entry: index + 36 B of record; per pixel: RGB, T, last
        return K * 40 + P * 20 + T * 8
    if phase == "loss":                # image + target in, dL/dI out
        return P * 36
    if phase == "backward_blend":      # entries + pixels (dL/dI, T, last) + one 2D gradient per Gaussian out
        return K * 40 + P * 20 + T * 8 + 36 * n_vis
    if phase == "prebwd_adam":         # params, m, v, one 2D gradient per Gaussian in; params, m, v out
        if batch > 1:
            return N * ((8 * R + (batch - 2) * 12 * R + 28 * R) / batch + 36)
        return N * (24 * R + 36)
    if phase == "prebwd_adam_next":    # as prebwd_adam, and the next view's preprocess outputs
        return alg_bytes("prebwd_adam", N, R, K, P, T, n_vis, batch) + N * 64
    if phase == "image_pass":          # the fused forward + L1 + backward blend
        return sum(alg_bytes(ph, N, R, K, P, T, n_vis) for ph in ("forward", "loss", "backward_blend"))
    return 0


# fp32 operations per (pixel, list entry) pair of the blends, counting add, mul, compare, min
# and exp as one each:
#   an evaluated pair (alpha formed at the pixel): dx, dy (2), power -(A dx^2 + C dy^2)/2 -
#     B dx dy (9), exp (1), o G (1), min with 0.99 (1), the power and 1/255 tests (2)  = 16
#   a composited pair adds, forward: T (1 - alpha) and its test (3), alpha T (1), three
#     colour FMAs (6)                                                                 = 10
#   and backward, which evaluates the pair again (16) and then: 1 - alpha, T / (1 - alpha)
#     (3), alpha T (1), dL/dalpha (11), the three running colour sums (9), dL/drgb (3),
#     dL/do and dL/dpower (2), dL/du, dL/dv (8), dL/dA, dL/dB, dL/dC (8), nine
#     accumulations (9)                                                               = 54
# The forward evaluates only the pairs whose record's conservative alpha box holds the pixel
# (blend_count[3]); the examined pairs outside it are rejected without evaluating alpha, and
# the backward evaluates only the composited pairs.  So the work credited per launch is
#   16 x evaluated + 10 x composited (forward) + (16 + 54) x composited (backward).
FLOPS_EVAL, FLOPS_FWD_BLEND, FLOPS_BWD_BLEND = 16, 10, 54
# fp32 operations of the L1 + D-SSIM loss per (pixel, channel) value, 11-tap separable windows:
#   five horizontal window sums (x, y, x^2, y^2, xy: 10 per tap) and five vertical ones (2 per
#   tap and sum): 110 + 110; SSIM and its three partials: 40; the three partial maps summed
#   horizontally and vertically: 66 + 66; the combination with x, y and the L1 sign: 8  = 400
FLOPS_SSIM = 400
# MI355X's published fp32 vector peak (packed FP32 dual issue: 256 CUs x 4 SIMDs x 16 lanes x
# 2 flops per FMA x 2 x 2.4 GHz); this library is built without packed FP32 instructions, so
# half of it is the most its kernels can issue (reported beside it)
ALU_PEAK_TFLOPS = 157.3
ALU_PEAK_NONPACKED_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12


def alg_flops(phase, examined, walked, composited, evaluated, ssim_values=0):
    """Operations performed per launch in the two blend kernels (and the D-SSIM loss): the pairs
    the kernels evaluate, not the examined pairs the box test rejects."""
    if phase == "loss":                # only the D-SSIM loss is counted (ssim_values = 3HW)
        return FLOPS_SSIM * ssim_values
    if phase == "forward":
        return FLOPS_EVAL * evaluated + FLOPS_FWD_BLEND * composited
    if phase == "backward_blend":      # evaluates the composited pairs again, back to front
        return (FLOPS_EVAL + FLOPS_BWD_BLEND) * composited
    if phase == "image_pass":          # both blends in the fused image pass
        return sum(alg_flops(ph, examined, walked, composited, evaluated) for ph in ("forward", "backward_blend"))
    return 0


# the kernel of each single-kernel phase and what bounds it: the image pass is the fused blend
# kernel plus a one-workgroup sum of the per-tile losses (a few microseconds); the separate
# forward and backward phases also run their plan and staging kernels, so their event time is
# not one kernel's
KERNEL_OF = {"preprocess": ("k_preprocess<3>", "hbm"), "image_pass": ("k_blend_step", "alu"),
             "prebwd_adam": ("k_preprocess_backward<3>", "hbm"),
             "prebwd_adam_next": ("k_preprocess_backward<3, true>", "hbm")}

# HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE passes over the workload named
# (gyroid_4m_2048), each scaled by the factor the same counter reads for a plain copy of known
# size; keyed by the SHA-256 of the kernel's source file, so a changed kernel (or another
# workload) reports null
COUNTER_TRAFFIC = {
    "preprocess": {"source": "preprocess.hip", "bytes": 1200091687,
                   "sha256": "2e44421290ff3ba679569f57331f2a8575e2df50829afcd43e503a78ae3ac4bb"},
    "image_pass": {"source": "blend.hip", "bytes": 6727245517,
                   "sha256": "68654025237fa93927d67fd1c8f920c01fbb96d229ac13f019d32e98d54f4fb7"},
    "prebwd_adam_next": {"source": "preprocess.hip", "bytes": 6199489056,
                         "sha256": "2e44421290ff3ba679569f57331f2a8575e2df50829afcd43e503a78ae3ac4bb"},
}


# VALU instructions per launch of the image pass (rocprofv3 SQ_INSTS_VALU, one wave64 instruction
# each) on the same workload, keyed like COUNTER_TRAFFIC: against what 1024 SIMDs issue in the
# launch's time (one wave64 VALU instruction per SIMD per 4 cycles at 2.4 GHz), the issue rate
# that bounds the kernel, box and mask arithmetic included
COUNTER_VALU = {
    "image_pass": {"source": "blend.hip", "insts": 643.7e6,
                   "sha256": "68654025237fa93927d67fd1c8f920c01fbb96d229ac13f019d32e98d54f4fb7"},
}
VALU_ISSUE_PER_S = 256 * 4 * 2.4e9 / 4  # wave64 VALU instructions per second, all SIMDs

COUNTER_WORKLOAD = "gyroid_4m_2048"


def counter_record(table, phase, workload):
    """The stored counter record of `phase` if it was taken on this workload and the kernel's
    source is unchanged since, else None."""
    rec = table.get(phase)
    if rec is None or workload != COUNTER_WORKLOAD:
        return None
    src = os.path.join(ROOT, "gaussian_splatting_differentiable_preprocess_amd", "csrc", rec["source"])
    import hashlib
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["sha256"]:
            return None
    return rec


def counter_traffic(phase, workload):
    rec = counter_record(COUNTER_TRAFFIC, phase, workload)
    return rec["bytes"] if rec else None


def render_targets(gsmi, torch, cfg, cams, tparams_np, targets, log_every=64):
    """Renders each view of the target Gaussian set into targets[v] (GPU forward; untimed)."""
    R, n = tparams_np.shape
    W = H = cfg.res
    tp = torch.from_numpy(tparams_np).cuda()
    buf = gsmi.StepBuffers(n, n, cfg.sh_degree, W, H, k_capacity=3 * n)
    ks = []
    for vi, cam in enumerate(cams):
        c = gsmi.make_camera(cam)
        gsmi.preprocess(buf.scene, tp, c, buf.proj)
        while True:
            try:
                K = gsmi.bin_and_sort(buf.scene, c, buf.proj, buf.ws, buf.k_capacity, buf.vals, buf.ranges)
                break
            except gsmi.GsCapacityError as e:
                buf.grow(int(e.required * 1.25) + 1024)
        gsmi.render_forward(c, n, buf.proj.splat, buf.vals, buf.ranges, (0.0, 0.0, 0.0), targets[vi], buf.T_final,
                            buf.last, buf.render_ws, k=K)
        ks.append(K)
        if vi % log_every == 0:
            log(f"  target view {vi}: K = {K}")
    torch.cuda.synchronize()
    del tp, buf
    return ks


def tile_histogram(ranges_np):
    lens = (ranges_np[:, 1].astype(np.int64) - ranges_np[:, 0].astype(np.int64))
    q = np.percentile(lens, [0, 50, 90, 99, 100]).tolist()
    edges = [0] + [2 ** k for k in range(0, 16)]
    hist = np.histogram(lens, bins=edges + [1 << 40])[0].tolist()
    return {"min": q[0], "median": q[1], "p90": q[2], "p99": q[3], "max": q[4],
            "log2_bins": {f"<{e}": h for e, h in zip(edges[1:] + ["inf"], hist)}}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, params_np, cams, budget_s=30.0):
    """The CPU oracle (test infrastructure, untouched) running whole steps of the same workload:
    preprocess, bin/sort, forward, loss (L1 against a seeded uniform target, or the seeded upstream
    dL/dI), backward blend, preprocess backward and Adam over every Gaussian and pixel.  Views in
    the order 0, 112, 224, 336 of the orbit (every view of a smaller set; the single camera
    repeated), until `budget_s` of oracle time is spent (at least one step).  Configurations of
    at most 262,144 Gaussians are also timed on one thread."""
    import oracle

    oracle.build()
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    oracle.set_num_threads(threads)
    deg, W = cfg.sh_degree, cfg.res
    V = len(cams)
    order = [0, 112, 224, 336] if V >= 448 else (list(range(V)) if V > 1 else [0] * 5)
    order = [v for v in order if v < V]
    p64 = params_np.astype(np.float64)
    up = inputs_mod().upstream_gradient(cfg, W, W).astype(np.float64) if cfg.loss == "upstream" else None
    target = None if up is not None else np.random.default_rng(cfg.index).uniform(0, 1, (W, W, 3))

    def run(nthreads, budget):
        oracle.set_num_threads(nthreads)
        times, blends, views = [], 0, []
        for v in order:
            t0 = time.perf_counter()
            out = oracle.train_step_reference(p64, deg, cams[v].flat(), W, W, target=target, upstream=up,
                                              m=np.zeros_like(p64), v=np.zeros_like(p64), t=1)
            times.append(time.perf_counter() - t0)
            blends += int(out["n_examined"].astype(np.int64).sum())
            views.append(v)
            del out
            if sum(times) >= budget:
                break
        return times, blends, views

    times, blends, views = run(threads, budget_s)
    sec = sum(times)
    res = {"value": blends / sec, "unit": "Gaussian-pixel blends/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(), "ms_per_step": round(1e3 * sec / len(times), 1),
           "sample": (f"{len(times)} whole oracle steps (views {views} of {V}; every Gaussian and pixel; "
                      f"{'seeded upstream dL/dI' if up is not None else 'L1 against a seeded uniform target'}; "
                      f"Adam included) in {sec:.1f} s on {threads} OpenMP threads, time-boxed at {budget_s:.0f} s")}
    if cfg.n <= 262144:
        t1, b1, v1 = run(1, budget_s / 2)
        res["single_thread"] = {"value": b1 / sum(t1), "ms_per_step": round(1e3 * sum(t1) / len(t1), 1),
                                "steps": len(t1)}
    oracle.set_num_threads(threads)
    return res


def inputs_mod():
    from gaussian_splatting_differentiable_preprocess_amd import inputs
    return inputs


def gpu_state():
    """Clocks and power of the GPU as rocm-smi reports them (None where it is unavailable)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"], capture_output=True, text=True,
                           timeout=20)
        return json.loads(r.stdout) if r.returncode == 0 and r.stdout.strip() else None
    except (OSError, ValueError, subprocess.SubprocessError):
        return None


def copy_calibration(mib, reps=10):
    """A plain elementwise copy (out = src * 1) of mib MiB, timed with events on the current stream."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.rand(n, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = 2 * n * 4
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "ms_per_copy": round(ms, 4),
                      "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 200 for the 16K sphere -- 200 fwd+bwd repetitions -- and the "
                         "262K torus -- its 8 views x 25 --, else one 448-view epoch)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="gyroid_4m_2048")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=30.0, help="seconds of oracle steps in the CPU baseline")
    ap.add_argument("--unfused-adam", action="store_true", help="separate Adam kernel instead of the fused one")
    ap.add_argument("--separate-preprocess", action="store_true",
                    help="preprocess each view in its own call instead of in the previous step's preprocess "
                         "backward (which reads the updated parameters once for both)")
    ap.add_argument("--separate-passes", action="store_true",
                    help="forward, L1 loss and backward blend as three calls instead of the fused image pass")
    ap.add_argument("--dssim", type=float, default=None, metavar="LAMBDA",
                    help="L1 + D-SSIM loss weighted by LAMBDA instead of L1 (the forward, the loss and the "
                         "backward blend then run as three calls)")
    ap.add_argument("--batch", type=int, default=1, metavar="BS",
                    help="views per optimizer step: each view's preprocess backward adds 1/BS of its gradient "
                         "to an accumulator and every BS-th view's runs Adam with the batch-scaled "
                         "hyper-parameters (a timed step is still one view)")
    ap.add_argument("--densify", action="store_true",
                    help="accumulate the densification statistics in every step (gs_densify_stats, its own "
                         "phase) and time one clone/split/prune pass (gs_densify) after the timed steps")
    ap.add_argument("--detail", default=None, help="write a detailed JSON record to this path")
    ap.add_argument("--views", type=int, default=0,
                    help="use only the first N orbit views (short profiling runs); default all")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain streaming copy (read MIB MiB, write MIB MiB) ten times: the "
                         "known-size kernel that scales the HBM byte counters")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs the single-GPU hot path only: one MI355X holds the whole scene "
              "(4M or 18.18M Gaussians); the multi-GPU exchange is design only. Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from gaussian_splatting_differentiable_preprocess_amd import gsmi, inputs

    gsmi.load()
    torch.cuda.set_device(0)
    cfg = inputs.CONFIGS[args.config]
    if args.steps is None:
        args.steps = 200 if cfg.n <= 262144 else 448
    upstream_mode = cfg.loss == "upstream"  # seeded dL/dI instead of a loss (the 16K sphere)
    if upstream_mode and (args.dssim is not None or args.batch > 1 or args.densify):
        raise SystemExit(f"{cfg.name} takes a seeded upstream dL/dI: no loss, batch or density control modes")
    W = H = cfg.res
    P = W * H
    T = gsmi.n_tiles(W, H)
    log(f"[bench] {cfg.name}: generating {cfg.n} Gaussians (scene) ...")
    t0 = time.time()
    params_np = inputs.gaussian_params(cfg)
    cams = inputs.cameras_for(cfg)
    if args.views:
        cams = cams[: args.views]
    V = len(cams)
    R, N = params_np.shape
    if upstream_mode:
        up_t = torch.from_numpy(inputs.upstream_gradient(cfg, W, H)).cuda()
        targets, tks = None, [3 * N]
    else:
        log(f"[bench]   {time.time() - t0:.1f} s; target set ...")
        tparams_np = inputs.gaussian_params(cfg, inputs.STREAM_TARGET)
        log(f"[bench] rendering {V} target views at {W}x{H} ...")
        targets = torch.empty((V, H, W, 3), dtype=torch.float32, device="cuda")
        tks = render_targets(gsmi, torch, cfg, cams, tparams_np, targets)
        del tparams_np

    p = torch.from_numpy(params_np).cuda()
    m = torch.zeros_like(p)
    v = torch.zeros_like(p)
    kcap = int(1.5 * max(tks)) + 4096
    buf = gsmi.StepBuffers(N, N, cfg.sh_degree, W, H, k_capacity=kcap)
    grads = torch.empty_like(p) if args.unfused_adam else None
    if args.batch > 1 and args.unfused_adam:
        raise SystemExit("--batch accumulates in the fused preprocess backward; drop --unfused-adam")
    grads_acc = torch.empty_like(p) if args.batch > 1 else None
    gcams = [gsmi.make_camera(c) for c in cams]
    blends = torch.zeros(4, dtype=torch.int64, device="cuda")
    bg = (0.0, 0.0, 0.0)
    fused = not args.separate_passes and args.dssim is None and not upstream_mode
    if args.densify and not fused:
        raise SystemExit("--densify reads the fused image pass's staged sums; drop --separate-passes / --dssim")
    dens_acc = torch.zeros(N, device="cuda") if args.densify else None
    dens_cnt = torch.zeros(N, device="cuda") if args.densify else None
    dssim_ws = (torch.empty(gsmi.loss_l1_dssim_workspace(W, H), dtype=torch.uint8, device="cuda")
                if args.dssim is not None else None)
    # the next view's preprocess runs in this step's preprocess backward (one read of the updated
    # parameters for both); the first step's view is preprocessed before the loop
    tail = fused and not args.unfused_adam and args.batch == 1 and not args.separate_preprocess
    phases = ((["bin_and_sort", "render_plan", "image_pass"] + (["densify_stats"] if args.densify else [])
               + ["prebwd_adam_next"]) if tail else
              ["preprocess", "bin_and_sort", "render_plan", "image_pass"] + (["densify_stats"] if args.densify else [])
              + ["prebwd_adam"] if fused else
              ["preprocess", "bin_and_sort", "forward"] + ([] if upstream_mode else ["loss"]) +
              ["backward_blend", "prebwd_adam"])

    ks_dev = torch.zeros(max(1, args.steps), dtype=torch.int64, device="cuda")
    kc = buf.k_capacity  # the render calls' capacity: the sort leaves K on the device

    def step(t, view, ev=None, kslot=None):
        cam = gcams[view]
        marks = iter(ev or ())

        def mark():
            e = next(marks, None)
            if e is not None:
                e.record()

        mark()
        if not tail:
            gsmi.preprocess(buf.scene, p, cam, buf.proj)
            mark()
        gsmi.bin_and_sort(buf.scene, cam, buf.proj, buf.ws, buf.k_capacity, buf.vals, buf.ranges, wait=False)
        if kslot is not None:  # this step's K, from the sort workspace's count (a device copy)
            ks_dev[kslot].copy_(buf.ws[:8].view(torch.int64)[0])
        mark()
        g2 = buf.grad2d if args.unfused_adam else None
        if fused:  # forward, L1 and backward blend in one kernel; the sums stay staged
            gsmi.render_plan(buf.scene, cam, buf.proj, buf.ranges, buf.render_ws, k=kc)
            mark()
            gsmi.render_step(buf.scene, cam, buf.proj, buf.vals, buf.ranges, bg, targets[view], buf.image,
                             buf.T_final, buf.last, buf.loss, buf.dLdI, buf.render_ws, grad2d=g2, blend_count=blends,
                             k=kc)
            mark()
            if args.densify:
                gsmi.densify_stats(buf.scene, cam, buf.proj, buf.render_ws, dens_acc, dens_cnt)
                mark()
        else:
            gsmi.render_forward(cam, N, buf.proj.splat, buf.vals, buf.ranges, bg, buf.image, buf.T_final, buf.last,
                                buf.render_ws, blend_count=blends, k=kc)
            mark()
            if upstream_mode:
                dl = up_t
            elif args.dssim is not None:
                gsmi.loss_l1_dssim(W, H, buf.image, targets[view], args.dssim, buf.loss, buf.dLdI, dssim_ws)
                dl = buf.dLdI
                mark()
            else:
                gsmi.loss_l1(3 * P, buf.image, targets[view], buf.loss, buf.dLdI, buf.loss_ws)
                dl = buf.dLdI
                mark()
            gsmi.render_backward(buf.scene, None, cam, buf.proj, buf.vals, buf.ranges, bg, buf.T_final, buf.last,
                                 dl, g2, buf.render_ws, k=kc)
            mark()
        if args.batch > 1:  # t counts views; the optimizer steps once per batch
            j = (t - 1) % args.batch
            adam = (gsmi.adam_batch(gsmi.make_adam(m, v, (t - 1) // args.batch + 1, 1e-3), args.batch)
                    if j == args.batch - 1 else None)
            gsmi.preprocess_backward_accumulate(buf.scene, p, cam, buf.proj, buf.render_ws, grads_acc, j == 0,
                                                1.0 / args.batch, adam)
            mark()
            return
        adam = gsmi.make_adam(m, v, t, 1e-3)
        if args.unfused_adam:
            gsmi.preprocess_backward(buf.scene, p, cam, buf.grad2d, grads)
            gsmi.adam_step(R * N, p, grads, adam)
        elif tail:
            gsmi.preprocess_backward_staged_next(buf.scene, p, cam, buf.proj, buf.render_ws, gcams[(view + 1) % V],
                                                 buf.proj, None, adam)
        else:
            gsmi.preprocess_backward_staged(buf.scene, p, cam, buf.proj, buf.render_ws, None, adam)
        mark()

    log(f"[bench] warmup {args.warmup} steps ...")
    if tail:  # the first step's view; each step then preprocesses the next view
        gsmi.preprocess(buf.scene, p, gcams[0], buf.proj)
    t = 0
    for w in range(args.warmup):
        t += 1
        step(t, w % V)
    torch.cuda.synchronize()
    blends.zero_()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps ...")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        t += 1
        step(t, (args.warmup + k) % V, evs[k], kslot=k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ks = [int(x) for x in ks_dev[: args.steps].cpu().tolist()]
    if max(ks) > buf.k_capacity:  # an overflowed sort renders nothing: the step is not valid
        raise SystemExit(f"K {max(ks)} exceeded the capacity {buf.k_capacity} in a timed step")
    # the device-side checks of every timed step: a bounded wait that gave up, or lists that
    # outgrew the workspace, would have left results incomplete
    flags, need = gsmi.render_status(buf.render_ws, raise_error=False)
    if flags:
        raise SystemExit(f"render status flags {flags} (need {need} intersections): timed results not valid")
    total_blends = int(blends[0].item())
    ms_per_step = wall * 1e3 / args.steps
    # the last step's split tiles (their forward runs in parallel segments) from the header
    hdr = buf.render_ws[:64].cpu().numpy().view(np.uint32)
    log(f"[bench] last view: {int(hdr[10])} split tiles, {int(hdr[11])} forward segments")
    ph_ms = {ph: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)]))
             for i, ph in enumerate(phases)}
    log("[bench] per-phase ms: " + ", ".join(f"{k} {v:.3f}" for k, v in ph_ms.items()))
    log(f"[bench] {ms_per_step:.3f} ms/step, {total_blends / wall:.4g} blends/s, K mean {np.mean(ks):.0f}")

    # roofline of the dominant kernel among the single-kernel phases (the longest kernel of the
    # step), HBM-bound: algorithmic bytes per launch / its event time against 8 TB/s
    Kmean = float(np.mean(ks))
    n_vis = N
    sums = blends.cpu().tolist()
    per_launch = [x / args.steps for x in sums]  # examined, walked, composited, evaluated per view
    single = {ph: ph_ms[ph] for ph in KERNEL_OF if ph in ph_ms}
    dom = max(single, key=single.get)
    sec = ph_ms[dom] * 1e-3
    kname, bound = KERNEL_OF[dom]
    traffic = counter_traffic(dom, cfg.name)
    bytes_alg = alg_bytes(dom, N, R, Kmean, P, T, n_vis, args.batch)
    if bound == "alu":
        work = alg_flops(dom, *per_launch)
        achieved = work / sec / 1e12
        roof = {"bound": "alu", "achieved": round(achieved, 2), "peak": ALU_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / ALU_PEAK_TFLOPS, 4),
                "frac_of_nonpacked_peak": round(achieved / ALU_PEAK_NONPACKED_TFLOPS, 4)}
        vrec = counter_record(COUNTER_VALU, dom, cfg.name)
        # the issue rate of all VALU instructions (the counters'), against the SIMDs' issue limit
        roof["valu_issue_frac"] = round(vrec["insts"] / sec / VALU_ISSUE_PER_S, 4) if vrec else None
    else:
        work = bytes_alg
        achieved = work / sec / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": traffic, "traffic_over_alg_bytes": round(traffic / bytes_alg, 2) if traffic else None,
                 # the counters' HBM bytes per launch over the launch time, against the 8 TB/s peak:
                 # the rate the hardware sustains, redundant re-reads included
                 "traffic_GBps": round(traffic / sec / 1e9, 1) if traffic else None,
                 "traffic_frac_of_hbm_peak": round(traffic / sec / 1e9 / HBM_PEAK_GBS, 4) if traffic else None,
                 "kernel": kname, "work_per_launch": work, "ms_per_launch": round(ph_ms[dom], 4)})
    per_phase = {}
    for ph in phases:
        d = {"ms": round(ph_ms[ph], 4),
             "alg_GBps": round(alg_bytes(ph, N, R, Kmean, P, T, n_vis, args.batch) / (ph_ms[ph] * 1e-3) / 1e9, 1)}
        if ph in ("forward", "backward_blend", "image_pass") or (ph == "loss" and args.dssim is not None):
            d["alg_TFLOPs"] = round(alg_flops(ph, *per_launch, ssim_values=3 * P) / (ph_ms[ph] * 1e-3) / 1e12, 3)
            if ph in ("forward", "image_pass"):  # every examined pair evaluated, as a plain walk would
                d["examined_equiv_TFLOPs"] = round(
                    alg_flops(ph, per_launch[0], per_launch[1], per_launch[2], per_launch[0]) /
                    (ph_ms[ph] * 1e-3) / 1e12, 3)
        per_phase[ph] = d
    log(f"[bench] roofline: {json.dumps(roof)}")
    # per-step event time (first mark to last) over the timed views, and the pair rates
    step_ms = np.array([evs[k][0].elapsed_time(evs[k][-1]) for k in range(args.steps)])
    step_stats = {"mean": round(float(step_ms.mean()), 4), "median": round(float(np.median(step_ms)), 4),
                  "p90": round(float(np.percentile(step_ms, 90)), 4), "min": round(float(step_ms.min()), 4),
                  "max": round(float(step_ms.max()), 4)}
    blend_ph = "image_pass" if fused else "forward"
    rates = {"examined_pairs_per_s_of_step": per_launch[0] / (ms_per_step * 1e-3),
             "composited_pairs_per_s_of_step": per_launch[2] / (ms_per_step * 1e-3),
             "examined_pairs_per_s_of_" + blend_ph: per_launch[0] / (ph_ms[blend_ph] * 1e-3)}
    if not fused:
        rates["walked_pairs_per_s_of_backward_blend"] = per_launch[1] / (ph_ms["backward_blend"] * 1e-3)
    log(f"[bench] per view: {per_launch[0]:.4g} examined, {per_launch[3]:.4g} evaluated, {per_launch[1]:.4g} walked "
        f"back, {per_launch[2]:.4g} composited (pixel, entry) pairs")

    dens = None
    if args.densify:  # one clone / split / prune pass over the statistics of the timed steps
        z = torch.randn((2, 3, N), generator=torch.Generator(device="cuda").manual_seed(5), device="cuda")
        cap = 2 * N
        outs = [torch.empty((R, cap), device="cuda") for _ in range(3)]
        dws = torch.empty(gsmi.densify_workspace(N), dtype=torch.uint8, device="cuda")
        codes = torch.empty(N, dtype=torch.int32, device="cuda")
        opts = gsmi.densify_opts(extent=cfg.bound_radius)  # the radius of a sphere holding the surface
        torch.cuda.synchronize()
        t0d = time.perf_counter()
        n_out = gsmi.densify(buf.scene, p, m, v, dens_acc, dens_cnt, z, opts, *outs, cap, dws, codes=codes)
        torch.cuda.synchronize()
        dms = (time.perf_counter() - t0d) * 1e3
        k = torch.bincount(codes.long(), minlength=4).tolist()
        dbytes = N * (12 * R + 8) + n_out * 12 * R + 24 * k[2]
        dens = {"ms_wall_incl_count_readback": round(dms, 4), "n_in": N, "n_out": n_out,
                "kept": k[0], "cloned": k[1], "split": k[2], "pruned": k[3], "alg_bytes": dbytes,
                "alg_GBps": round(dbytes / (dms * 1e-3) / 1e9, 1), "extent": opts.extent}
        log(f"[bench] densify: {json.dumps(dens)}")

    # K and tile-load statistics for the last view (untimed)
    rng_np = buf.ranges.cpu().numpy()
    hist = tile_histogram(rng_np)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline: whole steps, time-boxed ...")
        cpu = cpu_baseline(cfg, params_np, cams, budget_s=args.cpu_budget)
        log(f"[bench] CPU oracle: {cpu['ms_per_step']:.0f} ms/step on {cpu['cores']} threads ({cpu['sample']})")

    out = {
        "metric": METRIC, "value": total_blends / wall, "unit": "Gaussian-pixel blends/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "gaussians": N, "sh_degree": cfg.sh_degree, "resolution": [W, H],
                   "views": V, "loss": ("seeded upstream dL/dI" if upstream_mode else "l1" if args.dssim is None
                                        else f"l1+dssim(lambda={args.dssim})"),
                   "adam": "fused" if not args.unfused_adam else "separate", "batch": args.batch,
                   "image_pass": "fused" if fused else "separate",
                   "preprocess": "in the previous step's preprocess backward" if tail else "separate",
                   "intersections_mean": round(Kmean), "intersections_min": int(min(ks)),
                   "intersections_max": int(max(ks))},
        "roofline": roof,
        "cpu_baseline": cpu,
        "render_status_flags": flags,
    }
    if args.detail:
        with open(args.detail, "w") as f:
            json.dump(dict(out, per_phase=per_phase, step_event_ms=step_stats, pair_rates=rates,
                           pairs_per_view={"examined": per_launch[0], "walked": per_launch[1],
                                           "composited": per_launch[2], "evaluated": per_launch[3]},
                           tile_list_lengths=hist, target_K=tks, densify=dens, gpu_state=gpu_state()), f, indent=1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
