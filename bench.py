"""Benchmark of the conv-block backward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = the full backward pass of all five workloads (single 3x3 block,
LeNet, Darknet-53 residual unit, YOLOv3 stem, YOLOv3 head), each at its full
batch: that covers every step of the path (activation, BN, conv dW/dX/db,
shortcut, route, upsample, max-pool, inner product, softmax loss).  The five
are independent, so a step enqueues the three smaller ones on a second stream
(default priority): LeNet and the single block from the start, the residual unit
once the stem's stride-2 input-gradient kernel is queued, beside the rest of the
stem and the head; an event joins it back.  ``schedule`` gives the split and the
same step on one stream.
Inputs are seeded synthetic tensors already resident in HBM when timing
starts.  ``value`` = algorithmic conv + inner-product GFLOP (dW + dX) of one step /
seconds per step.

The JSON line also carries the roofline of the dominant kernel (the longest
single dW / dX / fused dW+dX kernel of the step, found by timing every kernel
in place through the library's launch hook; inside the timed steps it is
bracketed by HIP events on the stream it runs on), every gradient kernel's
rate (``kernels``), the peaks measured on the box (``calibration``: an fp32
matrix-core loop and a 1 GiB device copy) next to the published ones, warm and
cold (L2 and the 256 MB memory-side cache flushed by a 512 MB write) step-time
medians and minima, and the CPU oracle timed on a bounded sample of the same
workloads (``cpu_baseline``).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "conv-block backward GFLOP/s (dW+dX+BN) and % of fp32-MFMA / HBM roofline"
ORDER = ["single_block", "lenet", "darknet53_residual", "yolov3_stem", "yolov3_head"]
# Workloads of a step enqueued on a second stream (they share no buffer with the others).
# SIDE_EARLY start with the step and end well before the stem reaches FORK, a kernel that
# holds every CU's work-group slots (the stem's persistent stride-2 input gradient): work
# beside it only stretches it.  SIDE_LATE wait until FORK is queued, then run beside the
# first-layer kernel and the head, which leave room.
SIDE_EARLY = ("lenet", "single_block")
SIDE_LATE = ("darknet53_residual",)
SIDE = SIDE_EARLY + SIDE_LATE
FORK = ("yolov3_stem", "conv_dx3_s2p (act/BN sums below)")
PEAK_MFMA_F32 = 157.3e12   # MI355X dense fp32 matrix, FLOP/s
PEAK_HBM = 8.0e12          # MI355X HBM3E, B/s
RIDGE = PEAK_MFMA_F32 / PEAK_HBM


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time of the oracle baseline (whole suite steps)")
    ap.add_argument("--stage", default=None,
                    help="profiling mode: run only WORKLOAD.LAYER.STAGE (e.g. yolov3_stem.1.dW) "
                         "--reps times and print its event timings; no JSON line")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="profiling mode: run a plain device copy of this many bytes --reps times "
                         "(calibrates the HBM byte counters); no JSON line")
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--protocol-runs", type=int, default=30,
                    help="steps timed one by one for the warm and the cold median / min")
    return ap.parse_args()


def profile_stage(spec, reps, torch):
    """Run one stage of one conv layer on its own, ``reps`` times (for rocprofv3 counter
    passes).  For dW / dX the layer's act+BN stage runs once first to fill dz."""
    name, li, stage = spec.split(".")
    li = int(li)
    from cnn_backward_pass_amd import synth
    from cnn_backward_pass_amd.workloads import Runner
    r = Runner(name, synth.inputs(name), synth.saved_standins(name), "cuda:0")
    r.reset()
    if stage not in ("act_bn", "block", "actbn_dW"):
        r.run_stage(li, "act_bn")
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        r.run_stage(li, stage)
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    flops, nbytes = stage_work(r, li, stage)
    print(f"[stage] {spec}: ms {' '.join(f'{m:.4f}' for m in ms)}; algorithmic "
          f"{flops / 1e9:.3f} GFLOP, {nbytes / 1e6:.1f} MB", flush=True)


def profile_copy(nbytes, reps, torch):
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"[copy] {reps} copies of {n * 4} bytes", flush=True)


def build_runners(device):
    from cnn_backward_pass_amd import synth
    from cnn_backward_pass_amd.workloads import Runner
    runners = {}
    for name in ORDER:
        runners[name] = Runner(name, synth.inputs(name), synth.saved_standins(name), device)
    return runners


def stage_work(runner, li, stage):
    """(flops, bytes) of one stage of conv layer li, algorithmic (touch-once)."""
    c = runner.wl.convs[li]
    n = runner.convs[li]["desc"].batch
    out_elems = n * c.out_c * c.out_h * c.out_w
    in_elems = n * c.in_c * c.in_h * c.in_w
    w_elems = c.out_c * c.in_c * c.k * c.k
    macs = out_elems * c.in_c * c.k * c.k
    if stage == "act_bn":
        # reads delta, y, x_hat and writes dz (BN); bias-only: reads delta (+ y)
        per = (16 if c.bn else (12 if c.act != "linear" else 4))
        return 0.0, float(per * out_elems)
    # delta, y (unless linear, or the delta already holds g), x_hat
    nread = 1 + (runner.convs[li]["y"] is not None) + bool(c.bn)
    if stage == "actbn_dW":
        # act/BN sums, then dW forming dz: x, delta, y, x_hat read once; dz, dW written
        return 2.0 * macs, 4.0 * (in_elems + (nread + 1) * out_elems + w_elems)
    if stage == "block":
        # act/BN stage and the fused dW + dX kernel with dz formed in place: x, W and the
        # saved delta, y, x_hat read once; dW, dx written
        return 4.0 * macs, 4.0 * (2 * in_elems + nread * out_elems + 2 * w_elems)
    if stage == "dWdX":  # both gradients from one read of dz: x, dz, W read; dW, dx written
        return 4.0 * macs, 4.0 * (2 * in_elems + out_elems + 2 * w_elems)
    return 2.0 * macs, 4.0 * (in_elems + out_elems + w_elems)


def _act_bn_entry(runner, name, li, ms):
    """An act+BN stage: algorithmic (touch-once) GB/s and, where the committed counter
    summary matches the current sources, the HBM bytes it actually moved per second."""
    from cnn_backward_pass_amd import profsum
    e = {"ms": round(ms, 4),
         "algorithmic_GBps": round(stage_work(runner, li, "act_bn")[1] / (ms * 1e-3) / 1e9, 1)}
    rec = profsum.load_traffic(f"{name}.{li}.act_bn")
    if rec is not None:
        e["traffic_bytes"] = rec["traffic_bytes"]
        e["traffic_GBps"] = round(rec["traffic_bytes"] / (ms * 1e-3) / 1e9, 1)
        e["traffic_frac_of_hbm_peak"] = round(e["traffic_GBps"] / (PEAK_HBM / 1e9), 4)
    return e


def _block_entry(runner, name, li, ms, stage):
    """A stage in which a gradient kernel forms dz ("block": the fused dW + dX kernel;
    "actbn_dW": the dW kernel, which also writes dz): roofline of the stage (touch-once
    bytes) and, where the counter summary matches, its measured HBM bytes."""
    from cnn_backward_pass_amd import profsum
    e = _roof(ms, *stage_work(runner, li, stage))
    rec = profsum.load_traffic(f"{name}.{li}.{stage}")
    if rec is not None:
        e["traffic_bytes"] = rec["traffic_bytes"]
        e["traffic_GBps"] = round(rec["traffic_bytes"] / (ms * 1e-3) / 1e9, 1)
    return e


def time_stages(runners, torch, blocker, reps=3):
    """Time every stage of every conv layer in place (events around it, whole steps run
    behind the ~10 ms matrix-core loop, so that a short stage's time is its kernels' and
    not the host's enqueue latency)."""
    res = []
    for name, r in runners.items():
        for li in range(len(r.wl.convs)):
            for stage in r.stages(li):
                ms = []
                for _ in range(reps):
                    ev = {}

                    def mark(target, before, ev=ev):
                        if target:
                            e = torch.cuda.Event(enable_timing=True)
                            e.record()
                            ev["a" if before else "b"] = e
                    torch.cuda.synchronize()
                    blocker()
                    r.step(probe=(li, stage, mark))
                    torch.cuda.synchronize()
                    ms.append(ev["a"].elapsed_time(ev["b"]))
                res.append((min(ms), name, li, stage))
    return sorted(res, reverse=True)


# ----------------------------------------------------------------------------- peaks on the box
class Calib:
    """libcbb_calib.so: an fp32 matrix-core loop and a device copy (measurement only)."""

    def __init__(self, torch, dev):
        path = os.path.join(ROOT, "cnn_backward_pass_amd", "libcbb_calib.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build()")
        self.lib = ctypes.CDLL(path)
        self.lib.calib_mfma_f32.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                            ctypes.c_void_p]
        self.lib.calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        self.torch = torch
        self.blocks = 1024            # 4 work-groups of 4 waves per CU: every SIMD busy
        self.out = torch.empty(self.blocks * 256, dtype=torch.float32, device=dev)

    def _stream(self):
        return ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)

    def mfma(self, iters):
        rc = self.lib.calib_mfma_f32(self.blocks, iters, ctypes.c_void_p(self.out.data_ptr()),
                                     self._stream())
        if rc:
            raise RuntimeError("calib_mfma_f32 failed")
        return float(self.blocks) * 4 * iters * 4 * (32 * 32 * 2 * 2)   # FLOPs

    def copy(self, src, dst, blocks=0, unroll=1):
        rc = self.lib.calib_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                 src.numel() * src.element_size(), blocks, unroll, self._stream())
        if rc:
            raise RuntimeError("calib_copy failed")


def calibrate(calib, torch, dev, reps=5):
    """The fp32 matrix rate and the copy bandwidth this GPU sustains (best of ``reps``)."""
    def best(fn):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return min(ms)
    # short (~1 ms) and long (~10 ms) loops: the clock a sustained matrix load holds
    mfma = {}
    for iters in (2000, 20000):
        flops = calib.mfma(iters)
        mfma[iters] = flops / (best(lambda: calib.mfma(iters)) * 1e-3) / 1e12
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    copy = {}
    for blocks, unroll in ((0, 1), (8192, 1), (8192, 2), (4096, 4), (16384, 2)):
        t = best(lambda: calib.copy(src, dst, blocks, unroll))
        copy[f"{blocks or 'one-pass'}x{unroll}"] = 2.0 * (1 << 30) / (t * 1e-3) / 1e9
    del src, dst
    return {"mfma_f32_TFLOPs": round(max(mfma.values()), 2),
            "copy_GBps": round(max(copy.values()), 1),
            "mfma_by_iters": {str(k): round(v, 2) for k, v in mfma.items()},
            "copy_by_variant": {k: round(v, 1) for k, v in copy.items()},
            "mfma_probe": f"{calib.blocks} work-groups x 4 waves, rounds of 4 independent "
                          "v_mfma_f32_32x32x2_f32 chains from registers (best variant)",
            "copy_probe": "1 GiB device-to-device copy, non-temporal 16 B pieces (bytes read + "
                          "written; best of grid x pieces-in-flight variants)",
            "published": {"mfma_f32_TFLOPs": PEAK_MFMA_F32 / 1e12, "hbm_GBps": PEAK_HBM / 1e9}}


# ----------------------------------------------------------------------------- kernels
GRAD_KERNELS = ("conv_dw", "conv_dx", "conv1x1_dw", "conv1x1_dx", "conv_first_rows", "dwise_dw",
                "dwise_dx")


def kernel_role(kernel):
    """'dW', 'dX' or 'dWdX' for a gradient kernel of a conv layer, else None (reductions,
    act/BN passes, the layers' copy kernels)."""
    if kernel == "conv_first_rows":
        return "dWdX"
    if kernel.startswith(("conv_dw", "conv1x1_dw", "dwise_dw")) and "reduce" not in kernel:
        return "dW"
    if kernel.startswith(("conv_dx", "conv1x1_dx", "dwise_dx")):
        return "dX"
    return None


def kernel_work(runner, call, kernel):
    """(flops, bytes) of one launch of a gradient kernel, algorithmic (touch-once): the
    layer's dW and/or dX FLOPs; bytes read once and written once, including the delta, y
    and x_hat a kernel that forms dz reads, and the dz it writes."""
    role = kernel_role(kernel)
    li = next(i for i, c in enumerate(runner.wl.convs) if c.name == call)
    c, e = runner.wl.convs[li], runner.convs[li]
    n = e["desc"].batch
    out_e = n * c.out_c * c.out_h * c.out_w
    in_e = n * c.in_c * c.in_h * c.in_w
    w_e = c.out_c * c.in_c * c.k * c.k
    macs = out_e * c.in_c * c.k * c.k
    nread = 1 + (e["y"] is not None) + bool(c.bn)   # delta, y (unless not read), x_hat
    if role == "dWdX":
        zin = nread if e["form_dz"] else 1
        return 4.0 * macs, 4.0 * (2 * in_e + zin * out_e + 2 * w_e)
    if role == "dW" and e["dw_forms_dz"] and "dz formed" in kernel:
        return 2.0 * macs, 4.0 * (in_e + (nread + 1) * out_e + w_e)
    if role == "dX" and "sums below" in kernel:
        # also reads the block below's y and x_hat (dx's shape) for its act/BN sums
        return 2.0 * macs, 4.0 * (3 * in_e + out_e + w_e)
    return 2.0 * macs, 4.0 * (in_e + out_e + w_e)


def time_kernels(runners, torch, blocker, reps=3):
    """Every kernel of one step of every workload, timed in place: the step is enqueued
    behind a ~10 ms matrix-core loop (so its kernels then run back to back, as in the
    timed steps) with an event recorded after each kernel by the launch hook.  Returns
    [(min ms, workload, ordinal in the step, call, kernel)]."""
    rows = {}
    for name, r in runners.items():
        for _ in range(reps):
            evs = []

            def hook(call, kernel, evs=evs):
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                evs.append((call, kernel, e))
            torch.cuda.synchronize()
            blocker()
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record()
            r.step(hook=hook)
            torch.cuda.synchronize()
            prev = e0
            for i, (call, kernel, e) in enumerate(evs):
                ent = rows.setdefault((name, i), [call, kernel, []])
                if ent[1] != kernel:
                    raise RuntimeError(f"{name}: kernel {i} changed between steps")
                ent[2].append(prev.elapsed_time(e))
                prev = e
    return sorted(((min(ms), name, i, call, kernel) for (name, i), (call, kernel, ms)
                   in rows.items()), reverse=True)


def enqueue_step(runners, torch, side, hook_for=None):
    """One step of all workloads.  Stream `side` forks from the current stream at the start
    and runs SIDE_EARLY; the FORK workload goes first on the current stream, and an event
    recorded right after its FORK kernel is queued (or after the workload, should that
    kernel not run) releases SIDE_LATE on `side`; the other workloads follow on the current
    stream, and an event joins `side` back.  hook_for(name) gives the launch hook for that
    workload's step or None; a hook runs with the workload's stream current.  side=None:
    every workload on the current stream, in ORDER."""
    hook_for = hook_for or (lambda name: None)
    if side is None:
        for name, r in runners.items():
            r.step(hook=hook_for(name))
        return
    main = torch.cuda.current_stream()
    start = torch.cuda.Event()
    start.record(main)
    side.wait_event(start)
    with torch.cuda.stream(side):
        for name in SIDE_EARLY:
            runners[name].step(hook=hook_for(name))
    fork = torch.cuda.Event()
    forked = [False]
    fork_name, fork_kernel = FORK
    inner = hook_for(fork_name)

    def fork_hook(call, kernel):
        if inner is not None:
            inner(call, kernel)
        if kernel == fork_kernel and not forked[0]:
            fork.record(main)
            forked[0] = True
    runners[fork_name].step(hook=fork_hook)
    if not forked[0]:
        fork.record(main)
    side.wait_event(fork)
    with torch.cuda.stream(side):
        for name in SIDE_LATE:
            runners[name].step(hook=hook_for(name))
    for name, r in runners.items():
        if name not in SIDE and name != fork_name:
            r.step(hook=hook_for(name))
    join = torch.cuda.Event()
    join.record(side)
    main.wait_event(join)


def step_protocol(runners, torch, dev, runs, side, blocker):
    """Steps timed one at a time, each enqueued behind the ~10 ms matrix-core loop (which
    touches no memory to speak of) so that its kernels run back to back: warm, and cold (a
    512 MB write before each step, outside its events, evicts L2 and the 256 MB
    memory-side cache)."""
    flush = torch.empty(512 * (1 << 20) // 4, dtype=torch.float32, device=dev)
    out = {}
    for mode in ("warm", "cold"):
        ms = []
        for k in range(runs):
            torch.cuda.synchronize()
            if mode == "cold":
                flush.fill_(float(k))
            blocker()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            enqueue_step(runners, torch, side)
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        out[mode] = {"median_ms": round(statistics.median(ms), 4), "min_ms": round(min(ms), 4),
                     "runs": runs}
    del flush
    return out



def _roof(ms, flops, nbytes):
    """Roofline entry of one timed call: TFLOP/s against the fp32 matrix peak above the
    ridge, GB/s against HBM below it."""
    if flops / max(nbytes, 1.0) >= RIDGE:
        a = flops / (ms * 1e-3) / 1e12
        return {"ms": round(ms, 4), "bound": "mfma", "achieved": round(a, 2),
                "unit": "TFLOP/s", "frac": round(a / (PEAK_MFMA_F32 / 1e12), 4)}
    a = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "bound": "hbm", "achieved": round(a, 1), "unit": "GB/s",
            "frac": round(a / (PEAK_HBM / 1e9), 4)}


def time_variants(torch, blocker, reps=10):
    """The entry points beyond the five workloads' path (the other activations, batch
    norm with fixed statistics, the shortcut between different shapes, the generic
    softmax backward, grouped and dilated convolutions), each timed on its own with
    events at a size taken from the workloads' layers (the calls enqueued behind the
    ~10 ms matrix-core loop, so that they run back to back); algorithmic work
    touch-once."""
    from cnn_backward_pass_amd import cbb
    dev = "cuda:0"
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    rn = lambda *s: torch.randn(*s, device=dev, generator=g)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        blocker()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    out = {}
    # activation gradient (tanh) and act+BN with fixed statistics at the stem's first layer
    shp = (16, 32, 416, 416)
    cnt = 16 * 32 * 416 * 416
    y, d = torch.tanh(rn(*shp)), rn(*shp)
    gbuf = torch.empty_like(d)
    ms = timed(lambda: cbb.act_backward("tanh", 0.1, y, d, gbuf))
    out["act_backward.tanh.yolov3_stem_conv1"] = _roof(ms, 0.0, 12.0 * cnt)
    desc = cbb.conv_desc(16, 3, 416, 416, 32, 3, 1, 1, cbb.BN_FIXED, "leaky")
    xn, var, gam = rn(*shp), torch.rand(32, device=dev) + 0.5, torch.ones(32, device=dev)
    db, dg = torch.zeros(32, device=dev), torch.zeros(32, device=dev)
    ws = cbb.workspace(cbb.conv_block_workspace_size(desc), dev)
    ms = timed(lambda: cbb.conv_act_bn_backward(desc, y, xn, var, gam, d, gbuf, db, dg, ws))
    out["act_bn.fixed_statistics.yolov3_stem_conv1"] = _roof(ms, 0.0, 16.0 * cnt)
    # act+BN with batch statistics storing dz (two streaming passes) at the same size: the
    # stage the workloads' stem layers no longer run, since their gradient kernels form dz
    desc = cbb.conv_desc(16, 3, 416, 416, 32, 3, 1, 1, cbb.BN_BATCH, "leaky")
    ms = timed(lambda: cbb.conv_act_bn_backward(desc, y, xn, var, gam, d, gbuf, db, dg, ws))
    out["act_bn.batch_statistics.yolov3_stem_conv1"] = _roof(ms, 0.0, 16.0 * cnt)
    del y, d, gbuf, xn
    # shortcut into a source of half the size and channels (residual-unit delta)
    delta, dm, dfr = rn(8, 256, 52, 52), rn(8, 256, 52, 52), rn(8, 128, 26, 26)
    ms = timed(lambda: cbb.shortcut_backward_resize(delta, dm, dfr, 1.0, 1.0))
    out["shortcut_resize.256x52x52_to_128x26x26"] = _roof(
        ms, 0.0, 12.0 * delta.numel() + 12.0 * dfr.numel())
    # generic softmax backward over the head's 255 channels (strided along the channels)
    ys = torch.softmax(rn(8, 255, 26, 26), dim=1)
    dys, dxs = rn(8, 255, 26, 26), torch.empty(8, 255, 26, 26, device=dev)
    ms = timed(lambda: cbb.softmax_backward(ys, dys, dxs))
    out["softmax_backward.8x255x26x26"] = _roof(ms, 0.0, 12.0 * ys.numel())
    # grouped and dilated 3x3 convolutions at the residual unit's size (dW then dX)
    for name, c, oc, gr, dil, pad in (("depthwise_3x3", 256, 256, 256, 1, 1),
                                      ("grouped2_3x3", 256, 256, 2, 1, 1),
                                      ("dilated2_3x3", 128, 256, 1, 2, 2)):
        dsc = cbb.conv_desc(8, c, 52, 52, oc, 3, 1, pad, 0, "linear", groups=gr, dilation=dil)
        x, w = rn(8, c, 52, 52), rn(oc, c // gr, 3, 3)
        dz, dw, dx = rn(8, oc, 52, 52), torch.zeros(oc, c // gr, 3, 3, device=dev), torch.empty(
            8, c, 52, 52, device=dev)
        wsc = cbb.workspace(cbb.conv_block_workspace_size(dsc), dev)
        macs = 8.0 * oc * 52 * 52 * (c // gr) * 9
        by = 4.0 * (x.numel() + dz.numel() + w.numel())
        ms = timed(lambda: cbb.conv_backward_weights(dsc, x, dz, dw, wsc))
        out[f"conv_dW.{name}.8x{c}x52x52"] = _roof(ms, 2.0 * macs, by)
        ms = timed(lambda: cbb.conv_backward_data(dsc, w, dz, dx, False, wsc))
        out[f"conv_dX.{name}.8x{c}x52x52"] = _roof(ms, 2.0 * macs, by)
    # the parameter update after a full batch (cbb_sgd_update), over one flat buffer the
    # size of every weight, bias and BN scale of the five workloads (16 B per element)
    from cnn_backward_pass_amd import synth
    nparam = 0
    for wl in synth.WORKLOADS.values():
        for c in wl.convs:
            nparam += c.out_c * c.in_c * c.k * c.k + c.out_c * (2 if c.bn else 1)
    nparam += sum(i * o + o for i, o in synth.LENET_FC)
    pw, pg = rn(nparam), rn(nparam)
    ms = timed(lambda: cbb.sgd_update(pw, pg, 8, 1e-3, 0.9, 5e-4))
    out["sgd_update.all_parameters_of_the_five_workloads"] = _roof(ms, 0.0, 16.0 * nparam)
    del pw, pg
    # the block forward (cbb_conv_block_forward: convolution, batch statistics, BN and
    # activation in one call) at three workload layers; FLOPs of the convolution only
    for name, (n, c, hw, oc, s) in (("yolov3_stem_conv1", (16, 3, 416, 32, 1)),
                                    ("yolov3_stem_conv2", (16, 32, 416, 64, 2)),
                                    ("darknet53_residual_conv2", (8, 128, 52, 256, 1))):
        dsc = cbb.conv_desc(n, c, hw, hw, oc, 3, s, 1, 1, "leaky")
        oh = dsc.out_h
        x, w = rn(n, c, hw, hw), rn(oc, c, 3, 3) * 0.1
        gam, bet = torch.ones(oc, device=dev), torch.zeros(oc, device=dev)
        mu, va = torch.empty(oc, device=dev), torch.empty(oc, device=dev)
        xn, yy = torch.empty(n, oc, oh, oh, device=dev), torch.empty(n, oc, oh, oh, device=dev)
        wsf = cbb.workspace(cbb.conv_block_forward_workspace_size(dsc), dev)
        ms = timed(lambda: cbb.conv_block_forward(dsc, x, w, None, gam, bet, mu, va, xn, yy, wsf))
        macs = float(n) * oc * oh * oh * c * 9
        out[f"forward.{name}"] = _roof(ms, 2.0 * macs,
                                       4.0 * (x.numel() + w.numel() + 2 * xn.numel()))
        del x, xn, yy
    return out


def cpu_baseline(min_seconds=10.0, max_reps=4):
    """The oracle (double arithmetic on the fp32 inputs) on one full step of the suite at
    full batch, repeated until ``min_seconds`` of CPU time have passed (at most
    ``max_reps`` steps); GFLOP/s = the algorithmic FLOPs of the steps run / wall time."""
    import oracle
    import oracle.model as M
    from cnn_backward_pass_amd import synth
    oracle.build()
    cases = []
    step_flops = 0.0
    for name in ORDER:
        wl = synth.WORKLOADS[name]
        cases.append((wl, synth.inputs(name), synth.saved_standins(name)))
        for li, c in enumerate(wl.convs):
            macs = wl.batch * c.out_c * c.out_h * c.out_w * c.in_c * c.k * c.k
            step_flops += 2.0 * macs * (1 if (name == "lenet" and li == 0) else 2)
        if name == "lenet":
            step_flops += sum(2.0 * 2 * wl.batch * i * o for i, o in synth.LENET_FC)
    t_total, reps = 0.0, 0
    while reps < max_reps and (reps == 0 or t_total < min_seconds):
        t0 = time.perf_counter()
        for wl, inp, saved in cases:
            M.workload_backward(wl, inp, saved, inp.get("delta"))
        t_total += time.perf_counter() - t0
        reps += 1
    threads = oracle.num_threads()
    # the two small workloads on one core as well (median of three runs each)
    single = {}
    oracle.set_threads(1)
    try:
        for wl, inp, saved in cases[:2]:
            runs_flops = 0.0
            ts = []
            for _ in range(3):
                t0 = time.perf_counter()
                M.workload_backward(wl, inp, saved, inp.get("delta"))
                ts.append(time.perf_counter() - t0)
            for li, c in enumerate(wl.convs):
                macs = wl.batch * c.out_c * c.out_h * c.out_w * c.in_c * c.k * c.k
                runs_flops += 2.0 * macs * (1 if (wl.name == "lenet" and li == 0) else 2)
            if wl.name == "lenet":
                runs_flops += sum(2.0 * 2 * wl.batch * i * o for i, o in synth.LENET_FC)
            w = statistics.median(ts)
            single[wl.name] = {"value": round(runs_flops / w / 1e9, 3), "unit": "GFLOP/s",
                               "median_s": round(w, 4)}
    finally:
        oracle.set_threads(threads)
    return {"value": step_flops * reps / t_total / 1e9, "unit": "GFLOP/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{reps} full step(s) of the five-workload suite at full batch, "
                      f"{step_flops * reps / 1e9:.1f} GFLOP in {t_total:.1f} s, double precision",
            "seconds": t_total, "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(),
            "single_thread": single}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU (got --gpus {args.gpus}); the "
              "multi-GPU data-parallel path is a design note only.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    from cnn_backward_pass_amd import cbb, profsum
    cbb.lib()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.stage:
        profile_stage(args.stage, args.reps, torch)
        return
    if args.copy_bytes:
        profile_copy(args.copy_bytes, args.reps, torch)
        return
    calib = Calib(torch, dev)
    print("[bench] calibration (fp32 matrix loop, 1 GiB copy)", file=sys.stderr, flush=True)
    peaks = calibrate(calib, torch, dev)
    runners = build_runners(dev)
    step_flops = sum(r.flops() for r in runners.values())
    side = torch.cuda.Stream()   # default priority, like the current stream
    for r in runners.values():
        r.reset()
    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        enqueue_step(runners, torch, side)
    torch.cuda.synchronize()

    # Every kernel of the step timed in place, before the timed region; the dominant
    # kernel is the longest single gradient kernel (dW, dX or fused dW + dX, including
    # a dW kernel that forms dz), without its act/BN passes and split reductions.
    kern = time_kernels(runners, torch, lambda: calib.mfma(20000))   # ~10 ms blocker
    grads = [k for k in kern if kernel_role(k[4]) is not None]
    dom_ms, dom_name, dom_i, dom_call, dom_kernel = grads[0]
    print(f"[bench] dominant kernel {dom_name}.{dom_call}.{dom_kernel} (#{dom_i}) "
          f"{dom_ms:.3f} ms", file=sys.stderr, flush=True)
    stages = time_stages(runners, torch, lambda: calib.mfma(20000))

    # Timed region: K steps enqueued eagerly; the dominant kernel is bracketed by events
    # recorded (through the launch hook) after the kernel before it and after it.  (The
    # step captured as graphs split around the dominant kernel, so that events could
    # bracket it between replays, measured 1.83 ms against 1.72 eager: every graph
    # boundary drains the GPU.)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    seen = []

    def eager_step(k):
        def hook_for(name):
            if name != dom_name:
                return None
            cnt = [0]
            if dom_i == 0:
                ev[k][0].record()   # on the stream the workload runs on (current here)

            def hook(call, kernel):
                i = cnt[0]
                cnt[0] += 1
                if i == dom_i - 1:
                    ev[k][0].record()
                elif i == dom_i:
                    ev[k][1].record()
                    seen.append(kernel)
            return hook
        enqueue_step(runners, torch, side, hook_for)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(args.steps):
        eager_step(k)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(stop)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    if seen != [dom_kernel] * args.steps:
        raise RuntimeError(f"the timed steps ran {set(seen)} where {dom_kernel} was expected")
    dom_times = [a.elapsed_time(b) for a, b in ev]
    dom_avg_ms = sum(dom_times) / len(dom_times)

    print("[bench] per-workload and protocol timings", file=sys.stderr, flush=True)
    per = {}
    for name, r in runners.items():
        r.step()
        torch.cuda.synchronize()
        calib.mfma(20000)   # the five steps are enqueued before the GPU reaches them
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(5):
            r.step()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / 5
        per[name] = {"ms": round(ms, 4), "gflop": round(r.flops() / 1e9, 4),
                     "gflops": round(r.flops() / ms / 1e6, 1)}
    protocol = step_protocol(runners, torch, dev, args.protocol_runs, side,
                             lambda: calib.mfma(20000))
    # the same steps on one stream, for comparison
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        enqueue_step(runners, torch, None)
    b.record()
    torch.cuda.synchronize()
    schedule = {"side_stream_from_start": list(SIDE_EARLY),
                "side_stream_after": {".".join(FORK): list(SIDE_LATE)},
                "main_stream": [n for n in runners if n not in SIDE],
                "one_stream_ms_per_step": round(a.elapsed_time(b) / args.steps, 4)}

    def roof_of(ms, name, call, kernel):
        flops, nbytes = kernel_work(runners[name], call, kernel)
        if flops / nbytes >= RIDGE:
            ach = flops / (ms * 1e-3) / 1e12
            e = {"bound": "mfma", "achieved": ach, "peak": PEAK_MFMA_F32 / 1e12,
                 "unit": "TFLOP/s", "peak_measured": peaks["mfma_f32_TFLOPs"]}
        else:
            ach = nbytes / (ms * 1e-3) / 1e9
            e = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                 "peak_measured": peaks["copy_GBps"]}
        e["frac"] = ach / e["peak"]
        e["frac_of_measured"] = ach / e["peak_measured"]
        e["algorithmic_flops"], e["algorithmic_bytes"] = flops, nbytes
        return e

    roof = roof_of(dom_avg_ms, dom_name, dom_call, dom_kernel)
    # HBM bytes of one launch of this kernel from the committed rocprofv3 counter summary,
    # reported only while the kernel sources are the ones that were profiled.
    dom_li = next(i for i, c in enumerate(runners[dom_name].wl.convs) if c.name == dom_call)
    rec = profsum.load_kernel_traffic(dom_name, dom_li, dom_kernel)
    roof["traffic"] = None if rec is None else rec
    roof["kernel"] = f"{dom_name}.{dom_call}.{dom_kernel}"
    roof["avg_ms"] = dom_avg_ms
    roof["median_ms"] = statistics.median(dom_times)

    kernels = {}
    for ms, name, i, call, kernel in grads:
        e = roof_of(ms, name, call, kernel)
        kernels[f"{name}.{call}.{kernel}"] = {
            "ms": round(ms, 4), "bound": e["bound"], "achieved": round(e["achieved"], 2),
            "unit": e["unit"], "frac": round(e["frac"], 4),
            "frac_of_measured": round(e["frac_of_measured"], 4)}

    line = {"metric": METRIC, "value": round(step_flops / (ms_per_step * 1e-3) / 1e9, 1),
            "unit": "GFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "suite of the five conv-block backward workloads at full "
                                   "batch: single_block b2@32x32, lenet b64, darknet53_residual "
                                   "b8@52x52, yolov3_stem b16@416x416, yolov3_head b8@26x26",
                       "gflop_per_step": round(step_flops / 1e9, 3), "parallelism": "none"},
            "roofline": roof, "calibration": peaks, "protocol": protocol, "schedule": schedule,
            "per_workload": per, "kernels": kernels,
            "kernel_ms": {f"{n}#{i}.{call}.{k}": round(ms, 4)
                          for ms, n, i, call, k in sorted(kern, key=lambda t: (t[1], t[2]))},
            "stages_ms": {f"{n}.{li}.{st}": round(ms, 4) for ms, n, li, st in stages},
            "act_bn_stages": {f"{n}.{li}": _act_bn_entry(runners[n], n, li, ms)
                              for ms, n, li, st in stages if st == "act_bn" and ms > 0.015},
            # stages whose dz is formed inside a gradient kernel: the act/BN reduction,
            # the per-channel map and that kernel, timed together
            "dz_formed_stages": {f"{n}.{li}.{st}": _block_entry(runners[n], n, li, ms, st)
                                 for ms, n, li, st in stages if st in ("block", "actbn_dW")}}
    print("[bench] variants", file=sys.stderr, flush=True)
    line["variants"] = time_variants(torch, lambda: calib.mfma(20000))
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
