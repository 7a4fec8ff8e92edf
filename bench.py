"""Benchmark of the conv-block backward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = the full backward pass of all five workloads back to back (single
3x3 block, LeNet, Darknet-53 residual unit, YOLOv3 stem, YOLOv3 head), each at
its full batch: that covers every step of the path (activation, BN, conv
dW/dX/db, shortcut, route, upsample, max-pool, inner product, softmax loss).
Inputs are seeded synthetic tensors already resident in HBM when timing
starts.  ``value`` = algorithmic conv + inner-product GFLOP (dW + dX) of one step /
seconds per step.

The JSON line also carries the roofline of the dominant kernel (the stage of
one layer that takes the most time; it is timed in place inside the timed
steps with HIP events on the stream it runs on) and the CPU oracle timed on a
bounded sample of the same workloads (``cpu_baseline``).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "conv-block backward GFLOP/s (dW+dX+BN) and % of fp32-MFMA / HBM roofline"
ORDER = ["single_block", "lenet", "darknet53_residual", "yolov3_stem", "yolov3_head"]
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
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured as HIP graphs instead of eager "
                         "steps (measured no faster on MI355X: the step is GPU-bound)")
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
    if stage == "actbn_dW":
        # act/BN sums, then dW forming dz: x, delta, y, x_hat read once; dz, dW written
        nread = 1 + (c.act != "linear") + bool(c.bn)
        return 2.0 * macs, 4.0 * (in_elems + (nread + 1) * out_elems + w_elems)
    if stage == "block":
        # act/BN stage and the fused dW + dX kernel with dz formed in place: x, W and the
        # saved delta, y, x_hat read once; dW, dx written
        nread = 1 + (c.act != "linear") + bool(c.bn)
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


def time_stages(runners, torch, reps=3):
    """Time every stage of every conv layer in place (events around it, whole steps run)."""
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
                    r.step(probe=(li, stage, mark))
                    torch.cuda.synchronize()
                    ms.append(ev["a"].elapsed_time(ev["b"]))
                res.append((min(ms), name, li, stage))
    return sorted(res, reverse=True)


def capture_step(runners, torch, dom=None):
    """One step of every workload captured as HIP graphs (hipGraph, through
    torch.cuda.CUDAGraph): the step is ~60 small and large kernels, and replaying a
    graph removes the launch gaps between them.  With dom = (workload, layer, stage)
    the step is cut into three graphs -- before that stage, the stage, after it -- so
    that events recorded between their replays time the stage in every step."""
    graphs = [torch.cuda.CUDAGraph() for _ in range(3 if dom else 1)]
    cur = [0]

    def mark(target, before):
        if target:
            graphs[cur[0]].capture_end()
            cur[0] += 1
            graphs[cur[0]].capture_begin()

    capture_stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(capture_stream):
        graphs[0].capture_begin()
        for name, r in runners.items():
            r.step(probe=(dom[1], dom[2], mark) if dom and name == dom[0] else None)
        graphs[-1].capture_end()
    torch.cuda.synchronize()
    assert cur[0] == len(graphs) - 1, "the dominant stage was not captured"
    return graphs


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


def time_variants(torch, reps=10):
    """The entry points beyond the five workloads' path (the other activations, batch
    norm with fixed statistics, the shortcut between different shapes, the generic
    softmax backward, grouped and dilated convolutions), each timed on its own with
    events at a size taken from the workloads' layers; algorithmic work touch-once."""
    from cnn_backward_pass_amd import cbb
    dev = "cuda:0"
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    rn = lambda *s: torch.randn(*s, device=dev, generator=g)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
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
    return {"value": step_flops * reps / t_total / 1e9, "unit": "GFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} full step(s) of the five-workload suite at full batch, "
                      f"{step_flops * reps / 1e9:.1f} GFLOP in {t_total:.1f} s, double precision",
            "seconds": t_total, "host_cpus": os.cpu_count()}


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
    from cnn_backward_pass_amd import cbb
    cbb.lib()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.stage:
        profile_stage(args.stage, args.reps, torch)
        return
    if args.copy_bytes:
        profile_copy(args.copy_bytes, args.reps, torch)
        return
    runners = build_runners(dev)
    step_flops = sum(r.flops() for r in runners.values())
    for r in runners.values():
        r.reset()
    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        for r in runners.values():
            r.step()
    torch.cuda.synchronize()

    # Find the dominant kernel before the timed region: the longest dW, dX or fused
    # dW+dX stage (each is one kernel plus, for split reductions, a short
    # ordered-sum kernel);
    # act+BN stages are two streaming kernels of comparable size and are reported
    # separately (their longest kernel is shorter than the dominant conv kernel).
    stages = time_stages(runners, torch)
    conv_stages = [st for st in stages if st[3] in ("dW", "dX", "dWdX")]
    dom_ms, dom_name, dom_li, dom_stage = conv_stages[0]
    print(f"[bench] dominant stage {dom_name}.{dom_li}.{dom_stage} {dom_ms:.3f} ms",
          file=sys.stderr, flush=True)

    # Timed region: K steps enqueued eagerly (or, with --graph, replayed from HIP
    # graphs with the dominant stage as its own graph); the dominant stage is bracketed
    # by events on its stream in every step.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]

    def eager_step(k):
        def mark(target, before):
            if target:
                ev[k][0 if before else 1].record()
        for name, r in runners.items():
            r.step(probe=(dom_li, dom_stage, mark) if name == dom_name else None)

    if args.graph:
        g_pre, g_dom, g_post = capture_step(runners, torch, (dom_name, dom_li, dom_stage))
        for _ in range(2):  # the first replays upload the graphs
            g_pre.replay(); g_dom.replay(); g_post.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(args.steps):
        if not args.graph:
            eager_step(k)
            continue
        g_pre.replay()
        ev[k][0].record()
        g_dom.replay()
        ev[k][1].record()
        g_post.replay()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(stop)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    dom_avg_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)

    # Per-workload breakdown (outside the timed region), also from graph replays.
    per = {}
    for name, r in runners.items():
        run = r.step if not args.graph else capture_step({name: r}, torch)[0].replay
        run()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(5):
            run()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / 5
        per[name] = {"ms": round(ms, 4), "gflop": round(r.flops() / 1e9, 4),
                     "gflops": round(r.flops() / ms / 1e6, 1)}

    flops, nbytes = stage_work(runners[dom_name], dom_li, dom_stage)
    if dom_stage == "act_bn" or flops / nbytes < RIDGE:
        roof = {"bound": "hbm", "achieved": nbytes / (dom_avg_ms * 1e-3) / 1e9,
                "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / (dom_avg_ms * 1e-3) / 1e12,
                "peak": PEAK_MFMA_F32 / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # HBM bytes per launch of this stage from the committed rocprofv3 counter summary,
    # reported only while the kernel sources are the ones that were profiled.
    from cnn_backward_pass_amd import profsum
    rec = profsum.load_traffic(f"{dom_name}.{dom_li}.{dom_stage}")
    roof["traffic"] = None if rec is None else rec["traffic_bytes"]
    roof["kernel"] = f"{dom_name}.{runners[dom_name].wl.convs[dom_li].name}.{dom_stage}"
    roof["avg_ms"] = dom_avg_ms
    roof["algorithmic_flops"] = flops
    roof["algorithmic_bytes"] = nbytes

    line = {"metric": METRIC, "value": round(step_flops / (ms_per_step * 1e-3) / 1e9, 1),
            "unit": "GFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "suite of the five conv-block backward workloads at full "
                                   "batch: single_block b2@32x32, lenet b64, darknet53_residual "
                                   "b8@52x52, yolov3_stem b16@416x416, yolov3_head b8@26x26",
                       "gflop_per_step": round(step_flops / 1e9, 3), "parallelism": "none"},
            "roofline": roof, "per_workload": per,
            "stages_ms": {f"{n}.{li}.{st}": round(ms, 4) for ms, n, li, st in stages},
            "act_bn_stages": {f"{n}.{li}": _act_bn_entry(runners[n], n, li, ms)
                              for ms, n, li, st in stages if st == "act_bn" and ms > 0.015},
            # stages whose dz is formed inside a gradient kernel: the act/BN reduction,
            # the per-channel map and that kernel, timed together
            "dz_formed_stages": {f"{n}.{li}.{st}": _block_entry(runners[n], n, li, ms, st)
                                 for ms, n, li, st in stages if st in ("block", "actbn_dW")}}
    print("[bench] variants", file=sys.stderr, flush=True)
    line["variants"] = time_variants(torch)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
