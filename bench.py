"""Benchmark of the conv-block backward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = the full backward pass of all five workloads back to back (single
3x3 block, LeNet, Darknet-53 residual unit, YOLOv3 stem, YOLOv3 head), each at
its full batch: that covers every step of the path (activation, BN, conv
dW/dX/db, shortcut, route, upsample, max-pool, inner product, softmax loss).
Inputs are seeded synthetic tensors already resident in HBM when timing
starts.  ``value`` = algorithmic conv + inner-product GFLOP (dW + dX) of one
step / seconds per step.

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
    ap.add_argument("--cpu-sample-batch", type=int, default=4)
    return ap.parse_args()


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
    return 2.0 * macs, 4.0 * (in_elems + out_elems + w_elems)


def time_stages(runners, torch, reps=3):
    """Time every stage of every conv layer in place (events around it, whole steps run)."""
    res = []
    for name, r in runners.items():
        for li in range(len(r.wl.convs)):
            for stage in ("act_bn", "dW", "dX"):
                if stage == "dX" and name == "lenet" and li == 0:
                    continue
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


def cpu_baseline(sample_batch):
    """The oracle (parity mode: double arithmetic on the fp32 inputs) on every workload at a
    reduced batch; GFLOP/s = the sample's algorithmic FLOPs / wall time."""
    import oracle
    import oracle.model as M
    from cnn_backward_pass_amd import synth
    oracle.build()
    flops = 0.0
    t_total = 0.0
    for name in ORDER:
        wl = synth.WORKLOADS[name]
        b = sample_batch if name != "lenet" else 8 * sample_batch
        import dataclasses
        wls = dataclasses.replace(wl, batch=b)
        inp = synth.inputs(name, scale_batch=b)
        saved = synth.saved_standins(name, scale_batch=b)
        t0 = time.perf_counter()
        M.workload_backward(wls, inp, saved, inp.get("delta"))
        t_total += time.perf_counter() - t0
        for li, c in enumerate(wl.convs):
            macs = b * c.out_c * c.out_h * c.out_w * c.in_c * c.k * c.k
            flops += 2.0 * macs * (1 if (name == "lenet" and li == 0) else 2)
        if name == "lenet":
            flops += sum(2.0 * 2 * b * i * o for i, o in synth.LENET_FC)
    return {"value": flops / t_total / 1e9, "unit": "GFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"all five workloads at batch {sample_batch} (LeNet {8 * sample_batch}), "
                      f"{flops / 1e9:.2f} GFLOP in {t_total:.1f} s, double precision",
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
    runners = build_runners(dev)
    step_flops = sum(r.flops() for r in runners.values())
    for r in runners.values():
        r.reset()
    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        for r in runners.values():
            r.step()
    torch.cuda.synchronize()

    # Find the dominant stage (largest in-place duration) before the timed region.
    stages = time_stages(runners, torch)
    dom_ms, dom_name, dom_li, dom_stage = stages[0]
    print(f"[bench] dominant stage {dom_name}.{dom_li}.{dom_stage} {dom_ms:.3f} ms",
          file=sys.stderr, flush=True)

    # Timed region: K steps; the dominant stage is bracketed by events in every step.
    dom_events = []

    def mark(target, before):
        if target:
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            if before:
                dom_events.append([e, None])
            else:
                dom_events[-1][1] = e

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        for name, r in runners.items():
            r.step(probe=(dom_li, dom_stage, mark) if name == dom_name else None)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(stop)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    dom_avg_ms = sum(a.elapsed_time(b) for a, b in dom_events) / len(dom_events)

    # Per-workload breakdown (outside the timed region).
    per = {}
    for name, r in runners.items():
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(5):
            r.step()
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
    roof["traffic"] = None
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
            "top_stages_ms": [[f"{n}.{li}.{st}", round(ms, 4)] for ms, n, li, st in stages[:8]]}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args.cpu_sample_batch)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
