"""Short text summaries of rocprofv3 result databases (kernel trace, HBM byte counters).

    python -m cnn_backward_pass_amd.profsum trace --db RUN_results.db --out profiles/X.md \\
        --title "..." --cmd "rocprofv3 ... -- python bench.py ..."
    python -m cnn_backward_pass_amd.profsum traffic --stage yolov3_stem.1.dW --reps 3 \\
        --fetch F.db --write W.db --copy-fetch CF.db --copy-write CW.db --copy-bytes N \\
        --out profiles/Y.md --cmd "..." [--cmd "..."]
    python -m cnn_backward_pass_amd.profsum mfma --stage yolov3_stem.1.dX --db M.db \\
        --out profiles/Z.md --cmd "..."

``trace`` tabulates per-kernel durations of a ``--kernel-trace`` run.  ``mfma``
tabulates one ``--pmc`` run of the matrix-core counters per kernel.  ``traffic``
turns two ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of ``bench.py --stage``
into HBM bytes per launch of that stage, each counter scaled by what it reads for
a plain device copy of known size (``bench.py --copy-bytes``).  The traffic file
records a digest of the kernel sources; ``bench.py`` reports the figure only
while the sources still match it.
"""
from __future__ import annotations

import argparse
import collections
import glob
import hashlib
import json
import os
import sqlite3

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TRAFFIC_TAG = "traffic-json: "


def sources_digest() -> str:
    """sha256 over the HIP sources and headers the library is built from."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(HERE, "csrc", "*"))):
        if p.endswith((".hip", ".h")):
            h.update(os.path.basename(p).encode())
            with open(p, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    return name.split("(")[0].replace("void ", "").replace("cbb::", "")


def kernel_rows(db: str):
    con = sqlite3.connect(db)
    return con.execute("select name, grid_x, grid_y, grid_z, workgroup_x, duration, vgpr_count, "
                       "lds_size from kernels").fetchall()


def write_trace(db: str, out: str, title: str, cmd: str, top: int = 30) -> None:
    agg = collections.defaultdict(list)
    for name, gx, gy, gz, wx, dur, vgpr, lds in kernel_rows(db):
        agg[(_short(name), gx // max(wx, 1), gy, gz, vgpr, lds)].append(dur)
    tot = sum(sum(v) for v in agg.values())
    lines = [f"# {title}", "", "Command (from the repository root, one MI355X):", "", "```", cmd,
             "```", "",
             "Per kernel and launch grid (work-groups x, y, z): share of all kernel time in the "
             "run, dispatches, average and median duration in microseconds.", "",
             "| share | calls | avg us | median us | grid (WGs) | VGPR | LDS B | kernel |",
             "|---|---|---|---|---|---|---|---|"]
    for (short, gx, gy, gz, vgpr, lds), d in sorted(agg.items(), key=lambda kv: -sum(kv[1]))[:top]:
        d = sorted(d)
        lines.append(f"| {sum(d) / tot * 100:.1f}% | {len(d)} | {sum(d) / len(d) / 1e3:.1f} | "
                     f"{d[len(d) // 2] / 1e3:.1f} | ({gx},{gy},{gz}) | {vgpr} | {lds} | `{short}` |")
    lines.append("")
    lines.append(f"Total kernel time {tot / 1e6:.2f} ms over {sum(len(v) for v in agg.values())} "
                 "dispatches.")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def counter_rows(db: str, counter: str):
    """[(dispatch_id, kernel name, value)] of one counter, one row per dispatch."""
    con = sqlite3.connect(db)
    cols = [d[1] for d in con.execute("pragma table_info(counters_collection)")]
    idx = {c: i for i, c in enumerate(cols)}
    per = collections.defaultdict(float)
    names = {}
    for r in con.execute("select * from counters_collection"):
        if r[idx["counter_name"]] != counter:
            continue
        did = r[idx["dispatch_id"]]
        per[did] += r[idx["value"]]
        names[did] = r[idx["kernel_name"]]
    return [(d, names[d], per[d]) for d in sorted(per)]


def _stage_kib(db: str, counter: str, stage: str):
    """Counter total (KiB) over the dispatches of the profiled stage, per kernel."""
    kinds = collections.defaultdict(lambda: [0, 0.0])
    for _, name, v in counter_rows(db, counter):
        if "cbb::" not in name:
            continue
        if not stage.endswith(("act_bn", "block", "actbn_dW")) and "actbn_" in name:
            continue   # the one act+BN pass that fills dz before the timed reps
        k = kinds[_short(name)]
        k[0] += 1
        k[1] += v
    return kinds


def _copy_kib(db: str, counter: str) -> float:
    vals = [v for _, name, v in counter_rows(db, counter) if "copyBuffer" in name]
    if not vals:
        raise SystemExit(f"{db}: no copy dispatch found")
    return max(vals)


def write_traffic(a) -> None:
    f_copy = _copy_kib(a.copy_fetch, "FETCH_SIZE")
    w_copy = _copy_kib(a.copy_write, "WRITE_SIZE")
    f_scale = a.copy_bytes / (f_copy * 1024.0)
    w_scale = a.copy_bytes / (w_copy * 1024.0)
    fetch = _stage_kib(a.fetch, "FETCH_SIZE", a.stage)
    write = _stage_kib(a.write, "WRITE_SIZE", a.stage)
    f_bytes = sum(v for _, v in fetch.values()) * 1024.0 * f_scale / a.reps
    w_bytes = sum(v for _, v in write.values()) * 1024.0 * w_scale / a.reps
    per_kernel = {k: (fetch.get(k, (0, 0.0))[1] * f_scale + write.get(k, (0, 0.0))[1] * w_scale)
                  * 1024.0 / a.reps for k in sorted(set(fetch) | set(write))}
    rec = {"stage": a.stage, "reps": a.reps, "fetch_bytes": f_bytes, "write_bytes": w_bytes,
           "traffic_bytes": f_bytes + w_bytes, "fetch_scale": f_scale, "write_scale": w_scale,
           "kernels": per_kernel, "sources": sources_digest()}
    lines = [f"# HBM traffic of {a.stage} (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Commands (from the repository root, one MI355X), one counter per run:", "", "```"]
    lines += a.cmd
    lines += ["```", "",
              f"Calibration: a plain device copy of {a.copy_bytes} bytes reads FETCH_SIZE "
              f"{f_copy:.0f} KiB and WRITE_SIZE {w_copy:.0f} KiB per dispatch, so FETCH_SIZE is "
              f"scaled by {f_scale:.3f} and WRITE_SIZE by {w_scale:.3f} to give bytes.", "",
              f"Per launch of the stage ({a.reps} launches profiled):", "",
              "| kernel | dispatches | FETCH_SIZE KiB / launch | WRITE_SIZE KiB / launch |",
              "|---|---|---|---|"]
    for k in sorted(set(fetch) | set(write)):
        fn, fv = fetch.get(k, (0, 0.0))
        wn, wv = write.get(k, (0, 0.0))
        lines.append(f"| `{k}` | {max(fn, wn)} | {fv / a.reps:.0f} | {wv / a.reps:.0f} |")
    lines += ["", f"HBM bytes per launch after scaling: read {f_bytes / 1e6:.1f} MB, write "
                  f"{w_bytes / 1e6:.1f} MB, total {(f_bytes + w_bytes) / 1e6:.1f} MB.", "",
              TRAFFIC_TAG + json.dumps(rec)]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE",
                 "SQ_BUSY_CU_CYCLES")


def dispatch_counters(db: str):
    """{dispatch_id: (kernel name, {counter: [values of its rows]})} of a --pmc run."""
    con = sqlite3.connect(db)
    cols = [d[1] for d in con.execute("pragma table_info(counters_collection)")]
    idx = {c: i for i, c in enumerate(cols)}
    out = {}
    for r in con.execute("select * from counters_collection"):
        d = out.setdefault(r[idx["dispatch_id"]], (r[idx["kernel_name"]], {}))
        d[1].setdefault(r[idx["counter_name"]], []).append(r[idx["value"]])
    return out


def mfma_rows(db: str, simds: int, xcds: int = 8):
    """Per kernel of the profiled stage: dispatches, fp32 matrix FLOPs per launch
    (SQ_INSTS_VALU_MFMA_MOPS_F32 x 512, summed over the rows of a dispatch) and the
    matrix-core busy share SQ_VALU_MFMA_BUSY_CYCLES / (GUI cycles x SIMDs).

    GRBM_GUI_ACTIVE comes back as one value per dispatch summed over the chip's
    ``xcds`` dies (8 on MI355X: a 360 us launch reads ~6.3 M cycles, eight times its
    ~786 k cycles at 2.2 GHz), so the GPU's active cycles are that value / xcds.  The
    busy counter adds 64 cycles per 32x32x2 step and SIMD, so a share of 1.0 is every
    SIMD issuing matrix work on every active cycle."""
    kinds = collections.defaultdict(lambda: [0, 0.0, 0.0, 0.0])
    for name, vals in dispatch_counters(db).values():
        if "cbb::" not in name or not all(c in vals for c in MFMA_COUNTERS[:3]):
            continue
        k = kinds[_short(name)]
        gui = sum(vals["GRBM_GUI_ACTIVE"]) / max(xcds, 1)
        k[0] += 1
        k[1] += sum(vals["SQ_INSTS_VALU_MFMA_MOPS_F32"]) * 512.0
        k[2] += sum(vals["SQ_VALU_MFMA_BUSY_CYCLES"]) / max(gui * simds, 1.0)
        k[3] += gui
    return {k: {"dispatches": v[0], "mfma_flops": v[1] / v[0], "mfma_busy": v[2] / v[0],
                "gui_active_cycles": v[3] / v[0]} for k, v in kinds.items()}


def write_mfma(a) -> None:
    rows = mfma_rows(a.db, a.simds, a.xcds)
    rec = {"stage": a.stage, "simds": a.simds, "xcds": a.xcds, "kernels": rows,
           "sources": sources_digest()}
    lines = [f"# Matrix-core counters of {a.stage} (rocprofv3 --pmc)", "",
             "Command (from the repository root, one MI355X):", "", "```", a.cmd, "```", "",
             f"Per kernel: fp32 matrix FLOPs per launch counted by the hardware "
             f"(SQ_INSTS_VALU_MFMA_MOPS_F32 x 512) and the matrix-core busy share "
             f"SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {a.xcds} dies x {a.simds} SIMDs); "
             f"GRBM_GUI_ACTIVE is read summed over the {a.xcds} dies.", "",
             "| kernel | dispatches | MFMA GFLOP / launch | matrix cores busy | GPU active cycles |",
             "|---|---|---|---|---|"]
    for k in sorted(rows, key=lambda k: -rows[k]["mfma_flops"]):
        r = rows[k]
        lines.append(f"| `{k}` | {r['dispatches']} | {r['mfma_flops'] / 1e9:.3f} | "
                     f"{r['mfma_busy'] * 100:.1f}% | {r['gui_active_cycles']:.0f} |")
    lines += ["", "mfma-json: " + json.dumps(rec)]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")


LDS_COUNTERS = ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS")


def lds_rows(db: str):
    """Per kernel of the profiled stage: dispatches, LDS instructions per launch and the
    bank-conflict share SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (cycles the LDS stalled
    on bank conflicts over cycles it was busy with indexed accesses), each counter summed
    over the rows of a dispatch."""
    kinds = collections.defaultdict(lambda: [0, 0.0, 0.0, 0.0])
    for name, vals in dispatch_counters(db).values():
        if "cbb::" not in name or not all(c in vals for c in LDS_COUNTERS):
            continue
        k = kinds[_short(name)]
        k[0] += 1
        k[1] += sum(vals["SQ_INSTS_LDS"])
        k[2] += sum(vals["SQ_LDS_BANK_CONFLICT"])
        k[3] += sum(vals["SQ_LDS_IDX_ACTIVE"])
    return {k: {"dispatches": v[0], "lds_insts": v[1] / v[0],
                "conflict_share": v[2] / v[3] if v[3] > 0 else 0.0}
            for k, v in kinds.items() if v[1] > 0}


def write_lds(a) -> None:
    lines = ["# LDS bank conflicts (rocprofv3 --pmc)", "",
             "Per kernel of each stage: LDS instructions per launch (SQ_INSTS_LDS) and the share "
             "of the LDS-busy cycles (SQ_LDS_IDX_ACTIVE) stalled on bank conflicts "
             "(SQ_LDS_BANK_CONFLICT).", ""]
    for stage, db, cmd in zip(a.stage, a.db, a.cmd):
        rows = lds_rows(db)
        lines += [f"## {stage}", "", "```", cmd, "```", "",
                  "| kernel | dispatches | LDS instructions / launch | bank-conflict share |",
                  "|---|---|---|---|"]
        for k in sorted(rows, key=lambda k: -rows[k]["lds_insts"]):
            r = rows[k]
            lines.append(f"| `{k}` | {r['dispatches']} | {r['lds_insts']:.3g} | "
                         f"{r['conflict_share'] * 100:.1f}% |")
        lines += ["", "lds-json: " + json.dumps({"stage": stage, "kernels": rows,
                                                   "sources": sources_digest()}), ""]
    with open(a.out, "w") as f:
        f.write("\n".join(lines))


def load_traffic(stage: str, profiles_dir: str | None = None):
    """Traffic record for ``stage`` whose source digest matches the current sources, else None."""
    d = profiles_dir or os.path.join(ROOT, "profiles")
    cur = sources_digest()
    for p in sorted(glob.glob(os.path.join(d, "*.md"))):
        with open(p) as f:
            for line in f:
                if line.startswith(TRAFFIC_TAG):
                    rec = json.loads(line[len(TRAFFIC_TAG):])
                    if rec.get("stage") == stage and rec.get("sources") == cur:
                        return rec
    return None


def load_kernel_traffic(workload: str, layer: int, kernel: str, profiles_dir: str | None = None):
    """HBM bytes of one launch of ``kernel`` (a launch-hook name such as "conv_dx3_s2p" or
    "conv_dw3_rows (dz formed)") in a stage of conv layer ``layer`` of ``workload``, from a
    traffic record whose source digest matches the current sources; else None."""
    d = profiles_dir or os.path.join(ROOT, "profiles")
    cur = sources_digest()
    base = kernel.split(" ")[0]
    for p in sorted(glob.glob(os.path.join(d, "*.md"))):
        with open(p) as f:
            for line in f:
                if not line.startswith(TRAFFIC_TAG):
                    continue
                rec = json.loads(line[len(TRAFFIC_TAG):])
                if rec.get("sources") != cur or not str(rec.get("stage", "")).startswith(
                        f"{workload}.{layer}."):
                    continue
                hits = [v for k, v in rec.get("kernels", {}).items() if k.split("<")[0] == base]
                if len(hits) == 1:
                    return hits[0]
    return None


def main(argv=None) -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--db", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--title", required=True)
    t.add_argument("--cmd", required=True)
    r = sub.add_parser("traffic")
    r.add_argument("--stage", required=True)
    r.add_argument("--reps", type=int, required=True)
    for k in ("fetch", "write", "copy-fetch", "copy-write", "out"):
        r.add_argument(f"--{k}", required=True)
    r.add_argument("--copy-bytes", type=int, required=True)
    r.add_argument("--cmd", action="append", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--stage", required=True)
    m.add_argument("--db", required=True)
    m.add_argument("--out", required=True)
    m.add_argument("--cmd", required=True)
    m.add_argument("--simds", type=int, default=1024, help="SIMDs on the GPU (256 CUs x 4)")
    m.add_argument("--xcds", type=int, default=8, help="dies GRBM_GUI_ACTIVE is summed over")
    ld = sub.add_parser("lds")
    ld.add_argument("--stage", action="append", required=True)
    ld.add_argument("--db", action="append", required=True)
    ld.add_argument("--cmd", action="append", required=True)
    ld.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd_name == "lds":
        write_lds(a)
    elif a.cmd_name == "trace":
        write_trace(a.db, a.out, a.title, a.cmd)
    elif a.cmd_name == "mfma":
        write_mfma(a)
    else:
        write_traffic(a)


if __name__ == "__main__":
    main()
