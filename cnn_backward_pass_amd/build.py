"""Build libcbb.so (all HIP sources under csrc/) for gfx950 with hipcc.

    python -m cnn_backward_pass_amd.build

Compiles every time it is called: each source to an object file in parallel
(under _build/), then one link; also libcbb_calib.so (calib.hip), the peak
probes the benchmark reports against.  Flags: -O3, gfx950 only, packed-fp32
instructions disabled (they are not used by hand anywhere either).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libcbb.so")
# on-box peak probes for the benchmark (fp32 matrix loop, device copy); not the path
CALIB_SRC = os.path.join(PKG, "calib.hip")
CALIB_LIB = os.path.join(PKG, "libcbb_calib.so")
OBJ_DIR = os.path.join(os.path.dirname(PKG), "_build", "cbb")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-ffp-contract=fast", "-Wall", "-Wno-unused-result"]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd: list[str], verbose: bool) -> subprocess.CompletedProcess:
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    tag = f".{os.getpid()}"
    objs = [os.path.join(OBJ_DIR, os.path.basename(s) + tag + ".o") for s in sources()]
    jobs = max(1, min(len(objs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    calib_tmp = CALIB_LIB + f".tmp{os.getpid()}"
    cmds = [[HIPCC, *FLAGS, "-c", s, "-o", o] for s, o in zip(sources(), objs)]
    cmds.append([HIPCC, *FLAGS, "-shared", CALIB_SRC, "-o", calib_tmp])
    with ThreadPoolExecutor(jobs) as ex:
        res = list(ex.map(lambda c: _run(c, verbose), cmds))
    failed = [r for r in res if r.returncode != 0]
    for r in res:
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
    if failed:
        raise RuntimeError("hipcc failed building libcbb.so")
    tmp = LIB + f".tmp{os.getpid()}"
    r = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    for o in objs:
        os.remove(o)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed linking libcbb.so")
    os.replace(tmp, LIB)
    os.replace(calib_tmp, CALIB_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
