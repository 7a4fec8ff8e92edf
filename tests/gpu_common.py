"""Shared helpers of the GPU parity tests (imported only by tests marked gpu)."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest

TOL = 1e-4  # max |gpu - oracle| / max |oracle| per output tensor (fp32 gradients)


def require_gpu():
    import torch
    from cnn_backward_pass_amd import cbb
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a host without a GPU")
    cbb.lib()  # raises loudly when libcbb.so is missing: no fallback path exists
    return torch


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if scale == 0.0:
        return err
    return err / scale


def assert_close(name, got, ref, tol=TOL):
    e = rel_err(got, ref)
    assert e <= tol, f"{name}: max|err|/max|ref| = {e:.3e} > {tol:.1e}"
    return e


def assert_exact(name, got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{name}: {bad.size} elements differ, first at {bad[0]}: " \
                          f"{got.flat[bad[0]]} vs {ref.flat[bad[0]]}"


def with_batch(wl, batch):
    return dataclasses.replace(wl, batch=batch)


def expected_d_in(got, ref, saved, li):
    """The oracle's value for a workload's d_in[li]: its delta of conv li-1's output, or,
    where the runner left that block's g in it (results' "d_in_act"), that delta times
    act'(y) of conv li-1 by the oracle's own activation gradient."""
    act = got.get("d_in_act", [None] * (li + 1))[li]
    if act is None:
        return ref["d_in"][li]
    import oracle
    from cnn_backward_pass_amd import synth
    y = saved["layers"][li - 1]["y"]
    return oracle.act_backward(oracle.ACT_NAMES[act], synth.LEAKY_SLOPE, y, ref["d_in"][li])
