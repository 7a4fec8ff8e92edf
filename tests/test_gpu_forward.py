"""GPU forward of the conv block (the saved tensors of the backward) against the oracle's
double forward on the same fp32 inputs; the forward chained into the backward; and, on the
device alone, central differences of the forward against the backward's gradient."""
import types

import numpy as np
import pytest

import oracle.model as M
from gpu_common import announce, assert_close, require_gpu

pytestmark = pytest.mark.gpu

FWD_CASES = [  # n, c, h, w, oc, k, s, p, bn, act, groups, dilation
    (2, 3, 32, 32, 16, 3, 1, 1, 1, "leaky", 1, 1),       # single block
    (2, 16, 13, 11, 40, 3, 2, 1, 1, "leaky", 1, 1),      # stride 2, ragged
    (2, 64, 12, 12, 96, 1, 1, 0, 1, "logistic", 1, 1),   # 1x1
    (4, 20, 12, 12, 50, 5, 1, 0, 0, "linear", 1, 1),     # LeNet conv2 shape, bias, no BN
    (2, 1, 28, 28, 20, 5, 1, 0, 0, "relu", 1, 1),        # one input channel, bias + ReLU
    (2, 12, 10, 12, 24, 3, 1, 1, 1, "tanh", 4, 1),       # grouped
    (2, 16, 15, 14, 16, 3, 1, 2, 2, "selu", 16, 2),      # depthwise, dilated, fixed statistics
    (1, 8, 17, 16, 12, 5, 2, 4, 1, "relu", 1, 2),        # dilated 5x5, stride 2
    (3, 32, 9, 9, 48, 3, 1, 1, 2, "leaky", 1, 1),        # fixed statistics
    (2, 24, 14, 18, 130, 3, 2, 1, 1, "leaky", 1, 1),     # 128 x 128 tiles, ragged o and pixels
    (1, 32, 20, 20, 80, 3, 1, 1, 0, "relu", 1, 1),       # bias: general kernel, more than 64 o
    (2, 2, 15, 17, 24, 3, 2, 1, 1, "leaky", 1, 1),       # short reduction (J = 18), stride 2
    (1, 3, 20, 21, 32, 3, 1, 2, 0, "relu", 1, 2),        # short reduction, dilated, bias
    (2, 32, 40, 72, 64, 3, 2, 1, 1, "leaky", 1, 1),      # stride-2 tiles: 2 x 3, both ragged
    (1, 6, 34, 36, 100, 3, 2, 1, 0, "relu", 1, 1),       # stride 2: 2 chunks, 2 o blocks, bias
    (1, 6, 33, 35, 100, 3, 2, 1, 0, "relu", 1, 1),       # stride 2, width not a multiple of 4
    (3, 5, 16, 16, 20, 3, 2, 1, 1, "leaky", 1, 1),       # stride 2: odd channel count
    (2, 3, 20, 24, 32, 3, 1, 1, 2, "relu", 1, 1),        # first layer, fixed statistics
    (1, 3, 18, 19, 8, 3, 1, 1, 1, "tanh", 1, 1),         # first layer, run-time activation
]


def _layer(c, oc, k, s, p, bn, act, h, w, groups, dil):
    return types.SimpleNamespace(in_c=c, out_c=oc, k=k, stride=s, pad=p, bn=bn, act=act,
                                 in_h=h, in_w=w, groups=groups, dilation=dil)


def _inputs(case, seed):
    n, c, h, w, oc, k, s, p, bn, act, groups, dil = case
    r = np.random.default_rng(seed)
    x = r.normal(size=(n, c, h, w)).astype(np.float32)
    wt = (r.normal(size=(oc, c // groups, k, k)) * 0.2).astype(np.float32)
    gamma = (1 + 0.3 * r.normal(size=oc)).astype(np.float32) if bn else None
    beta = r.normal(size=oc).astype(np.float32) if bn else None
    bias = None if bn else r.normal(size=oc).astype(np.float32)
    mean, var = ((r.normal(size=oc).astype(np.float32), r.uniform(0.5, 2, oc).astype(np.float32))
                 if bn == 2 else (None, None))
    return x, wt, gamma, beta, bias, mean, var


def gpu_forward(torch, case, x, wt, gamma, beta, bias, mean, var):
    from cnn_backward_pass_amd import cbb
    n, c, h, w, oc, k, s, p, bn, act, groups, dil = case
    desc = cbb.conv_desc(n, c, h, w, oc, k, s, p, bn, act, groups=groups, dilation=dil)
    T = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    oshape = (n, oc, desc.out_h, desc.out_w)
    y = torch.empty(oshape, device="cuda")
    xn = torch.empty(oshape, device="cuda") if bn else None
    mu = (T(mean) if bn == 2 else torch.empty(oc, device="cuda")) if bn else None
    va = (T(var) if bn == 2 else torch.empty(oc, device="cuda")) if bn else None
    ws = cbb.workspace(cbb.conv_block_forward_workspace_size(desc))
    cbb.conv_block_forward(desc, T(x), T(wt), T(bias), T(gamma), T(beta), mu, va, xn, y, ws)
    torch.cuda.synchronize()
    h_ = lambda t: None if t is None else t.cpu().double().numpy()
    return {"y": h_(y), "xhat": h_(xn), "mean": h_(mu), "var": h_(va)}, desc


@pytest.mark.parametrize("case,offset", [(FWD_CASES[1], 40.0), (FWD_CASES[2], -25.0),
                                         ((4, 3, 64, 64, 32, 3, 1, 1, 1, "leaky", 1, 1), 60.0),
                                         ((2, 16, 40, 72, 64, 3, 2, 1, 1, "leaky", 1, 1), 40.0)])
def test_forward_statistics_with_a_large_mean(case, offset):
    """Batch statistics when the conv output's mean is large against its spread (the
    one-pass shifted sums of the statistics pass and of the first-layer kernels; the
    last case's z comes from the stride-2 tile kernel): mean, var and x_norm still match
    the oracle's two-pass double statistics."""
    torch = require_gpu()
    announce(f"forward statistics, input offset {offset}: {case}")
    n, c, h, w, oc, k, s, p, bn, act, groups, dil = case
    x, wt, gamma, beta, bias, mean, var = _inputs(case, 950)
    x = (x + np.float32(offset)).astype(np.float32)
    wt = (np.abs(wt) + np.float32(0.05)).astype(np.float32)   # same-sign weights: z far from 0
    got, _ = gpu_forward(torch, case, x, wt, gamma, beta, bias, mean, var)
    L = _layer(c, oc, k, s, p, bn, act, h, w, groups, dil)
    ref = M.conv_block_forward(L, x, wt, bias=bias, gamma=gamma, beta=beta, mean=mean, var=var)
    assert_close("mean", got["mean"], ref["mean"])
    assert_close("var", got["var"], ref["var"])
    assert_close("x_norm", got["xhat"], ref["xhat"])
    assert_close("y", got["y"], ref["y"])


@pytest.mark.parametrize("case", FWD_CASES)
def test_conv_block_forward_parity(case):
    torch = require_gpu()
    announce(f"forward {case}")
    n, c, h, w, oc, k, s, p, bn, act, groups, dil = case
    x, wt, gamma, beta, bias, mean, var = _inputs(case, 900 + FWD_CASES.index(case))
    got, _ = gpu_forward(torch, case, x, wt, gamma, beta, bias, mean, var)
    L = _layer(c, oc, k, s, p, bn, act, h, w, groups, dil)
    ref = M.conv_block_forward(L, x, wt, bias=bias, gamma=gamma, beta=beta, mean=mean, var=var)
    assert_close("y", got["y"], ref["y"])
    if bn:
        assert_close("x_norm", got["xhat"], ref["xhat"])
        assert_close("mean", got["mean"], ref["mean"])
        assert_close("var", got["var"], ref["var"])


def test_stride2_forward_full_size_stem_conv2_sampled():
    """The stem's stride-2 layer at its full batch and size (z + bias, so y is the
    convolution itself), in the launch the benchmark times: 16 x 16 output windows at the
    corners, the ragged edges and inside, against the oracle's convolution of the input
    patch under each window (pad applied to the patch, the same definition)."""
    import oracle
    torch = require_gpu()
    case = (16, 32, 416, 416, 64, 3, 2, 1, 0, "linear", 1, 1)
    announce(f"stride-2 forward full size {case}")
    x, wt, gamma, beta, bias, mean, var = _inputs(case, 78)
    got, desc = gpu_forward(torch, case, x, wt, gamma, beta, bias, mean, var)
    oh, ow = desc.out_h, desc.out_w
    for b, h0, w0 in [(0, 0, 0), (15, oh - 16, ow - 16), (7, 100, 37), (3, 0, ow - 16),
                      (11, oh - 16, 5), (5, 61, 144)]:
        xp = np.pad(x[b], ((0, 0), (1, 1), (1, 1)))
        patch = xp[:, 2 * h0:2 * h0 + 33, 2 * w0:2 * w0 + 33][None]
        ref = oracle.conv_forward(patch, wt, 2, 0, bias=bias)[0]
        assert_close(f"y window {(b, h0, w0)}", got["y"][b, :, h0:h0 + 16, w0:w0 + 16], ref)


def test_first_layer_forward_full_size_stem_conv1():
    """The stem's first layer at its full batch and size, in the launch the benchmark
    times (z computed twice, never stored: statistics, then x_norm and y), every element
    and the statistics against the oracle in double."""
    torch = require_gpu()
    case = (16, 3, 416, 416, 32, 3, 1, 1, 1, "leaky", 1, 1)
    announce(f"first-layer forward full size {case}")
    x, wt, gamma, beta, bias, mean, var = _inputs(case, 79)
    got, _ = gpu_forward(torch, case, x, wt, gamma, beta, bias, mean, var)
    L = _layer(3, 32, 3, 1, 1, 1, "leaky", 416, 416, 1, 1)
    ref = M.conv_block_forward(L, x, wt, gamma=gamma, beta=beta)
    for key in ("y", "xhat", "mean", "var"):
        assert_close(key, got[key], ref[key])


def test_conv_block_forward_full_size_residual_conv2():
    """The residual unit's 3x3 layer at its full batch, every element (the forward's largest
    contraction class), against the oracle in double."""
    torch = require_gpu()
    case = (8, 128, 52, 52, 256, 3, 1, 1, 1, "leaky", 1, 1)
    announce(f"forward full size {case}")
    x, wt, gamma, beta, bias, mean, var = _inputs(case, 77)
    got, _ = gpu_forward(torch, case, x, wt, gamma, beta, bias, mean, var)
    L = _layer(128, 256, 3, 1, 1, 1, "leaky", 52, 52, 1, 1)
    ref = M.conv_block_forward(L, x, wt, gamma=gamma, beta=beta)
    for key in ("y", "xhat", "mean", "var"):
        assert_close(key, got[key], ref[key])


@pytest.mark.parametrize("case", [FWD_CASES[0], FWD_CASES[1], FWD_CASES[5], FWD_CASES[8]])
def test_forward_then_backward_matches_oracle_chain(case):
    """GPU forward -> GPU backward (from the GPU's saved tensors) against the oracle's
    forward -> backward on the same fp32 inputs."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    announce(f"forward+backward {case}")
    n, c, h, w, oc, k, s, p, bn, act, groups, dil = case
    x, wt, gamma, beta, bias, mean, var = _inputs(case, 1200 + FWD_CASES.index(case))
    got, desc = gpu_forward(torch, case, x, wt, gamma, beta, bias, mean, var)
    L = _layer(c, oc, k, s, p, bn, act, h, w, groups, dil)
    saved = M.round_saved_to_f32(M.conv_block_forward(L, x, wt, bias=bias, gamma=gamma, beta=beta,
                                                      mean=mean, var=var))
    delta = np.random.default_rng(5).normal(size=got["y"].shape).astype(np.float32)
    ref = M.conv_block_backward(L, saved, delta)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    dw = torch.zeros(wt.shape, device="cuda")
    db = torch.zeros(oc, device="cuda")
    dg = torch.zeros(oc, device="cuda") if bn else None
    dx = torch.zeros(x.shape, device="cuda")
    dz = torch.empty(got["y"].shape, device="cuda")
    ws = cbb.workspace(cbb.conv_block_workspace_size(desc))
    cbb.conv_block_backward(desc, T(x), T(wt), T(got["y"]), T(got["xhat"]) if bn else None,
                            T(got["var"]) if bn else None, T(gamma) if bn else None, T(delta), dz,
                            dw, db, dg, dx, False, ws)
    torch.cuda.synchronize()
    assert_close("dw", dw.cpu().double().numpy(), ref["dw"])
    assert_close("db", db.cpu().double().numpy(), ref["db"])
    assert_close("dx", dx.cpu().double().numpy(), ref["dx"])
    if bn:
        assert_close("dgamma", dg.cpu().double().numpy(), ref["dgamma"])


def test_device_finite_differences_of_the_forward():
    """On the device alone: with L = sum(delta * y), the central difference of the GPU
    forward along a random direction of W agrees with <dW, v> from the GPU backward
    (batch-statistics BN, smooth activation; fp32, so a loose bound: a consistency check
    between the two halves, not a parity claim)."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    case = (2, 4, 8, 8, 8, 3, 1, 1, 1, "logistic", 1, 1)
    announce(f"device finite differences {case}")
    x, wt, gamma, beta, bias, mean, var = _inputs(case, 31)
    r = np.random.default_rng(32)
    v = r.normal(size=wt.shape).astype(np.float32)
    delta = r.normal(size=(2, 8, 8, 8)).astype(np.float32)
    loss = lambda W: float(np.sum(gpu_forward(torch, case, x, W, gamma, beta, bias, mean, var)[0]
                                  ["y"] * delta.astype(np.float64)))
    h = 1e-2
    fd = (loss((wt + h * v).astype(np.float32)) - loss((wt - h * v).astype(np.float32))) / (2 * h)
    got, desc = gpu_forward(torch, case, x, wt, gamma, beta, bias, mean, var)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    dw = torch.zeros(wt.shape, device="cuda")
    ws = cbb.workspace(cbb.conv_block_workspace_size(desc))
    cbb.conv_block_backward(desc, T(x), T(wt), T(got["y"]), T(got["xhat"]), T(got["var"]),
                            T(gamma), T(delta), torch.empty(2, 8, 8, 8, device="cuda"), dw,
                            torch.zeros(8, device="cuda"), torch.zeros(8, device="cuda"), None,
                            False, ws)
    torch.cuda.synchronize()
    an = float(np.sum(dw.cpu().double().numpy() * v))
    assert abs(fd - an) <= 1e-2 * abs(an) + 1e-3, (fd, an)
