"""Seeded synthetic inputs for the five conv-block backward workloads.

This module holds the workloads' geometry (layer shapes, strides, paddings)
and draws every input tensor from its own seeded stream.  It contains none of
the backward arithmetic: the HIP path and the CPU oracle both take their
inputs from here and from nowhere else.

Seeding: tensor number ``t`` of workload ``k`` (k = 1..5, in the order below)
is drawn from ``numpy.random.Generator(PCG64(1000*k + t))`` in float64 and
rounded to float32.

Workloads (stand-ins for the pages' networks; no dataset is used):
  1 single_block        -- one 3x3 conv block (conv + BN + leaky), batch 2 at 32x32
  2 lenet               -- Caffe's LeNet (MNIST-shaped 1x28x28 input, 10 classes), batch 64
  3 darknet53_residual  -- 1x1 + 3x3 conv blocks and a shortcut, batch 8 at 52x52
  4 yolov3_stem         -- 3x3 conv 3->32 at 416x416, 3x3 stride-2 conv 32->64, batch 16
  5 yolov3_head         -- route of a 26x26 map and a 2x-upsampled 13x13 map, 1x1/3x3/1x1 convs
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

LEAKY_SLOPE = 0.1
BN_EPS = 1e-5


@dataclass(frozen=True)
class ConvLayer:
    """Geometry of one convolutional layer (Darknet layer fields n/size/stride/pad)."""
    name: str
    in_c: int
    out_c: int
    k: int
    stride: int
    pad: int
    bn: bool           # batch_normalize: BN follows the conv, the conv bias merges into beta
    act: str           # "leaky" | "linear" | "logistic" | "relu"
    in_h: int
    in_w: int

    @property
    def out_h(self) -> int:
        return (self.in_h + 2 * self.pad - self.k) // self.stride + 1

    @property
    def out_w(self) -> int:
        return (self.in_w + 2 * self.pad - self.k) // self.stride + 1


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    batch: int
    convs: tuple = field(default_factory=tuple)
    description: str = ""


def _conv(name, in_c, out_c, k, s, p, bn, act, hw):
    return ConvLayer(name, in_c, out_c, k, s, p, bn, act, hw, hw)


WORKLOADS = {
    "single_block": Workload(
        1, "single_block", 2,
        (_conv("conv", 3, 16, 3, 1, 1, True, "leaky", 32),),
        "x 2x3x32x32 ~U(0,1); 3x3 conv pad1 3->16, BN, leaky 0.1; delta 2x16x32x32 ~N(0,1)"),
    "lenet": Workload(
        2, "lenet", 64,
        (_conv("conv1", 1, 20, 5, 1, 0, False, "linear", 28),
         _conv("conv2", 20, 50, 5, 1, 0, False, "linear", 12)),
        "batch 64, 1x28x28 ~U(0,1); conv1 5x5 1->20, pool 2, conv2 5x5 20->50, pool 2, "
        "ip1 800->500, ReLU, ip2 500->10, softmax-with-loss; Xavier-uniform weights"),
    "darknet53_residual": Workload(
        3, "darknet53_residual", 8,
        (_conv("conv1", 256, 128, 1, 1, 0, True, "leaky", 52),
         _conv("conv2", 128, 256, 3, 1, 1, True, "leaky", 52)),
        "x 8x256x52x52 ~N(0,1); 1x1 256->128 BN leaky, 3x3 128->256 BN leaky, shortcut; "
        "delta ~N(0,1); weights ~N(0,0.05)"),
    "yolov3_stem": Workload(
        4, "yolov3_stem", 16,
        (_conv("conv1", 3, 32, 3, 1, 1, True, "leaky", 416),
         _conv("conv2", 32, 64, 3, 2, 1, True, "leaky", 416)),
        "x 16x3x416x416 ~U(0,1); 3x3 3->32 BN leaky, 3x3 s2 32->64 BN leaky; "
        "delta 16x64x208x208 ~N(0,1); weights ~N(0,0.05)"),
    "yolov3_head": Workload(
        5, "yolov3_head", 8,
        (_conv("conv1", 384, 256, 1, 1, 0, True, "leaky", 26),
         _conv("conv2", 256, 512, 3, 1, 1, True, "leaky", 26),
         _conv("conv3", 512, 255, 1, 1, 0, False, "linear", 26)),
        "route(8x256x26x26, up2(8x128x13x13)) -> 384ch; 1x1 384->256 BN leaky, 3x3 256->512 "
        "BN leaky, 1x1 512->255 linear; delta 8x255x26x26 ~N(0,0.1); weights ~N(0,0.05)"),
}

LENET_FC = ((800, 500), (500, 10))   # (in, out) of ip1, ip2
LENET_CLASSES = 10


def rng(wid: int, t: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * wid + t))


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))


def normal(wid, t, shape, std=1.0):
    return _f32(rng(wid, t).normal(0.0, std, size=shape))


def uniform(wid, t, shape, lo=0.0, hi=1.0):
    return _f32(rng(wid, t).uniform(lo, hi, size=shape))


def xavier_uniform(wid, t, shape, fan_in, fan_out):
    """Glorot-uniform: U(+-sqrt(6/(fan_in+fan_out)))."""
    a = np.sqrt(6.0 / (fan_in + fan_out))
    return _f32(rng(wid, t).uniform(-a, a, size=shape))


def inputs(name: str, scale_batch: int | None = None) -> dict:
    """Primary inputs (image / feature maps, weights, upstream delta, labels) of a workload.

    ``scale_batch`` replaces the batch size (small parity cases); every other
    shape is the workload's own.
    """
    wl = WORKLOADS[name]
    k = wl.wid
    n = wl.batch if scale_batch is None else scale_batch
    out: dict = {}
    if name == "single_block":
        c = wl.convs[0]
        out["x"] = uniform(k, 0, (n, 3, 32, 32))
        out["w"] = [normal(k, 1, (c.out_c, c.in_c, c.k, c.k), 0.1)]
        out["delta"] = normal(k, 2, (n, c.out_c, c.out_h, c.out_w), 1.0)
    elif name == "lenet":
        c1, c2 = wl.convs
        out["x"] = uniform(k, 0, (n, 1, 28, 28))
        out["w"] = [xavier_uniform(k, 1, (20, 1, 5, 5), 1 * 25, 20 * 25),
                    xavier_uniform(k, 2, (50, 20, 5, 5), 20 * 25, 50 * 25)]
        out["fc_w"] = [xavier_uniform(k, 3, (500, 800), 800, 500),
                       xavier_uniform(k, 4, (10, 500), 500, 10)]
        out["labels"] = np.ascontiguousarray(
            rng(k, 5).integers(0, LENET_CLASSES, size=(n,)).astype(np.int32))
        out["conv_b"] = [np.zeros(20, np.float32), np.zeros(50, np.float32)]
        out["fc_b"] = [np.zeros(500, np.float32), np.zeros(10, np.float32)]
    elif name == "darknet53_residual":
        c1, c2 = wl.convs
        out["x"] = normal(k, 0, (n, 256, 52, 52), 1.0)
        out["w"] = [normal(k, 1, (c1.out_c, c1.in_c, 1, 1), 0.05),
                    normal(k, 2, (c2.out_c, c2.in_c, 3, 3), 0.05)]
        out["delta"] = normal(k, 3, (n, 256, 52, 52), 1.0)
    elif name == "yolov3_stem":
        c1, c2 = wl.convs
        out["x"] = uniform(k, 0, (n, 3, 416, 416))
        out["w"] = [normal(k, 1, (32, 3, 3, 3), 0.05), normal(k, 2, (64, 32, 3, 3), 0.05)]
        out["delta"] = normal(k, 3, (n, 64, 208, 208), 1.0)
    elif name == "yolov3_head":
        out["route_a"] = normal(k, 0, (n, 256, 26, 26), 1.0)
        out["up_src"] = normal(k, 1, (n, 128, 13, 13), 1.0)
        out["w"] = [normal(k, 2, (256, 384, 1, 1), 0.05), normal(k, 3, (512, 256, 3, 3), 0.05),
                    normal(k, 4, (255, 512, 1, 1), 0.05)]
        out["conv_b"] = [None, None, np.zeros(255, np.float32)]
        out["delta"] = normal(k, 5, (n, 255, 26, 26), 0.1)
    else:
        raise KeyError(name)
    return out


def bn_params(c: int):
    """BN scale and shift as the workloads fix them: gamma = 1, beta = 0."""
    return np.ones(c, np.float32), np.zeros(c, np.float32)


def saved_standins(name: str, scale_batch: int | None = None) -> dict:
    """Stand-ins for the forward-pass tensors a backward pass reads.

    Drawn directly from distributions of the right shape and range (no forward
    arithmetic): per conv layer the activation output y ~ N(0,1) (signs mixed
    half and half, as after leaky ReLU of a zero-mean input), the normalised
    pre-activation xhat ~ N(0,1), the batch variance var ~ U(0.5, 2); for LeNet
    the pooled-max indices are drawn uniformly inside each 2x2 window, the ReLU
    output is 0 with probability 1/2 and |N(0,1)| otherwise, and the class
    probabilities are Dirichlet(1,...,1) rows.  Used at full sizes, where a
    double-precision forward would cost more than the check it feeds.
    """
    wl = WORKLOADS[name]
    k = wl.wid
    n = wl.batch if scale_batch is None else scale_batch
    out: dict = {"layers": []}
    for li, c in enumerate(wl.convs):
        shp = (n, c.out_c, c.out_h, c.out_w)
        t = 100 + 10 * li
        d = {"y": normal(k, t, shp, 1.0)}
        if c.bn:
            d["xhat"] = normal(k, t + 1, shp, 1.0)
            d["var"] = uniform(k, t + 2, (c.out_c,), 0.5, 2.0)
            d["gamma"], d["beta"] = bn_params(c.out_c)
        out["layers"].append(d)
    if name == "lenet":
        for li, (c, hw) in enumerate(((20, 24), (50, 8))):
            ph = hw // 2
            r = rng(k, 200 + li)
            a = r.integers(0, 2, size=(n, c, ph, ph))
            b = r.integers(0, 2, size=(n, c, ph, ph))
            py = np.arange(ph).reshape(1, 1, ph, 1)
            px = np.arange(ph).reshape(1, 1, 1, ph)
            out.setdefault("pool_idx", []).append(
                np.ascontiguousarray(((2 * py + a) * hw + 2 * px + b).astype(np.int32)))
        r = rng(k, 210)
        zero = r.random((n, 500)) < 0.5
        out["relu_y"] = _f32(np.where(zero, 0.0, np.abs(r.normal(size=(n, 500)))))
        out["pool2_out"] = normal(k, 211, (n, 800), 1.0)      # ip1 input (flattened pool2 output)
        out["relu_in_ip2"] = out["relu_y"]                    # ip2 input is the ReLU output
        out["prob"] = _f32(rng(k, 212).dirichlet(np.ones(LENET_CLASSES), size=n))
        out["pool1_out"] = normal(k, 213, (n, 20, 12, 12), 1.0)  # conv2 input
    if name == "yolov3_head":
        out["route_out"] = normal(k, 220, (n, 384, 26, 26), 1.0)   # conv1 input (route output)
    # Each conv layer's input is the previous layer's output (or the workload's
    # own input for the first layer): plain references, no arithmetic.
    firsts = {"single_block": lambda: inputs(name, scale_batch)["x"],
              "darknet53_residual": lambda: inputs(name, scale_batch)["x"],
              "yolov3_stem": lambda: inputs(name, scale_batch)["x"],
              "yolov3_head": lambda: out["route_out"],
              "lenet": lambda: inputs(name, scale_batch)["x"]}
    for li, d in enumerate(out["layers"]):
        if li == 0:
            d["x_in"] = firsts[name]()
        elif name == "lenet":
            d["x_in"] = out["pool1_out"]
        else:
            d["x_in"] = out["layers"][li - 1]["y"]
    return out
