"""Per-block and per-workload composition of the oracle's layer steps.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

A conv block is Darknet's convolutional layer: conv, then (optionally) batch
normalisation whose shift absorbs the conv bias, then an activation.  Its
backward runs the steps of backward_convolutional_layer in the order of
"YOLOv3 backpropagation: full-flow source analysis", section 3.1: activation
gradient (gradient_array), BN backward (section 4) or the bias sum, then the
weight gradient, then -- when the previous layer wants one -- the input
gradient.  The workloads chain such blocks with the shortcut (section 5) and
route (section 6) layers of the same page and with Caffe's LeNet layers of
"Caffe source study ch.4 (5): the LeNet backward pass" (layers 9..4).

Geometry comes in as plain data (objects with in_c/out_c/k/stride/pad/bn/act
fields and a ``batch``); this module does not import the input generators.
"""
from __future__ import annotations

import numpy as np

from . import (ACT_NAMES, act_backward, act_forward, bn_backward, bn_backward_fixed, bn_forward,
               bn_forward_fixed, conv_backward_bias, conv_backward_data_gd,
               conv_backward_weights_gd, conv_forward_gd,
               conv_backward_data, conv_backward_weights, conv_forward, fc_backward, fc_forward,
               maxpool_backward, maxpool_forward, route_backward, shortcut_backward,
               softmax_forward, softmax_loss_backward, upsample_backward, upsample_forward)

SLOPE = 0.1
EPS = 1e-5


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def conv_block_forward(layer, x, w, bias=None, gamma=None, beta=None, eps=EPS, slope=SLOPE,
                       mean=None, var=None):
    """Forward of one conv block; returns the tensors its backward reads (and more).
    layer.bn: 0 none, 1 (or True) batch statistics, 2 the fixed statistics mean, var."""
    act = ACT_NAMES[layer.act]
    groups, dil = getattr(layer, "groups", 1), getattr(layer, "dilation", 1)
    if groups != 1 or dil != 1:
        z = conv_forward_gd(x, w, layer.stride, layer.pad, dil, groups,
                            bias=None if layer.bn else bias)
    else:
        z = conv_forward(x, w, layer.stride, layer.pad, bias=None if layer.bn else bias)
    out = {"x_in": _f64(x), "w": _f64(w), "z": z}
    if layer.bn == 2:
        xhat, u = bn_forward_fixed(z, mean, var, gamma, beta, eps)
        out.update(mean=_f64(mean), var=_f64(var), xhat=xhat, gamma=_f64(gamma),
                   beta=_f64(beta))
    elif layer.bn:
        mean, var, xhat, u = bn_forward(z, gamma, beta, eps)
        out.update(mean=mean, var=var, xhat=xhat, gamma=_f64(gamma), beta=_f64(beta))
    else:
        u = z
    out["u"] = u
    out["y"] = act_forward(act, slope, u)
    return out


def conv_block_backward(layer, saved, delta, want_dx=True, dx_init=None, eps=EPS, slope=SLOPE,
                        w=None):
    """Backward of one conv block from delta = dL/dy.

    Returns g, dz, dw, db (= dbeta when BN follows), dgamma (BN only) and dx
    (added onto ``dx_init`` when given: the input gradient is the total over
    every consumer of the input).
    """
    act = ACT_NAMES[layer.act]
    g = act_backward(act, slope, saved["y"], delta)
    res = {"g": g}
    if layer.bn:
        bwd = bn_backward_fixed if layer.bn == 2 else bn_backward
        dz, dgamma, dbeta = bwd(g, saved["xhat"], saved["var"], saved["gamma"], eps)
        res.update(dz=dz, db=dbeta, dgamma=dgamma)
    else:
        dz = g
        res.update(dz=dz, db=conv_backward_bias(dz))
    x = saved["x_in"]
    groups, dil = getattr(layer, "groups", 1), getattr(layer, "dilation", 1)
    wt = saved["w"] if w is None else w
    if groups != 1 or dil != 1:
        res["dw"] = conv_backward_weights_gd(x, dz, layer.k, layer.stride, layer.pad, dil, groups)
        if want_dx:
            res["dx"] = conv_backward_data_gd(wt, dz, x.shape[2:], layer.stride, layer.pad, dil,
                                              groups, dx=dx_init)
        return res
    res["dw"] = conv_backward_weights(x, dz, layer.k, layer.stride, layer.pad)
    if want_dx:
        res["dx"] = conv_backward_data(wt, dz, x.shape[2:], layer.stride, layer.pad, dx=dx_init)
    return res


# ----------------------------------------------------------------------------- workloads
def workload_forward(wl, inp) -> dict:
    """Forward pass of a workload in double; returns the saved tensors its backward reads.

    ``inp`` holds the primary inputs (float32 arrays from the seeded generators).
    """
    saved: dict = {"layers": []}
    name = wl.name
    convs = wl.convs
    if name == "lenet":
        c1, c2 = convs
        s1 = conv_block_forward(c1, inp["x"], inp["w"][0], bias=inp["conv_b"][0])
        p1, idx1 = maxpool_forward(s1["y"], 2, 2)
        s2 = conv_block_forward(c2, p1, inp["w"][1], bias=inp["conv_b"][1])
        p2, idx2 = maxpool_forward(s2["y"], 2, 2)
        flat = p2.reshape(p2.shape[0], -1)
        ip1 = fc_forward(flat, inp["fc_w"][0], inp["fc_b"][0])
        relu = act_forward(ACT_NAMES["relu"], 0.0, ip1)
        logits = fc_forward(relu, inp["fc_w"][1], inp["fc_b"][1])
        prob = softmax_forward(logits)
        saved["layers"] = [s1, s2]
        saved.update(pool_idx=[idx1, idx2], pool1_out=p1, pool2_out=flat, relu_y=relu,
                     logits=logits, prob=prob)
        return saved
    if name == "yolov3_head":
        up = upsample_forward(inp["up_src"], 2)
        x = np.concatenate([_f64(inp["route_a"]), up], axis=1)
        saved["route_out"] = x
    else:
        x = _f64(inp["x"])
    for li, layer in enumerate(convs):
        gamma = beta = None
        if layer.bn:
            gamma, beta = np.ones(layer.out_c), np.zeros(layer.out_c)
        bias = None
        if "conv_b" in inp and inp["conv_b"][li] is not None:
            bias = inp["conv_b"][li]
        s = conv_block_forward(layer, x, inp["w"][li], bias=bias, gamma=gamma, beta=beta)
        saved["layers"].append(s)
        x = s["y"]
    if name == "darknet53_residual":
        saved["out"] = x + _f64(inp["x"])       # shortcut: y2 + x (alpha = beta = 1, linear)
    else:
        saved["out"] = x
    return saved


def round_saved_to_f32(saved: dict) -> dict:
    """The fp32 copy of the saved tensors that both sides of a parity test read."""
    def r(v):
        if isinstance(v, np.ndarray) and v.dtype == np.float64:
            return np.ascontiguousarray(v.astype(np.float32))
        if isinstance(v, list):
            return [r(e) for e in v]
        if isinstance(v, dict):
            return {k: r(e) for k, e in v.items()}
        return v
    return r(saved)


def workload_backward(wl, inp, saved, delta=None) -> dict:
    """Backward pass of a workload from its upstream delta (LeNet: from the loss).

    ``saved`` may be the float64 forward output (self-check mode) or its fp32
    rounding / the fp32 stand-ins (parity mode); either way every value is read
    as double.  Returns every parameter gradient, the input gradients and the
    intermediate deltas.
    """
    name = wl.name
    convs = wl.convs
    L = saved["layers"]
    out: dict = {"dw": [None] * len(convs), "db": [None] * len(convs),
                 "dgamma": [None] * len(convs), "dz": [None] * len(convs),
                 "d_in": [None] * len(convs)}

    def put(li, r):
        out["dw"][li], out["db"][li], out["dz"][li] = r["dw"], r["db"], r["dz"]
        out["dgamma"][li] = r.get("dgamma")
        out["d_in"][li] = r.get("dx")

    if name == "lenet":
        c1, c2 = convs
        dlogits = softmax_loss_backward(saved["prob"], inp["labels"], 1.0)
        dw2, db2, d_relu = fc_backward(saved["relu_y"], inp["fc_w"][1], dlogits)
        g_relu = act_backward(ACT_NAMES["relu"], 0.0, saved["relu_y"], d_relu)
        dw1, db1, d_pool2 = fc_backward(saved["pool2_out"], inp["fc_w"][0], g_relu)
        n = d_pool2.shape[0]
        d_pool2 = d_pool2.reshape(n, c2.out_c, c2.out_h // 2, c2.out_w // 2)
        d_c2 = maxpool_backward(saved["pool_idx"][1], d_pool2, (c2.out_h, c2.out_w))
        r2 = conv_block_backward(c2, L[1], d_c2, want_dx=True, w=inp["w"][1])
        put(1, r2)
        d_c1 = maxpool_backward(saved["pool_idx"][0], r2["dx"], (c1.out_h, c1.out_w))
        r1 = conv_block_backward(c1, L[0], d_c1, want_dx=False, w=inp["w"][0])
        put(0, r1)
        out.update(dlogits=dlogits, fc_dw=[dw1, dw2], fc_db=[db1, db2], d_relu=d_relu,
                   g_relu=g_relu, d_pool2=d_pool2, d_c2=d_c2, d_c1=d_c1)
        return out

    delta = _f64(delta)
    if name == "darknet53_residual":
        # shortcut backward: the delta reaches the last conv's output (alpha) and the
        # shortcut source, i.e. the block input (beta); both buffers start at zero.
        d_y2, d_x = shortcut_backward(delta, np.zeros_like(delta), np.zeros_like(delta), 1.0, 1.0)
        r2 = conv_block_backward(convs[1], L[1], d_y2, want_dx=True, w=inp["w"][1])
        put(1, r2)
        r1 = conv_block_backward(convs[0], L[0], r2["dx"], want_dx=True, dx_init=d_x,
                                 w=inp["w"][0])
        put(0, r1)
        out["dx"] = r1["dx"]
        return out

    d = delta
    for li in range(len(convs) - 1, -1, -1):
        r = conv_block_backward(convs[li], L[li], d, want_dx=True, w=inp["w"][li])
        put(li, r)
        d = r["dx"]
    if name == "yolov3_head":
        up_c = np.asarray(inp["up_src"]).shape[1]
        a_c = wl.convs[0].in_c - up_c
        n, _, hh, ww = d.shape
        d_a, d_up = route_backward(d, [np.zeros((n, a_c, hh, ww)), np.zeros((n, up_c, hh, ww))])
        d_src = upsample_backward(d_up, 2)
        out.update(d_route=d, d_route_a=d_a, d_up=d_up, d_up_src=d_src)
    else:
        out["dx"] = d
    return out
