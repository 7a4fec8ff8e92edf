"""Whole-workload pins: the oracle's composed backward against float64 autograd of the
same network written with an independent library (CPU only, reduced sizes)."""
import dataclasses

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.model as M
from cnn_backward_pass_amd import synth


def _shrink(name, batch, hw):
    """Same layer structure, smaller batch / spatial size (parity of structure, cheap to run)."""
    wl = synth.WORKLOADS[name]
    convs = []
    for c in wl.convs:
        convs.append(dataclasses.replace(c, in_h=hw, in_w=hw))
        if c.stride == 2:
            hw = convs[-1].out_h
    return dataclasses.replace(wl, batch=batch, convs=tuple(convs))


def _rng_inputs(wl, seed):
    r = np.random.default_rng(seed)
    n = wl.batch
    c0 = wl.convs[0]
    inp = {"w": [r.normal(0, 0.2, (c.out_c, c.in_c, c.k, c.k)) for c in wl.convs]}
    if wl.name == "yolov3_head":
        hw = c0.in_h
        inp["route_a"] = r.normal(size=(n, c0.in_c - 128, hw, hw))
        inp["up_src"] = r.normal(size=(n, 128, hw // 2, hw // 2))
        inp["conv_b"] = [None, None, r.normal(size=wl.convs[-1].out_c)]
    else:
        inp["x"] = r.normal(size=(n, c0.in_c, c0.in_h, c0.in_w))
    last = wl.convs[-1]
    inp["delta"] = r.normal(size=(n, last.out_c, last.out_h, last.out_w))
    return inp


def _torch_net(wl, inp):
    """The network, forward, in torch float64; returns (out, leaves dict)."""
    T = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    leaves = {"w": [T(w) for w in inp["w"]]}
    bn = [c.bn for c in wl.convs]
    leaves["gamma"] = [T(np.ones(c.out_c)) if c.bn else None for c in wl.convs]
    leaves["beta"] = [T(np.zeros(c.out_c)) if c.bn else None for c in wl.convs]
    leaves["b"] = [None] * len(wl.convs)
    if wl.name == "yolov3_head":
        leaves["route_a"], leaves["up_src"] = T(inp["route_a"]), T(inp["up_src"])
        leaves["b"][-1] = T(inp["conv_b"][-1])
        x = torch.cat([leaves["route_a"],
                       F.interpolate(leaves["up_src"], scale_factor=2, mode="nearest")], 1)
    else:
        leaves["x"] = T(inp["x"])
        x = leaves["x"]
    h = x
    for li, c in enumerate(wl.convs):
        z = F.conv2d(h, leaves["w"][li], leaves["b"][li], stride=c.stride, padding=c.pad)
        if bn[li]:
            z = F.batch_norm(z, None, None, leaves["gamma"][li], leaves["beta"][li], training=True,
                             eps=1e-5)
        h = F.leaky_relu(z, 0.1) if c.act == "leaky" else z
    if wl.name == "darknet53_residual":
        h = h + leaves["x"]
    return h, leaves


@pytest.mark.parametrize("name,batch,hw", [("single_block", 2, 32), ("darknet53_residual", 2, 13),
                                           ("yolov3_stem", 2, 24), ("yolov3_head", 2, 10)])
def test_conv_workload_backward_matches_autograd(name, batch, hw):
    wl = _shrink(name, batch, hw)
    inp = _rng_inputs(wl, 100 + wl.wid)
    saved = M.workload_forward(wl, inp)
    out, leaves = _torch_net(wl, inp)
    np.testing.assert_allclose(saved["out"], out.detach().numpy(), rtol=0, atol=1e-10)
    out.backward(torch.tensor(inp["delta"]))
    g = M.workload_backward(wl, inp, saved, inp["delta"])
    tol = dict(rtol=0, atol=1e-9)
    for li, c in enumerate(wl.convs):
        np.testing.assert_allclose(g["dw"][li], leaves["w"][li].grad.numpy(), **tol)
        if c.bn:
            np.testing.assert_allclose(g["dgamma"][li], leaves["gamma"][li].grad.numpy(), **tol)
            np.testing.assert_allclose(g["db"][li], leaves["beta"][li].grad.numpy(), **tol)
        elif leaves["b"][li] is not None:
            np.testing.assert_allclose(g["db"][li], leaves["b"][li].grad.numpy(), **tol)
    if name == "yolov3_head":
        np.testing.assert_allclose(g["d_route_a"], leaves["route_a"].grad.numpy(), **tol)
        np.testing.assert_allclose(g["d_up_src"], leaves["up_src"].grad.numpy(), **tol)
    else:
        np.testing.assert_allclose(g["dx"], leaves["x"].grad.numpy(), **tol)


def test_lenet_backward_matches_autograd():
    wl = synth.WORKLOADS["lenet"]
    inp = synth.inputs("lenet", scale_batch=8)
    inp = {k: v for k, v in inp.items()}
    saved = M.workload_forward(wl, inp)
    T = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    cw = [T(w) for w in inp["w"]]
    cb = [T(b) for b in inp["conv_b"]]
    fw = [T(w) for w in inp["fc_w"]]
    fb = [T(b) for b in inp["fc_b"]]
    x = torch.tensor(np.asarray(inp["x"], np.float64))
    h = F.max_pool2d(F.conv2d(x, cw[0], cb[0]), 2, 2)
    h = F.max_pool2d(F.conv2d(h, cw[1], cb[1]), 2, 2)
    h = torch.relu(F.linear(h.reshape(h.shape[0], -1), fw[0], fb[0]))
    logits = F.linear(h, fw[1], fb[1])
    np.testing.assert_allclose(saved["logits"], logits.detach().numpy(), atol=1e-11)
    loss = F.cross_entropy(logits, torch.tensor(inp["labels"], dtype=torch.long))
    loss.backward()
    g = M.workload_backward(wl, inp, saved)
    tol = dict(rtol=0, atol=1e-12)
    for i in range(2):
        np.testing.assert_allclose(g["dw"][i], cw[i].grad.numpy(), **tol)
        np.testing.assert_allclose(g["db"][i], cb[i].grad.numpy(), **tol)
        np.testing.assert_allclose(g["fc_dw"][i], fw[i].grad.numpy(), **tol)
        np.testing.assert_allclose(g["fc_db"][i], fb[i].grad.numpy(), **tol)


def test_synth_is_deterministic_and_seeded_per_tensor():
    a = synth.inputs("single_block")
    b = synth.inputs("single_block")
    for k in ("x", "delta"):
        np.testing.assert_array_equal(a[k], b[k])
        assert a[k].dtype == np.float32
    # tensor t of workload k comes from PCG64(1000 k + t)
    ref = np.random.Generator(np.random.PCG64(1000 * 1 + 2)).normal(0, 1, (2, 16, 32, 32))
    np.testing.assert_array_equal(a["delta"], ref.astype(np.float32))
    s = synth.saved_standins("lenet", scale_batch=4)
    for li, hw in enumerate((24, 8)):
        idx = s["pool_idx"][li]
        assert idx.min() >= 0 and idx.max() < hw * hw
        ph = hw // 2
        r, q = idx // hw, idx % hw
        assert np.all(r // 2 == np.arange(ph)[None, None, :, None])
        assert np.all(q // 2 == np.arange(ph)[None, None, None, :])
    np.testing.assert_allclose(s["prob"].sum(axis=1), 1.0, atol=1e-6)
