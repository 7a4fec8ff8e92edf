"""Pins for the oracle's LeNet layers and the shortcut / route / upsample steps (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------- softmax loss
def test_softmax_loss_backward_matches_autograd_and_closed_form():
    logits = _rand(1, 64, 10) * 3
    labels = np.random.default_rng(2).integers(0, 10, 64).astype(np.int32)
    prob = O.softmax_forward(logits)
    np.testing.assert_allclose(prob.sum(axis=1), 1.0, atol=1e-15)
    tl = torch.tensor(logits, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(tl, torch.tensor(labels, dtype=torch.long))
    assert O.softmax_loss(prob, labels) == pytest.approx(loss.item(), rel=1e-13)
    loss.backward()
    d = O.softmax_loss_backward(prob, labels, 1.0)
    np.testing.assert_allclose(d, tl.grad.numpy(), rtol=0, atol=1e-15)
    # rows of (p - onehot)/N sum to zero
    np.testing.assert_allclose(d.sum(axis=1), 0.0, atol=1e-16)
    # loss_weight scales linearly
    np.testing.assert_allclose(O.softmax_loss_backward(prob, labels, 0.5), 0.5 * d, rtol=1e-15)


def test_softmax_loss_equals_generic_softmax_backward_composed_with_ce():
    """Caffe's generic softmax backward dx = (dy - sum(dy*y)) * y, fed the cross-entropy
    gradient dy = -onehot/(N*p), reproduces SoftmaxWithLoss's (p - onehot)/N."""
    n, c = 16, 10
    prob = O.softmax_forward(_rand(3, n, c))
    labels = np.random.default_rng(4).integers(0, c, n).astype(np.int32)
    dy = np.zeros((n, c))
    dy[np.arange(n), labels] = -1.0 / (n * prob[np.arange(n), labels])
    generic = (dy - np.sum(dy * prob, axis=1, keepdims=True)) * prob
    np.testing.assert_allclose(O.softmax_loss_backward(prob, labels), generic, rtol=0, atol=1e-16)


# ----------------------------------------------------------------------------- inner product
def test_fc_backward_matches_autograd():
    x, w, b = _rand(5, 64, 800), _rand(6, 500, 800) * 0.05, _rand(7, 500)
    tx, tw, tb = (torch.tensor(a, requires_grad=True) for a in (x, w, b))
    ty = torch.nn.functional.linear(tx, tw, tb)
    np.testing.assert_allclose(O.fc_forward(x, w, b), ty.detach().numpy(), atol=1e-12)
    d = _rand(8, 64, 500)
    ty.backward(torch.tensor(d))
    dw, db, dx = O.fc_backward(x, w, d)
    np.testing.assert_allclose(dw, tw.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(db, tb.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dx, tx.grad.numpy(), atol=1e-12)
    # textbook matmul forms: dW = d^T X, db = d^T 1, dX = d W
    np.testing.assert_allclose(dw, d.T @ x, atol=1e-11)
    np.testing.assert_allclose(dx, d @ w, atol=1e-12)
    # parameter gradients accumulate, dX overwrites unless asked to accumulate
    dw2, db2, dx2 = O.fc_backward(x, w, d, dw=dw, db=db, dx=np.ones_like(dx))
    np.testing.assert_allclose(dw2, 2 * dw, rtol=1e-15)
    np.testing.assert_allclose(db2, 2 * db, rtol=1e-15)
    np.testing.assert_allclose(dx2, dx, rtol=0, atol=0)
    _, _, dx3 = O.fc_backward(x, w, d, dx=np.ones_like(dx), dx_accumulate=True)
    np.testing.assert_allclose(dx3, dx + 1.0, rtol=1e-15, atol=1e-15)
    _, _, none = O.fc_backward(x, w, d, want_dx=False)
    assert none is None


# ----------------------------------------------------------------------------- max pool
def test_maxpool_backward_matches_autograd():
    x = _rand(9, 4, 3, 8, 8)
    y, idx = O.maxpool_forward(x, 2, 2)
    tx = torch.tensor(x, requires_grad=True)
    ty, tidx = torch.nn.functional.max_pool2d(tx, 2, 2, return_indices=True)
    np.testing.assert_array_equal(y, ty.detach().numpy())
    np.testing.assert_array_equal(idx, tidx.numpy())          # per-plane flat index h*W+w
    d = _rand(10, *y.shape)
    ty.backward(torch.tensor(d))
    dx = O.maxpool_backward(idx, d, (8, 8))
    np.testing.assert_array_equal(dx, tx.grad.numpy())
    # every pooled delta lands once: per-plane sums agree exactly for integer deltas
    di = np.random.default_rng(11).integers(-50, 50, y.shape).astype(float)
    dxi = O.maxpool_backward(idx, di, (8, 8))
    np.testing.assert_array_equal(dxi.sum(axis=(2, 3)), di.sum(axis=(2, 3)))
    assert np.count_nonzero(dxi) <= np.count_nonzero(di)


def test_maxpool_tie_takes_first_in_window():
    x = np.zeros((1, 1, 4, 4))
    _, idx = O.maxpool_forward(x, 2, 2)
    np.testing.assert_array_equal(idx[0, 0], [[0, 2], [8, 10]])


def test_maxpool_backward_overlapping_indices_add():
    """Two pooled outputs naming the same bottom pixel both add into it."""
    idx = np.array([[[[5, 5], [5, 0]]]], dtype=np.int32)
    d = np.array([[[[1.0, 2.0], [4.0, 8.0]]]])
    dx = O.maxpool_backward(idx, d, (4, 4))
    assert dx[0, 0, 1, 1] == 7.0 and dx[0, 0, 0, 0] == 8.0 and dx.sum() == 15.0


@pytest.mark.parametrize("shape", [(64, 10), (3, 5, 4, 6), (2, 7, 9)])
def test_softmax_backward_matches_autograd(shape):
    """Generic softmax backward over axis 1 against float64 autograd of torch.softmax."""
    logits = torch.tensor(_rand(51, *shape), requires_grad=True)
    y = torch.softmax(logits, dim=1)
    dy = _rand(52, *shape)
    y.backward(torch.tensor(dy))
    dx = O.softmax_backward(y.detach().numpy(), dy)
    np.testing.assert_allclose(dx, logits.grad.numpy(), rtol=0, atol=1e-15)


def test_softmax_backward_composed_with_ce_is_softmax_loss_gradient():
    """Fed dp = -onehot / (N p), the generic backward gives SoftmaxWithLoss's (p - onehot)/N."""
    n, c = 64, 10
    prob = O.softmax_forward(_rand(53, n, c))
    labels = np.random.default_rng(54).integers(0, c, size=n).astype(np.int32)
    dp = np.zeros((n, c))
    dp[np.arange(n), labels] = -1.0 / (n * prob[np.arange(n), labels])
    np.testing.assert_allclose(O.softmax_backward(prob, dp), O.softmax_loss_backward(prob, labels),
                               rtol=0, atol=1e-16)


# ----------------------------------------------------------------------------- shortcut / route / upsample
def test_shortcut_backward():
    d = _rand(12, 2, 3, 4, 4)
    m0, f0 = _rand(13, *d.shape), _rand(14, *d.shape)
    m, f = O.shortcut_backward(d, m0, f0, 1.0, 1.0)
    np.testing.assert_array_equal(m, m0 + d)
    np.testing.assert_array_equal(f, f0 + d)
    m, f = O.shortcut_backward(d, m0, f0, 0.5, 2.0)
    np.testing.assert_allclose(m, m0 + 0.5 * d, rtol=1e-15)
    np.testing.assert_allclose(f, f0 + 2.0 * d, rtol=1e-15)


def test_route_backward_is_adjoint_of_concat():
    a, b = _rand(15, 2, 5, 3, 3), _rand(16, 2, 2, 3, 3)
    d = _rand(17, 2, 7, 3, 3)
    da, db = O.route_backward(d, [np.zeros_like(a), np.zeros_like(b)])
    np.testing.assert_array_equal(da, d[:, :5])
    np.testing.assert_array_equal(db, d[:, 5:])
    ta, tb = torch.tensor(a, requires_grad=True), torch.tensor(b, requires_grad=True)
    torch.cat([ta, tb], 1).backward(torch.tensor(d))
    np.testing.assert_array_equal(da, ta.grad.numpy())
    np.testing.assert_array_equal(db, tb.grad.numpy())
    da2, _ = O.route_backward(d, [np.ones_like(a), np.zeros_like(b)])
    np.testing.assert_allclose(da2, d[:, :5] + 1.0, rtol=1e-15)


def test_upsample_backward_adjoint_and_autograd():
    x = _rand(18, 2, 3, 5, 4)
    y = O.upsample_forward(x, 2)
    tx = torch.tensor(x, requires_grad=True)
    ty = torch.nn.functional.interpolate(tx, scale_factor=2, mode="nearest")
    np.testing.assert_array_equal(y, ty.detach().numpy())
    d = _rand(19, *y.shape)
    ty.backward(torch.tensor(d))
    dx = O.upsample_backward(d, 2)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=0, atol=1e-14)
    assert float(np.sum(y * d)) == pytest.approx(float(np.sum(x * dx)), rel=1e-13)
    di = np.random.default_rng(20).integers(-9, 9, y.shape).astype(float)
    np.testing.assert_array_equal(O.upsample_backward(di, 2),
                                  di[:, :, ::2, ::2] + di[:, :, 1::2, ::2]
                                  + di[:, :, ::2, 1::2] + di[:, :, 1::2, 1::2])


# ----------------------------------------------------------------------------- page shapes
def test_lenet_shapes_fixture():
    """Shapes the LeNet page prints for layer 4 (conv2) and layer 9 (softmax loss)."""
    with open(os.path.join(GOLDEN, "lenet_shapes.json")) as f:
        g = json.load(f)
    n, c, h, w = g["conv2_bottom"]
    oc, k = g["conv2_top"][1], g["conv2_kernel"]
    assert g["conv2_top"] == [n, oc, O.conv_out_dim(h, k, 1, 0), O.conv_out_dim(w, k, 1, 0)]
    assert g["conv2_weight_matrix"] == [oc, c * k * k]
    oh = O.conv_out_dim(h, k, 1, 0)
    assert g["conv2_col_matrix"] == [oh * oh, c * k * k]
    x = np.zeros((n, c, h, w))
    z = O.conv_forward(x, np.zeros((oc, c, k, k)), 1, 0)
    assert list(z.shape) == g["conv2_top"]
    prob = O.softmax_forward(np.zeros(g["loss_bottom_diff"]))
    labels = np.zeros(g["loss_bottom_diff"][0], np.int32)
    d = O.softmax_loss_backward(prob, labels)
    assert list(d.shape) == g["loss_bottom_diff"]
    assert d.shape[1] == g["loss_dim"] and d.shape[0] == g["loss_nthreads"]


def _shortcut_forward_torch(prev, src, alpha, beta):
    """The page's forward shortcut between different shapes, written as strided slices:
    out = alpha * prev, then over the smaller shape out[.., j*sample, i*sample] +=
    beta * src[.., j*stride, i*stride] with stride = w_src / w_out, sample = w_out / w_src."""
    _, cd, hd, wd = prev.shape
    _, cs, hs, ws = src.shape
    stride, sample = max(1, ws // wd), max(1, wd // ws)
    mc, mh, mw = min(cd, cs), min(hd, hs), min(wd, ws)
    out = alpha * prev
    out = out.clone()
    out[:, :mc, 0:mh * sample:sample, 0:mw * sample:sample] += \
        beta * src[:, :mc, 0:mh * stride:stride, 0:mw * stride:stride]
    return out


@pytest.mark.parametrize("dshape,sshape", [((2, 4, 8, 8), (2, 6, 4, 4)), ((2, 6, 4, 4), (2, 3, 8, 8)),
                                           ((1, 3, 12, 6), (1, 3, 4, 2)), ((3, 5, 6, 6), (3, 5, 6, 6))])
def test_shortcut_backward_resize_is_adjoint_of_forward(dshape, sshape):
    """Backward between different shapes against float64 autograd of the forward shortcut."""
    r = np.random.default_rng(31)
    alpha, beta = 0.75, 1.5
    prev = torch.tensor(r.normal(size=dshape), requires_grad=True)
    src = torch.tensor(r.normal(size=sshape), requires_grad=True)
    delta = r.normal(size=dshape)
    _shortcut_forward_torch(prev, src, alpha, beta).backward(torch.tensor(delta))
    m0, f0 = r.normal(size=dshape), r.normal(size=sshape)
    dm, df = O.shortcut_backward_resize(delta, m0, f0, alpha, beta)
    np.testing.assert_allclose(dm - m0, prev.grad.numpy(), rtol=0, atol=1e-14)
    np.testing.assert_allclose(df - f0, src.grad.numpy(), rtol=0, atol=1e-14)
    if dshape == sshape:   # equal shapes: the plain shortcut
        pm, pf = O.shortcut_backward(delta, m0, f0, alpha, beta)
        np.testing.assert_array_equal(dm, pm)
        np.testing.assert_array_equal(df, pf)
