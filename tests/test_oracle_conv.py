"""Pins for the oracle's convolution steps (CPU only).

Each check comes from outside the oracle's own loops: an independent float64
autograd library, central finite differences of the oracle's forward, the
adjoint (dot-product) identity, integer coverage counts with a closed form,
one-hot probes, and the pages' own im2col -> gemm -> col2im route written with
numpy matmul.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle as O

SHAPES = [  # (n, c, h, w, oc, k, s, p)
    (2, 1, 5, 5, 2, 1, 1, 0),
    (2, 3, 7, 5, 4, 3, 1, 1),
    (2, 3, 7, 7, 2, 3, 2, 1),
    (1, 2, 9, 8, 3, 5, 1, 2),
    (2, 3, 6, 7, 4, 5, 2, 0),
    (2, 2, 8, 8, 3, 3, 2, 0),
    (1, 4, 5, 6, 2, 1, 2, 0),
    (2, 3, 5, 5, 2, 5, 1, 0),
]


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("shape", SHAPES)
def test_conv_backward_matches_float64_autograd(shape):
    n, c, h, w, oc, k, s, p = shape
    x, wt, b = _rand(1, n, c, h, w), _rand(2, oc, c, k, k), _rand(3, oc)
    z = O.conv_forward(x, wt, s, p, bias=b)
    dz = _rand(4, *z.shape)
    tx = torch.tensor(x, requires_grad=True)
    tw = torch.tensor(wt, requires_grad=True)
    tb = torch.tensor(b, requires_grad=True)
    tz = torch.nn.functional.conv2d(tx, tw, tb, stride=s, padding=p)
    np.testing.assert_allclose(z, tz.detach().numpy(), rtol=0, atol=1e-12)
    tz.backward(torch.tensor(dz))
    dw = O.conv_backward_weights(x, dz, k, s, p)
    dx = O.conv_backward_data(wt, dz, (h, w), s, p)
    db = O.conv_backward_bias(dz)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(db, tb.grad.numpy(), rtol=0, atol=1e-11)
    # single-element forms agree with the full ones
    for (o, i, kh, kw) in [(0, 0, 0, 0), (oc - 1, c - 1, k - 1, k - 1), (oc // 2, c // 2, k // 2, 0)]:
        assert O.conv_dw_at(x, dz, k, s, p, o, i, kh, kw) == pytest.approx(dw[o, i, kh, kw], abs=1e-12)
    for (bb, i, r, q) in [(0, 0, 0, 0), (n - 1, c - 1, h - 1, w - 1), (0, c // 2, h // 2, w // 3)]:
        assert O.conv_dx_at(wt, dz, (h, w), s, p, bb, i, r, q) == pytest.approx(dx[bb, i, r, q], abs=1e-12)


def test_accumulate_semantics():
    """dW and db add onto what the buffers hold (the beta=1 gemm of the pages); dx adds too."""
    n, c, h, w, oc, k, s, p = SHAPES[1]
    x, wt = _rand(1, n, c, h, w), _rand(2, oc, c, k, k)
    dz = _rand(4, n, oc, O.conv_out_dim(h, k, s, p), O.conv_out_dim(w, k, s, p))
    dw0, dx0, db0 = _rand(5, oc, c, k, k), _rand(6, n, c, h, w), _rand(7, oc)
    np.testing.assert_allclose(O.conv_backward_weights(x, dz, k, s, p, dw=dw0),
                               dw0 + O.conv_backward_weights(x, dz, k, s, p), atol=1e-12)
    np.testing.assert_allclose(O.conv_backward_data(wt, dz, (h, w), s, p, dx=dx0),
                               dx0 + O.conv_backward_data(wt, dz, (h, w), s, p), atol=1e-12)
    np.testing.assert_allclose(O.conv_backward_bias(dz, db=db0), db0 + O.conv_backward_bias(dz),
                               atol=1e-12)


def test_finite_differences_tiny():
    """Central differences of the oracle's own forward, L = <conv(x; W), dz>."""
    n, c, h, w, oc, k, s, p = 2, 2, 5, 5, 2, 3, 2, 1
    x, wt = _rand(11, n, c, h, w), _rand(12, oc, c, k, k)
    dz = _rand(13, n, oc, O.conv_out_dim(h, k, s, p), O.conv_out_dim(w, k, s, p))
    loss = lambda xx, ww: float(np.sum(O.conv_forward(xx, ww, s, p) * dz))
    dw = O.conv_backward_weights(x, dz, k, s, p)
    dx = O.conv_backward_data(wt, dz, (h, w), s, p)
    eps = 1e-6
    for idx in itertools.product(*[range(d) for d in wt.shape]):
        wp, wm = wt.copy(), wt.copy()
        wp[idx] += eps
        wm[idx] -= eps
        assert (loss(x, wp) - loss(x, wm)) / (2 * eps) == pytest.approx(dw[idx], rel=1e-6, abs=1e-8)
    for idx in itertools.product(*[range(d) for d in x.shape]):
        xp, xm = x.copy(), x.copy()
        xp[idx] += eps
        xm[idx] -= eps
        assert (loss(xp, wt) - loss(xm, wt)) / (2 * eps) == pytest.approx(dx[idx], rel=1e-6, abs=1e-8)


@pytest.mark.parametrize("shape", [(2, 3, 52, 52, 16, 3, 1, 1), (1, 3, 97, 83, 8, 3, 2, 1),
                                   (2, 20, 12, 12, 50, 5, 1, 0), (2, 16, 26, 26, 8, 1, 1, 0)])
def test_adjoint_identity(shape):
    """<conv_W(x), d> = <x, dX(d)> and <conv_x(W), d> = <W, dW(d)> (exact up to rounding)."""
    n, c, h, w, oc, k, s, p = shape
    x, wt = _rand(21, n, c, h, w), _rand(22, oc, c, k, k)
    z = O.conv_forward(x, wt, s, p)
    d = _rand(23, *z.shape)
    lhs = float(np.sum(z * d))
    rhs_x = float(np.sum(x * O.conv_backward_data(wt, d, (h, w), s, p)))
    rhs_w = float(np.sum(wt * O.conv_backward_weights(x, d, k, s, p)))
    scale = float(np.sum(np.abs(z * d)))
    assert abs(lhs - rhs_x) <= 1e-12 * scale
    assert abs(lhs - rhs_w) <= 1e-12 * scale


def _cov(size, osize, k, s, p, pos):
    """#{output rows o: input row pos lies in o's window} = #{o: 0 <= pos+p-s*o <= k-1}."""
    return sum(1 for o in range(osize) if 0 <= pos + p - s * o <= k - 1)


def _valid(size, osize, k, s, p, tap):
    """#{output rows o whose tap `tap` lands inside the image} = #{o: 0 <= s*o+tap-p <= size-1}."""
    return sum(1 for o in range(osize) if 0 <= s * o + tap - p <= size - 1)


@pytest.mark.parametrize("shape", SHAPES + [(2, 3, 32, 32, 16, 3, 1, 1), (1, 2, 41, 41, 4, 3, 2, 1)])
def test_coverage_closed_form(shape):
    """W = 1, delta = 1: dx counts the windows covering each pixel; x = 1: dW counts valid taps."""
    n, c, h, w, oc, k, s, p = shape
    oh, ow = O.conv_out_dim(h, k, s, p), O.conv_out_dim(w, k, s, p)
    dz = np.ones((n, oc, oh, ow))
    dx = O.conv_backward_data(np.ones((oc, c, k, k)), dz, (h, w), s, p)
    ch = np.array([_cov(h, oh, k, s, p, r) for r in range(h)], float)
    cw = np.array([_cov(w, ow, k, s, p, q) for q in range(w)], float)
    np.testing.assert_array_equal(dx, np.broadcast_to(oc * ch[:, None] * cw[None, :], dx.shape))
    dw = O.conv_backward_weights(np.ones((n, c, h, w)), dz, k, s, p)
    vh = np.array([_valid(h, oh, k, s, p, t) for t in range(k)], float)
    vw = np.array([_valid(w, ow, k, s, p, t) for t in range(k)], float)
    np.testing.assert_array_equal(dw, np.broadcast_to(n * vh[:, None] * vw[None, :], dw.shape))
    np.testing.assert_array_equal(O.conv_backward_bias(dz), np.full(oc, n * oh * ow, float))


@pytest.mark.parametrize("shape", [(2, 3, 7, 7, 2, 3, 2, 1), (1, 2, 6, 9, 3, 3, 1, 1),
                                   (1, 1, 8, 8, 2, 5, 1, 2)])
def test_one_hot_probes(shape):
    """delta = e_(n,o,ho,wo): dX is W[o] pasted at the window (clipped), dW is the x patch."""
    n, c, h, w, oc, k, s, p = shape
    oh, ow = O.conv_out_dim(h, k, s, p), O.conv_out_dim(w, k, s, p)
    x, wt = _rand(31, n, c, h, w), _rand(32, oc, c, k, k)
    probes = {(0, 0, 0, 0), (n - 1, oc - 1, oh - 1, ow - 1), (0, oc - 1, 0, ow - 1),
              (n - 1, 0, oh - 1, 0), (0, 0, oh // 2, ow // 2)}
    if oh > 1 and ow > 1:
        probes |= {(0, 0, 1, 0), (0, 0, 0, 1), (0, 0, 1, 1)}
    for (b, o, y0, x0) in sorted(probes):
        dz = np.zeros((n, oc, oh, ow))
        dz[b, o, y0, x0] = 1.0
        exp_dx = np.zeros((n, c, h, w))
        exp_dw = np.zeros((oc, c, k, k))
        for kh in range(k):
            for kw in range(k):
                r, q = y0 * s + kh - p, x0 * s + kw - p
                if 0 <= r < h and 0 <= q < w:
                    exp_dx[b, :, r, q] = wt[o, :, kh, kw]
                    exp_dw[o, :, kh, kw] = x[b, :, r, q]
        np.testing.assert_array_equal(O.conv_backward_data(wt, dz, (h, w), s, p), exp_dx)
        np.testing.assert_array_equal(O.conv_backward_weights(x, dz, k, s, p), exp_dw)


def _im2col(img, k, s, p):
    """The pages' im2col index map: row c of the column matrix is (c_im, h_off, w_off) =
    (c / k^2, (c / k) % k, c % k); column (h, w) reads img[c_im, h_off + h*s - p, w_off + w*s - p],
    zero outside the image."""
    c, h, w = img.shape
    oh, ow = (h + 2 * p - k) // s + 1, (w + 2 * p - k) // s + 1
    col = np.zeros((c * k * k, oh * ow))
    for cc in range(c * k * k):
        w_off, h_off, c_im = cc % k, (cc // k) % k, cc // k // k
        for y in range(oh):
            for xx in range(ow):
                r, q = h_off + y * s - p, w_off + xx * s - p
                if 0 <= r < h and 0 <= q < w:
                    col[cc, y * ow + xx] = img[c_im, r, q]
    return col


def _col2im(col, c, h, w, k, s, p):
    """col2im: add every column value back at the pixel im2col read it from."""
    oh, ow = (h + 2 * p - k) // s + 1, (w + 2 * p - k) // s + 1
    img = np.zeros((c, h, w))
    for cc in range(c * k * k):
        w_off, h_off, c_im = cc % k, (cc // k) % k, cc // k // k
        for y in range(oh):
            for xx in range(ow):
                r, q = h_off + y * s - p, w_off + xx * s - p
                if 0 <= r < h and 0 <= q < w:
                    img[c_im, r, q] += col[cc, y * ow + xx]
    return img


@pytest.mark.parametrize("shape", [(2, 3, 9, 8, 4, 3, 1, 1), (2, 2, 9, 9, 3, 3, 2, 1),
                                   (1, 3, 10, 10, 2, 5, 1, 2), (2, 4, 6, 6, 5, 1, 1, 0)])
def test_im2col_gemm_route(shape):
    """Second path: per image, dW += dz(m x k) . col^T and dX = col2im(W^T(n x m) . dz)."""
    n, c, h, w, oc, k, s, p = shape
    x, wt = _rand(41, n, c, h, w), _rand(42, oc, c, k, k)
    oh, ow = O.conv_out_dim(h, k, s, p), O.conv_out_dim(w, k, s, p)
    dz = _rand(43, n, oc, oh, ow)
    dw = np.zeros((oc, c * k * k))
    dx = np.zeros((n, c, h, w))
    wm = wt.reshape(oc, c * k * k)
    for b in range(n):
        col = _im2col(x[b], k, s, p)
        a = dz[b].reshape(oc, oh * ow)
        dw += a @ col.T
        dx[b] = _col2im(wm.T @ a, c, h, w, k, s, p)
    np.testing.assert_allclose(O.conv_backward_weights(x, dz, k, s, p), dw.reshape(wt.shape),
                               rtol=0, atol=1e-11)
    np.testing.assert_allclose(O.conv_backward_data(wt, dz, (h, w), s, p), dx, rtol=0, atol=1e-11)


def test_output_dims():
    # im2col: (size + 2 pad - k)/stride + 1; the workloads' shapes
    assert O.conv_out_dim(416, 3, 2, 1) == 208
    assert O.conv_out_dim(416, 3, 1, 1) == 416
    assert O.conv_out_dim(12, 5, 1, 0) == 8
    assert O.conv_out_dim(28, 5, 1, 0) == 24
    assert O.lib().orc_conv_out_dim(52, 3, 1, 1) == 52


# ----------------------------------------------------------------------------- groups, dilation
GD_SHAPES = [  # n, c, h, w, oc, k, s, p, d, groups
    (2, 4, 9, 9, 6, 3, 1, 1, 1, 2),
    (2, 6, 11, 10, 6, 3, 2, 2, 2, 3),
    (1, 3, 12, 12, 4, 3, 1, 2, 2, 1),
    (2, 8, 13, 9, 8, 5, 1, 4, 2, 8),     # depthwise
    (1, 4, 10, 11, 2, 1, 1, 0, 1, 2),    # grouped 1x1
    (2, 2, 15, 14, 4, 3, 3, 1, 3, 2),    # stride 3, dilation 3
]


@pytest.mark.parametrize("shape", GD_SHAPES)
def test_grouped_dilated_conv_matches_float64_autograd(shape):
    """Forward, dW and dX of the grouped / dilated convolution against float64 autograd of
    torch's conv2d with the same groups and dilation."""
    n, c, h, w, oc, k, s, p, d, g = shape
    r = np.random.default_rng(71)
    x = r.normal(size=(n, c, h, w))
    wt = r.normal(size=(oc, c // g, k, k))
    tx = torch.tensor(x, requires_grad=True)
    tw = torch.tensor(wt, requires_grad=True)
    tz = torch.nn.functional.conv2d(tx, tw, stride=s, padding=p, dilation=d, groups=g)
    z = O.conv_forward_gd(x, wt, s, p, d, g)
    assert z.shape == tuple(tz.shape)
    np.testing.assert_allclose(z, tz.detach().numpy(), rtol=0, atol=1e-12)
    dz = r.normal(size=z.shape)
    tz.backward(torch.tensor(dz))
    np.testing.assert_allclose(O.conv_backward_weights_gd(x, dz, k, s, p, d, g), tw.grad.numpy(),
                               rtol=0, atol=1e-11)
    np.testing.assert_allclose(O.conv_backward_data_gd(wt, dz, (h, w), s, p, d, g),
                               tx.grad.numpy(), rtol=0, atol=1e-11)


def test_grouped_dilated_conv_reduces_to_plain_conv():
    """groups = dilation = 1 gives the ungrouped functions' results exactly."""
    n, c, h, w, oc, k, s, p = 2, 3, 9, 8, 5, 3, 2, 1
    r = np.random.default_rng(72)
    x, wt = r.normal(size=(n, c, h, w)), r.normal(size=(oc, c, k, k))
    z = O.conv_forward(x, wt, s, p)
    np.testing.assert_array_equal(O.conv_forward_gd(x, wt, s, p, 1, 1), z)
    dz = r.normal(size=z.shape)
    np.testing.assert_array_equal(O.conv_backward_weights_gd(x, dz, k, s, p, 1, 1),
                                  O.conv_backward_weights(x, dz, k, s, p))
    np.testing.assert_allclose(O.conv_backward_data_gd(wt, dz, (h, w), s, p, 1, 1),
                               O.conv_backward_data(wt, dz, (h, w), s, p), rtol=0, atol=1e-13)
