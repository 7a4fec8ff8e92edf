"""Pins for the oracle's activation and batch-norm steps (CPU only)."""
import numpy as np
import pytest
import torch

import oracle as O

EPS = 1e-5


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------- activations
def test_leaky_and_relu_gradients_take_page_values():
    y = np.array([-2.0, -1e-30, 0.0, 1e-30, 3.0])
    d = np.ones_like(y)
    # leaky_gradient: (x>0) ? 1 : .1, evaluated on the output
    np.testing.assert_array_equal(O.act_backward(O.ACT_LEAKY, 0.1, y, d), [0.1, 0.1, 0.1, 1, 1])
    np.testing.assert_array_equal(O.act_backward(O.ACT_RELU, 0.0, y, d), [0, 0, 0, 1, 1])
    np.testing.assert_array_equal(O.act_backward(O.ACT_LINEAR, 0.0, y, d), [1, 1, 1, 1, 1])


def test_logistic_two_forms_and_derivative():
    """Caffe's sigmoid 0.5*tanh(0.5x)+0.5 equals Darknet's 1/(1+e^-x); the gradient on the
    output, (1-y)y, equals the finite-difference derivative of the forward."""
    u = np.linspace(-8, 8, 161)
    y = O.act_forward(O.ACT_LOGISTIC, 0.0, u)
    np.testing.assert_allclose(y, 0.5 * np.tanh(0.5 * u) + 0.5, rtol=0, atol=1e-15)
    g = O.act_backward(O.ACT_LOGISTIC, 0.0, y, np.ones_like(y))
    h = 1e-6
    fd = (O.act_forward(O.ACT_LOGISTIC, 0, u + h) - O.act_forward(O.ACT_LOGISTIC, 0, u - h)) / (2 * h)
    np.testing.assert_allclose(g, fd, rtol=1e-7, atol=1e-10)


@pytest.mark.parametrize("act,slope", [(O.ACT_LEAKY, 0.1), (O.ACT_RELU, 0.0), (O.ACT_LINEAR, 0.0),
                                       (O.ACT_LOGISTIC, 0.0)])
def test_activation_backward_matches_autograd(act, slope):
    u = _rand(1, 4, 3, 5, 5)
    u[np.abs(u) < 1e-3] = 0.5          # keep away from the kink
    d = _rand(2, *u.shape)
    tu = torch.tensor(u, requires_grad=True)
    f = {O.ACT_LEAKY: lambda t: torch.nn.functional.leaky_relu(t, slope),
         O.ACT_RELU: torch.relu, O.ACT_LINEAR: lambda t: t * 1.0, O.ACT_LOGISTIC: torch.sigmoid}[act]
    ty = f(tu)
    ty.backward(torch.tensor(d))
    y = O.act_forward(act, slope, u)
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.act_backward(act, slope, y, d), tu.grad.numpy(), rtol=0, atol=1e-14)


# The other ten activations of Darknet's activation list.  Each forward is pinned to an
# independent definition (a torch routine or a mathematical identity), each gradient to the
# central finite difference of the forward away from its breakpoints.
A = O.ACT_NAMES
_F = torch.nn.functional
_FWD_PINS = {
    "tanh": lambda t: torch.tanh(t),
    "elu": lambda t: _F.elu(t, alpha=1.0),
    "selu": lambda t: 1.0507 * _F.elu(t, alpha=1.6732),
    "hardtan": lambda t: _F.hardtanh(t, -1.0, 1.0),
    "relie": lambda t: _F.leaky_relu(t, 0.01),
    "ramp": lambda t: torch.relu(t) + 0.1 * t,
    "loggy": lambda t: torch.tanh(t / 2),                 # 2*sigmoid(x)-1 == tanh(x/2)
    # piecewise-linear ones: a min/max composition of their three pieces
    "plse": lambda t: torch.maximum(torch.minimum(0.125 * t + 0.5, 0.01 * (t - 4) + 1), 0.01 * (t + 4)),
    "lhtan": lambda t: torch.minimum(torch.maximum(0.001 * t, t), 0.001 * (t - 1) + 1),
    # flat at k on [2k, 2k+1), rising from k to k+1 on [2k+1, 2k+2)
    "stair": lambda t: torch.floor(t / 2) + torch.relu(t - 2 * torch.floor(t / 2) - 1),
}
_BREAKS = {"plse": [-4, 4], "lhtan": [0, 1], "hardtan": [-1, 1], "relie": [0], "ramp": [0],
           "elu": [0], "selu": [0], "stair": list(range(-8, 9))}


@pytest.mark.parametrize("name", sorted(_FWD_PINS))
def test_extra_activation_forward_pins(name):
    u = np.linspace(-7.3, 7.3, 2921)
    y = O.act_forward(A[name], 0.0, u)
    ref = _FWD_PINS[name](torch.tensor(u)).numpy()
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-14)


@pytest.mark.parametrize("name", sorted(_FWD_PINS))
def test_extra_activation_gradient_is_derivative_of_forward(name):
    u = np.random.default_rng(7).uniform(-7, 7, 4000)
    for b in _BREAKS.get(name, []):
        u = u[np.abs(u - b) > 1e-3]
    h = 1e-6
    fd = (O.act_forward(A[name], 0, u + h) - O.act_forward(A[name], 0, u - h)) / (2 * h)
    y = O.act_forward(A[name], 0.0, u)
    d = np.random.default_rng(8).standard_normal(u.shape)
    g = O.act_backward(A[name], 0.0, y, d)
    np.testing.assert_allclose(g, d * fd, rtol=1e-6, atol=1e-8)


def test_extra_activation_gradients_at_page_breakpoints():
    """Values the gradient functions take at and around their thresholds, read from the output."""
    one = np.ones(5)
    g = lambda n, y: O.act_backward(A[n], 0.0, np.array(y, dtype=np.float64), one[:len(y)])
    np.testing.assert_array_equal(g("plse", [-0.5, 0.0, 0.5, 1.0, 1.5]), [.01, .125, .125, .125, .01])
    np.testing.assert_array_equal(g("lhtan", [-0.5, 0.0, 0.5, 1.0, 1.5]), [.001, .001, 1, .001, .001])
    np.testing.assert_array_equal(g("hardtan", [-1.0, -0.5, 0.5, 1.0]), [0, 1, 1, 0])
    np.testing.assert_array_equal(g("stair", [-1.0, -0.5, 0.0, 2.0, 2.25]), [0, 1, 0, 0, 1])
    np.testing.assert_array_equal(g("ramp", [-1.0, 0.0, 1.0]), [.1, .1, 1.1])
    np.testing.assert_array_equal(g("relie", [-1.0, 0.0, 1.0]), [.01, .01, 1])
    np.testing.assert_array_equal(g("elu", [-0.5, 0.0, 2.0]), [0.5, 1, 1])
    np.testing.assert_allclose(g("selu", [-0.5, 0.0, 2.0]), [1.0507 * 1.6732 - 0.5, 1.0507, 1.0507],
                               rtol=0, atol=1e-15)
    np.testing.assert_allclose(g("loggy", [-1.0, 0.0, 1.0]), [0, 0.5, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(g("tanh", [-1.0, 0.0, 0.5]), [0, 1, 0.75], rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------- batch norm
def _bn_case(seed, shape, gamma_scale=1.0):
    z = _rand(seed, *shape) * 2.0 + 0.3
    c = shape[1]
    gamma = 1.0 + gamma_scale * _rand(seed + 1, c)
    beta = _rand(seed + 2, c)
    return z, gamma, beta


@pytest.mark.parametrize("shape", [(2, 3, 4, 4), (4, 5, 3, 7), (1, 2, 6, 6), (8, 3, 1, 1)])
def test_bn_forward_backward_match_autograd(shape):
    z, gamma, beta = _bn_case(3, shape)
    mean, var, xhat, u = O.bn_forward(z, gamma, beta, EPS)
    tz = torch.tensor(z, requires_grad=True)
    tg = torch.tensor(gamma, requires_grad=True)
    tb = torch.tensor(beta, requires_grad=True)
    tu = torch.nn.functional.batch_norm(tz, None, None, tg, tb, training=True, eps=EPS)
    np.testing.assert_allclose(u, tu.detach().numpy(), rtol=0, atol=1e-12)
    g = _rand(9, *shape)
    tu.backward(torch.tensor(g))
    dz, dgamma, dbeta = O.bn_backward(g, xhat, var, gamma, EPS)
    np.testing.assert_allclose(dz, tz.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dgamma, tg.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dbeta, tb.grad.numpy(), rtol=0, atol=1e-11)


def _darknet_three_step(g, z, mean, var, gamma):
    """Darknet's route: scale_bias (delta *= gamma), mean_delta = sum(delta) * (-1/sqrt(var+eps)),
    variance_delta = sum(delta (x-mean)) * (-1/2) (var+eps)^(-3/2),
    delta = delta/sqrt(var+eps) + variance_delta * 2 (x-mean)/m + mean_delta/m."""
    n, c = g.shape[:2]
    m = g.size // c
    ax = (0, 2, 3)
    d = g * gamma[None, :, None, None]
    md = d.sum(axis=ax) * (-1.0 / np.sqrt(var + EPS))
    xm = z - mean[None, :, None, None]
    vd = (d * xm).sum(axis=ax) * (-0.5 * (var + EPS) ** -1.5)
    b = lambda v: v[None, :, None, None]
    return d / b(np.sqrt(var + EPS)) + b(vd) * 2.0 * xm / m + b(md) / m


@pytest.mark.parametrize("shape", [(2, 3, 4, 4), (3, 4, 5, 2), (2, 6, 13, 13)])
def test_bn_backward_two_page_formulas_agree(shape):
    """The Caffe closed form the oracle uses equals Darknet's three-step chain rule."""
    z, gamma, _ = _bn_case(5, shape)
    mean, var, xhat, _ = O.bn_forward(z, gamma, np.zeros(shape[1]), EPS)
    g = _rand(6, *shape)
    dz, dgamma, dbeta = O.bn_backward(g, xhat, var, gamma, EPS)
    np.testing.assert_allclose(dz, _darknet_three_step(g, z, mean, var, gamma), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dbeta, g.sum(axis=(0, 2, 3)), atol=1e-12)
    np.testing.assert_allclose(dgamma, (g * xhat).sum(axis=(0, 2, 3)), atol=1e-12)


@pytest.mark.parametrize("shape", [(2, 3, 4, 4), (8, 5, 13, 13)])
def test_bn_invariants(shape):
    """With a consistent forward, sum dz = 0 per channel and
    sum dz*xhat = (gamma/sigma) dgamma eps/(var+eps) (not zero: eps > 0)."""
    z, gamma, beta = _bn_case(7, shape)
    mean, var, xhat, _ = O.bn_forward(z, gamma, beta, EPS)
    ax = (0, 2, 3)
    np.testing.assert_allclose(xhat.sum(axis=ax), 0.0, atol=1e-10)
    np.testing.assert_allclose((xhat ** 2).mean(axis=ax), var / (var + EPS), rtol=1e-12)
    g = _rand(8, *shape)
    dz, dgamma, _ = O.bn_backward(g, xhat, var, gamma, EPS)
    scale = np.abs(dz).sum(axis=ax)
    assert np.all(np.abs(dz.sum(axis=ax)) <= 1e-12 * scale)
    sig = np.sqrt(var + EPS)
    np.testing.assert_allclose((dz * xhat).sum(axis=ax), gamma / sig * dgamma * EPS / (var + EPS),
                               rtol=1e-6, atol=1e-12 * scale.max())


def test_bn_finite_differences_tiny():
    shape = (2, 2, 3, 3)
    z, gamma, beta = _bn_case(11, shape)
    g = _rand(12, *shape)

    def loss(zz, gg, bb):
        return float(np.sum(O.bn_forward(zz, gg, bb, EPS)[3] * g))

    _, var, xhat, _ = O.bn_forward(z, gamma, beta, EPS)
    dz, dgamma, dbeta = O.bn_backward(g, xhat, var, gamma, EPS)
    h = 1e-6
    for idx in np.ndindex(*shape):
        zp, zm = z.copy(), z.copy()
        zp[idx] += h
        zm[idx] -= h
        fd = (loss(zp, gamma, beta) - loss(zm, gamma, beta)) / (2 * h)
        assert fd == pytest.approx(dz[idx], rel=1e-6, abs=1e-8)
    for ch in range(shape[1]):
        gp, gm = gamma.copy(), gamma.copy()
        gp[ch] += h
        gm[ch] -= h
        assert (loss(z, gp, beta) - loss(z, gm, beta)) / (2 * h) == pytest.approx(dgamma[ch], rel=1e-6)
        bp, bm = beta.copy(), beta.copy()
        bp[ch] += h
        bm[ch] -= h
        assert (loss(z, gamma, bp) - loss(z, gamma, bm)) / (2 * h) == pytest.approx(dbeta[ch], rel=1e-6)


def test_bn_parameter_gradients_accumulate():
    shape = (2, 3, 4, 4)
    z, gamma, beta = _bn_case(13, shape)
    _, var, xhat, _ = O.bn_forward(z, gamma, beta, EPS)
    g = _rand(14, *shape)
    _, dg1, db1 = O.bn_backward(g, xhat, var, gamma, EPS)
    _, dg2, db2 = O.bn_backward(g, xhat, var, gamma, EPS, dgamma=dg1, dbeta=db1)
    np.testing.assert_allclose(dg2, 2 * dg1, rtol=1e-15)
    np.testing.assert_allclose(db2, 2 * db1, rtol=1e-15)


# ----------------------------------------------------------------------------- fixed statistics
def _fixed_stats(seed, c):
    r = np.random.default_rng(seed)
    return r.normal(size=c), r.uniform(0.3, 3.0, size=c)


@pytest.mark.parametrize("shape", [(2, 3, 4, 4), (4, 5, 3, 7), (8, 3, 1, 1)])
def test_bn_fixed_statistics_match_autograd(shape):
    """Forward and backward with stored statistics against float64 autograd of torch's
    batch_norm in evaluation mode (running mean and variance, no batch statistics)."""
    z, gamma, beta = _bn_case(21, shape)
    mean, var = _fixed_stats(22, shape[1])
    xhat, u = O.bn_forward_fixed(z, mean, var, gamma, beta, EPS)
    tz = torch.tensor(z, requires_grad=True)
    tg = torch.tensor(gamma, requires_grad=True)
    tb = torch.tensor(beta, requires_grad=True)
    tu = torch.nn.functional.batch_norm(tz, torch.tensor(mean), torch.tensor(var), tg, tb,
                                        training=False, eps=EPS)
    np.testing.assert_allclose(u, tu.detach().numpy(), rtol=0, atol=1e-12)
    g = _rand(23, *shape)
    tu.backward(torch.tensor(g))
    dz, dgamma, dbeta = O.bn_backward_fixed(g, xhat, var, gamma, EPS)
    np.testing.assert_allclose(dz, tz.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dgamma, tg.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dbeta, tb.grad.numpy(), rtol=0, atol=1e-11)


def test_bn_fixed_statistics_finite_differences_and_caffe_form():
    """Central differences of the fixed-statistics forward; with gamma = 1 the input
    gradient is Caffe's use_global_stats branch: the top gradient divided by
    sqrt(var + eps) (a division, as the code on the BatchNorm page does)."""
    shape = (2, 2, 3, 3)
    z, gamma, beta = _bn_case(24, shape)
    mean, var = _fixed_stats(25, shape[1])
    g = _rand(26, *shape)

    def loss(zz, gg, bb):
        return float(np.sum(O.bn_forward_fixed(zz, mean, var, gg, bb, EPS)[1] * g))

    xhat, _ = O.bn_forward_fixed(z, mean, var, gamma, beta, EPS)
    dz, dgamma, dbeta = O.bn_backward_fixed(g, xhat, var, gamma, EPS)
    h = 1e-6
    for idx in np.ndindex(*shape):
        zp, zm = z.copy(), z.copy()
        zp[idx] += h
        zm[idx] -= h
        assert (loss(zp, gamma, beta) - loss(zm, gamma, beta)) / (2 * h) == \
            pytest.approx(dz[idx], rel=1e-6, abs=1e-8)
    for ch in range(shape[1]):
        gp, gm = gamma.copy(), gamma.copy()
        gp[ch] += h
        gm[ch] -= h
        assert (loss(z, gp, beta) - loss(z, gm, beta)) / (2 * h) == pytest.approx(dgamma[ch], rel=1e-6)
        bp, bm = beta.copy(), beta.copy()
        bp[ch] += h
        bm[ch] -= h
        assert (loss(z, gamma, bp) - loss(z, gamma, bm)) / (2 * h) == pytest.approx(dbeta[ch], rel=1e-6)
    dz1, _, _ = O.bn_backward_fixed(g, xhat, var, np.ones(shape[1]), EPS)
    np.testing.assert_allclose(dz1, g / np.sqrt(var + EPS)[None, :, None, None], rtol=1e-15)


@pytest.mark.parametrize("shape", [(4, 3, 5, 7), (16, 2, 9, 9)])
def test_bn_forward_statistics_are_batch_mean_and_biased_variance(shape):
    """The statistics the forward returns (and the GPU forward must reproduce): per channel
    over (batch, space), the mean and the variance with divisor m (numpy's ddof = 0)."""
    z, gamma, beta = _bn_case(41, shape)
    z = z * 3.0 + 5.0   # an offset mean: the two-pass variance must not cancel
    mean, var, xhat, _ = O.bn_forward(z, gamma, beta, EPS)
    np.testing.assert_allclose(mean, z.mean(axis=(0, 2, 3)), rtol=1e-14)
    np.testing.assert_allclose(var, z.var(axis=(0, 2, 3), ddof=0), rtol=1e-12)
    np.testing.assert_allclose(xhat, (z - mean[None, :, None, None])
                               / np.sqrt(var + EPS)[None, :, None, None], rtol=1e-12, atol=1e-13)
