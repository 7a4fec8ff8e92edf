"""Pins of the oracle's parameter update (the step after the backward pass).

The pages name the step (update_network -> l.update(layer, batch, learning_rate,
momentum, decay) once per full batch; weight_updates is the gradient term that the
step size multiplies) but print no formula.  The reading -- gradient descent with
momentum and L2 decay, the accumulated-gradient buffer doubling as the momentum
buffer -- is pinned to torch.optim.SGD, an independent implementation of the same
recursion: SGD(lr, momentum, weight_decay=decay) fed the batch-mean gradient
dw_new / batch reproduces the oracle's weights step after step, when the backward
adds each new batch's gradient onto the buffer the previous update left."""
import numpy as np
import pytest

import oracle as O


@pytest.mark.parametrize("lr,mom,decay,batch", [(0.1, 0.9, 5e-4, 8), (0.01, 0.0, 0.0, 1),
                                                (1e-3, 0.95, 1e-2, 64), (0.5, 0.5, 0.0, 3)])
def test_update_matches_torch_sgd_over_several_steps(lr, mom, decay, batch):
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(17)
    w0 = r.normal(size=(6, 5))
    grads = [r.normal(size=w0.shape) * batch for _ in range(5)]   # summed over the batch
    # oracle: the backward adds each batch's gradient onto the buffer, then the update
    w, buf = w0.copy(), np.zeros_like(w0)
    # torch: the same batch-mean gradients
    p = torch.nn.Parameter(torch.tensor(w0, dtype=torch.float64))
    opt = torch.optim.SGD([p], lr=lr, momentum=mom, weight_decay=decay)
    for gsum in grads:
        w, buf = O.sgd_update(w, buf + gsum, batch, lr, mom, decay)
        p.grad = torch.tensor(gsum / batch, dtype=torch.float64)
        opt.step()
        np.testing.assert_allclose(w, p.detach().numpy(), rtol=1e-12, atol=1e-12)


def test_update_special_cases():
    r = np.random.default_rng(3)
    w0, g = r.normal(size=40), r.normal(size=40)
    # no momentum, no decay: one plain step, the buffer cleared
    w, d = O.sgd_update(w0, g, 4, 0.2, 0.0, 0.0)
    np.testing.assert_array_equal(d, np.zeros(40))
    np.testing.assert_allclose(w, w0 - 0.05 * g, rtol=0, atol=1e-15)
    # zero gradient: decay alone shrinks the weights by (1 - lr * decay)
    w, d = O.sgd_update(w0, np.zeros(40), 16, 0.1, 0.9, 0.01)
    np.testing.assert_allclose(w, w0 * (1 - 0.1 * 0.01), rtol=1e-14)
    np.testing.assert_allclose(d, 0.9 * 0.01 * 16 * w0, rtol=1e-14)


def test_update_descends_a_quadratic():
    """Gradient descent on L(w) = 1/2 sum_b |w - t_b|^2 (gradient summed over b)
    reaches the mean target."""
    r = np.random.default_rng(5)
    t = r.normal(size=(8, 10))
    w, buf = np.zeros(10), np.zeros(10)
    for _ in range(200):
        w, buf = O.sgd_update(w, buf + (8 * w - t.sum(axis=0)), 8, 0.1, 0.5, 0.0)
    np.testing.assert_allclose(w, t.mean(axis=0), atol=1e-8)
