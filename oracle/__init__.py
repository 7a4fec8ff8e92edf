"""CPU oracle for the convolutional-block backward pass (double precision).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product path
(the HIP library ``libcbb.so`` and its binding ``cnn_backward_pass_amd``) never
does, and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, direct loops, OpenMP over
independent outputs).  This module only compiles it with gcc, marshals numpy
float64 arrays through ctypes, and composes the per-layer steps into the
per-block and per-workload passes in ``oracle/model.py``.

Parity status: every function exported here is pinned by a ``-m "not gpu"``
test in ``tests/test_oracle_*.py`` (finite differences, an independent float64
autograd library, closed forms and invariants); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "oracle.c")
_LIB_PATH = os.path.join(_DIR, "liboracle.so")
_lock = threading.Lock()
_lib = None

ACT_LINEAR, ACT_LEAKY, ACT_LOGISTIC, ACT_RELU = 0, 1, 2, 3
ACT_NAMES = {"linear": ACT_LINEAR, "leaky": ACT_LEAKY, "logistic": ACT_LOGISTIC, "relu": ACT_RELU,
             "tanh": 4, "elu": 5, "selu": 6, "plse": 7, "lhtan": 8, "hardtan": 9, "stair": 10,
             "ramp": 11, "relie": 12, "loggy": 13}


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, no fast-math)."""
    with _lock:
        if (not force and os.path.exists(_LIB_PATH)
                and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC)):
            return _LIB_PATH
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
        return _LIB_PATH


_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int)
_L = ctypes.POINTER(ctypes.c_long)
_i, _l, _d = ctypes.c_int, ctypes.c_long, ctypes.c_double

_SIGS = {
    "orc_version": ([], _i),
    "orc_num_threads": ([], _i),
    "orc_set_threads": ([_i], None),
    "orc_act_forward": ([_i, _d, _D, _D, _l], None),
    "orc_act_backward": ([_i, _d, _D, _D, _D, _l], None),
    "orc_bn_forward": ([_i, _i, _l, _d, _D, _D, _D, _D, _D, _D, _D], None),
    "orc_bn_backward": ([_i, _i, _l, _d, _D, _D, _D, _D, _D, _D, _D], None),
    "orc_bn_forward_fixed": ([_i, _i, _l, _d, _D, _D, _D, _D, _D, _D, _D], None),
    "orc_bn_backward_fixed": ([_i, _i, _l, _d, _D, _D, _D, _D, _D, _D, _D], None),
    "orc_conv_out_dim": ([_i, _i, _i, _i], _i),
    "orc_conv_forward": ([_i] * 8 + [_D, _D, _D, _D], None),
    "orc_conv_backward_weights": ([_i] * 8 + [_D, _D, _D], None),
    "orc_conv_dw_at": ([_i] * 8 + [_D, _D, _i, _i, _i, _i], _d),
    "orc_conv_backward_bias": ([_i, _i, _l, _D, _D], None),
    "orc_conv_backward_data": ([_i] * 8 + [_D, _D, _D], None),
    "orc_conv_dx_at": ([_i] * 8 + [_D, _D, _i, _i, _i, _i], _d),
    "orc_maxpool_forward": ([_i] * 6 + [_D, _D, _I], None),
    "orc_maxpool_backward": ([_i] * 6 + [_I, _D, _D], None),
    "orc_fc_forward": ([_i, _i, _i, _D, _D, _D, _D], None),
    "orc_fc_backward": ([_i, _i, _i, _D, _D, _D, _D, _D, _D, _i], None),
    "orc_softmax_forward": ([_i, _i, _D, _D], None),
    "orc_conv_out_dim_d": ([_i] * 5, _i),
    "orc_conv_forward_gd": ([_i] * 10 + [_D, _D, _D, _D], None),
    "orc_conv_backward_weights_gd": ([_i] * 10 + [_D, _D, _D], None),
    "orc_conv_backward_data_gd": ([_i] * 10 + [_D, _D, _D], None),
    "orc_softmax_loss": ([_i, _i, _D, _I], _d),
    "orc_softmax_backward": ([_i, _i, _l, _D, _D, _D], None),
    "orc_softmax_loss_backward": ([_i, _i, _D, _I, _d, _D], None),
    "orc_shortcut_backward": ([_l, _d, _d, _D, _D, _D], None),
    "orc_shortcut_backward_resize": ([_i] * 7 + [_d, _d, _D, _D, _D], None),
    "orc_route_backward": ([_i, _i, _L, _D, ctypes.POINTER(_D)], None),
    "orc_upsample_forward": ([_i] * 5 + [_D, _D], None),
    "orc_upsample_backward": ([_i] * 5 + [_D, _D], None),
    "orc_sgd_update": ([_l, _i, _d, _d, _d, _D, _D], None),
}


def lib():
    global _lib
    if _lib is None:
        build()
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(_D)


def _pi(a: np.ndarray):
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(_I)


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use (omp_get_max_threads)."""
    return lib().orc_num_threads()


def set_threads(n: int) -> None:
    """Threads of the oracle's following OpenMP loops (1: single core)."""
    lib().orc_set_threads(int(n))


def conv_out_dim(size: int, k: int, s: int, p: int) -> int:
    return (size + 2 * p - k) // s + 1


# ---------------------------------------------------------------- activations
def act_forward(act: int, slope: float, u) -> np.ndarray:
    u = _f64(u)
    y = np.empty_like(u)
    lib().orc_act_forward(act, slope, _p(u), _p(y), u.size)
    return y


def act_backward(act: int, slope: float, y, delta) -> np.ndarray:
    """g = delta * act'(y), act' read from the output y (Darknet gradient_array)."""
    y, delta = _f64(y), _f64(delta)
    assert y.shape == delta.shape
    g = np.empty_like(y)
    lib().orc_act_backward(act, slope, _p(y), _p(delta), _p(g), y.size)
    return g


# ---------------------------------------------------------------- batch norm
def bn_forward(z, gamma, beta, eps: float):
    """Training-mode BN over (N, H*W) per channel; returns mean, var(biased), xhat, u."""
    z = _f64(z)
    n, c = z.shape[0], z.shape[1]
    hw = int(np.prod(z.shape[2:])) if z.ndim > 2 else 1
    gamma, beta = _f64(gamma), _f64(beta)
    mean, var = np.empty(c), np.empty(c)
    xhat, u = np.empty_like(z), np.empty_like(z)
    lib().orc_bn_forward(n, c, hw, eps, _p(z), _p(gamma), _p(beta), _p(mean), _p(var), _p(xhat),
                         _p(u))
    return mean, var, xhat, u


def bn_backward(g, xhat, var, gamma, eps: float, dgamma=None, dbeta=None):
    """Returns dz, dgamma (+= into the given array), dbeta (+=)."""
    g, xhat = _f64(g), _f64(xhat)
    n, c = g.shape[0], g.shape[1]
    hw = int(np.prod(g.shape[2:])) if g.ndim > 2 else 1
    var, gamma = _f64(var), _f64(gamma)
    dgamma = np.zeros(c) if dgamma is None else _f64(dgamma).copy()
    dbeta = np.zeros(c) if dbeta is None else _f64(dbeta).copy()
    dz = np.empty_like(g)
    lib().orc_bn_backward(n, c, hw, eps, _p(g), _p(xhat), _p(var), _p(gamma), _p(dz), _p(dgamma),
                          _p(dbeta))
    return dz, dgamma, dbeta


def bn_forward_fixed(z, mean, var, gamma, beta, eps: float):
    """BN with fixed (stored) statistics; returns xhat, u."""
    z = _f64(z)
    n, c = z.shape[0], z.shape[1]
    hw = int(np.prod(z.shape[2:])) if z.ndim > 2 else 1
    mean, var, gamma, beta = _f64(mean), _f64(var), _f64(gamma), _f64(beta)
    xhat, u = np.empty_like(z), np.empty_like(z)
    lib().orc_bn_forward_fixed(n, c, hw, eps, _p(z), _p(mean), _p(var), _p(gamma), _p(beta),
                               _p(xhat), _p(u))
    return xhat, u


def bn_backward_fixed(g, xhat, var, gamma, eps: float, dgamma=None, dbeta=None):
    """BN backward with fixed statistics; returns dz, dgamma (+=), dbeta (+=)."""
    g, xhat = _f64(g), _f64(xhat)
    n, c = g.shape[0], g.shape[1]
    hw = int(np.prod(g.shape[2:])) if g.ndim > 2 else 1
    var, gamma = _f64(var), _f64(gamma)
    dgamma = np.zeros(c) if dgamma is None else _f64(dgamma).copy()
    dbeta = np.zeros(c) if dbeta is None else _f64(dbeta).copy()
    dz = np.empty_like(g)
    lib().orc_bn_backward_fixed(n, c, hw, eps, _p(g), _p(xhat), _p(var), _p(gamma), _p(dz),
                                _p(dgamma), _p(dbeta))
    return dz, dgamma, dbeta


# ---------------------------------------------------------------- convolution
def conv_forward(x, w, stride: int, pad: int, bias=None) -> np.ndarray:
    x, w = _f64(x), _f64(w)
    n, c, h, wd = x.shape
    oc, c2, k, k2 = w.shape
    assert c2 == c and k == k2
    oh, ow = conv_out_dim(h, k, stride, pad), conv_out_dim(wd, k, stride, pad)
    z = np.empty((n, oc, oh, ow))
    b = None if bias is None else _f64(bias)
    lib().orc_conv_forward(n, c, h, wd, oc, k, stride, pad, _p(x), _p(w), _p(b), _p(z))
    return z


def conv_backward_weights(x, dz, k: int, stride: int, pad: int, dw=None) -> np.ndarray:
    x, dz = _f64(x), _f64(dz)
    n, c, h, wd = x.shape
    oc = dz.shape[1]
    assert dz.shape == (n, oc, conv_out_dim(h, k, stride, pad), conv_out_dim(wd, k, stride, pad))
    dw = np.zeros((oc, c, k, k)) if dw is None else _f64(dw).copy()
    lib().orc_conv_backward_weights(n, c, h, wd, oc, k, stride, pad, _p(x), _p(dz), _p(dw))
    return dw


def conv_dw_at(x, dz, k: int, stride: int, pad: int, o: int, i: int, kh: int, kw: int) -> float:
    x, dz = _f64(x), _f64(dz)
    n, c, h, wd = x.shape
    oc = dz.shape[1]
    return lib().orc_conv_dw_at(n, c, h, wd, oc, k, stride, pad, _p(x), _p(dz), o, i, kh, kw)


def conv_backward_bias(dz, db=None) -> np.ndarray:
    dz = _f64(dz)
    n, oc = dz.shape[0], dz.shape[1]
    ohw = int(np.prod(dz.shape[2:])) if dz.ndim > 2 else 1
    db = np.zeros(oc) if db is None else _f64(db).copy()
    lib().orc_conv_backward_bias(n, oc, ohw, _p(dz), _p(db))
    return db


def conv_backward_data(w, dz, in_hw, stride: int, pad: int, dx=None) -> np.ndarray:
    w, dz = _f64(w), _f64(dz)
    oc, c, k, _ = w.shape
    n = dz.shape[0]
    h, wd = in_hw
    assert dz.shape == (n, oc, conv_out_dim(h, k, stride, pad), conv_out_dim(wd, k, stride, pad))
    dx = np.zeros((n, c, h, wd)) if dx is None else _f64(dx).copy()
    lib().orc_conv_backward_data(n, c, h, wd, oc, k, stride, pad, _p(w), _p(dz), _p(dx))
    return dx


def conv_out_dim_d(size: int, k: int, s: int, p: int, d: int) -> int:
    return int(lib().orc_conv_out_dim_d(size, k, s, p, d))


def conv_forward_gd(x, w, stride: int, pad: int, dilation: int, groups: int, bias=None):
    """Grouped, dilated convolution; w is [oc, c/groups, k, k]."""
    x, w = _f64(x), _f64(w)
    n, c, h, wd = x.shape
    oc, cg, k, _ = w.shape
    assert cg * groups == c and oc % groups == 0
    oh, ow = conv_out_dim_d(h, k, stride, pad, dilation), conv_out_dim_d(wd, k, stride, pad, dilation)
    z = np.empty((n, oc, oh, ow))
    b = None if bias is None else _f64(bias)
    lib().orc_conv_forward_gd(n, c, h, wd, oc, k, stride, pad, dilation, groups, _p(x), _p(w), _p(b),
                              _p(z))
    return z


def conv_backward_weights_gd(x, dz, k: int, stride: int, pad: int, dilation: int, groups: int,
                             dw=None):
    x, dz = _f64(x), _f64(dz)
    n, c, h, wd = x.shape
    oc = dz.shape[1]
    assert dz.shape == (n, oc, conv_out_dim_d(h, k, stride, pad, dilation),
                        conv_out_dim_d(wd, k, stride, pad, dilation))
    dw = np.zeros((oc, c // groups, k, k)) if dw is None else _f64(dw).copy()
    lib().orc_conv_backward_weights_gd(n, c, h, wd, oc, k, stride, pad, dilation, groups, _p(x),
                                       _p(dz), _p(dw))
    return dw


def conv_backward_data_gd(w, dz, in_hw, stride: int, pad: int, dilation: int, groups: int, dx=None):
    w, dz = _f64(w), _f64(dz)
    oc, cg, k, _ = w.shape
    n = dz.shape[0]
    h, wd = in_hw
    c = cg * groups
    assert dz.shape == (n, oc, conv_out_dim_d(h, k, stride, pad, dilation),
                        conv_out_dim_d(wd, k, stride, pad, dilation))
    dx = np.zeros((n, c, h, wd)) if dx is None else _f64(dx).copy()
    lib().orc_conv_backward_data_gd(n, c, h, wd, oc, k, stride, pad, dilation, groups, _p(w),
                                    _p(dz), _p(dx))
    return dx


def conv_dx_at(w, dz, in_hw, stride: int, pad: int, b: int, i: int, row: int, col: int) -> float:
    w, dz = _f64(w), _f64(dz)
    oc, c, k, _ = w.shape
    n = dz.shape[0]
    h, wd = in_hw
    return lib().orc_conv_dx_at(n, c, h, wd, oc, k, stride, pad, _p(w), _p(dz), b, i, row, col)


# ---------------------------------------------------------------- pooling
def maxpool_forward(x, k: int, s: int):
    x = _f64(x)
    n, c, h, w = x.shape
    oh, ow = (h - k) // s + 1, (w - k) // s + 1
    y = np.empty((n, c, oh, ow))
    idx = np.empty((n, c, oh, ow), dtype=np.int32)
    lib().orc_maxpool_forward(n, c, h, w, k, s, _p(x), _p(y), _pi(idx))
    return y, idx


def maxpool_backward(idx, delta, in_hw) -> np.ndarray:
    delta = _f64(delta)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    n, c, oh, ow = delta.shape
    assert idx.shape == delta.shape
    ih, iw = in_hw
    assert idx.min() >= 0 and idx.max() < ih * iw
    dx = np.empty((n, c, ih, iw))
    lib().orc_maxpool_backward(n, c, ih, iw, oh, ow, _pi(idx), _p(delta), _p(dx))
    return dx


# ---------------------------------------------------------------- inner product / softmax
def fc_forward(x, w, bias=None) -> np.ndarray:
    x, w = _f64(x), _f64(w)
    batch, din = x.shape
    dout = w.shape[0]
    y = np.empty((batch, dout))
    b = None if bias is None else _f64(bias)
    lib().orc_fc_forward(batch, din, dout, _p(x), _p(w), _p(b), _p(y))
    return y


def fc_backward(x, w, delta, dw=None, db=None, dx=None, want_dx=True, dx_accumulate=False):
    x, w, delta = _f64(x), _f64(w), _f64(delta)
    batch, din = x.shape
    dout = w.shape[0]
    assert delta.shape == (batch, dout)
    dw = np.zeros((dout, din)) if dw is None else _f64(dw).copy()
    db = np.zeros(dout) if db is None else _f64(db).copy()
    if want_dx:
        dx = np.zeros((batch, din)) if dx is None else _f64(dx).copy()
    else:
        dx = None
    lib().orc_fc_backward(batch, din, dout, _p(x), _p(w), _p(delta), _p(dw), _p(db), _p(dx),
                          int(dx_accumulate))
    return dw, db, dx


def softmax_forward(logits) -> np.ndarray:
    logits = _f64(logits)
    b, c = logits.shape
    prob = np.empty_like(logits)
    lib().orc_softmax_forward(b, c, _p(logits), _p(prob))
    return prob


def softmax_backward(y, dy) -> np.ndarray:
    """Softmax backward along axis 1 of y (outer = axis 0, inner = the axes after 1)."""
    y, dy = _f64(y), _f64(dy)
    outer, channels = y.shape[0], y.shape[1]
    inner = int(np.prod(y.shape[2:])) if y.ndim > 2 else 1
    dx = np.empty_like(y)
    lib().orc_softmax_backward(outer, channels, inner, _p(np.ascontiguousarray(y)),
                               _p(np.ascontiguousarray(dy)), _p(dx))
    return dx


def softmax_loss(prob, labels) -> float:
    prob = _f64(prob)
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    return lib().orc_softmax_loss(prob.shape[0], prob.shape[1], _p(prob), _pi(labels))


def softmax_loss_backward(prob, labels, loss_weight: float = 1.0) -> np.ndarray:
    prob = _f64(prob)
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    b, c = prob.shape
    assert labels.shape == (b,) and labels.min() >= 0 and labels.max() < c
    d = np.empty_like(prob)
    lib().orc_softmax_loss_backward(b, c, _p(prob), _pi(labels), loss_weight, _p(d))
    return d


# ---------------------------------------------------------------- shortcut / route / upsample
def shortcut_backward(delta, d_main, d_from, alpha: float = 1.0, beta: float = 1.0):
    delta = _f64(delta)
    d_main, d_from = _f64(d_main).copy(), _f64(d_from).copy()
    assert d_main.shape == delta.shape == d_from.shape
    lib().orc_shortcut_backward(delta.size, alpha, beta, _p(delta), _p(d_main), _p(d_from))
    return d_main, d_from


def shortcut_backward_resize(delta, d_main, d_from, alpha: float = 1.0, beta: float = 1.0):
    """Shortcut backward between shapes that differ (delta [b,c1,h1,w1], d_from [b,c2,h2,w2]);
    d_main (same shape as delta, or None) += alpha*delta.  Returns (d_main, d_from) copies."""
    delta = _f64(delta)
    b, c1, h1, w1 = delta.shape
    _, c2, h2, w2 = d_from.shape
    d_from = _f64(d_from).copy()
    d_main = None if d_main is None else _f64(d_main).copy()
    lib().orc_shortcut_backward_resize(b, w1, h1, c1, w2, h2, c2, alpha, beta, _p(delta),
                                       None if d_main is None else _p(d_main), _p(d_from))
    return d_main, d_from


def route_backward(delta, d_ins):
    """delta: (batch, sum C_t, ...); d_ins: list of (batch, C_t, ...) arrays (+= into copies)."""
    delta = _f64(delta)
    batch = delta.shape[0]
    outs = [_f64(d).copy() for d in d_ins]
    sizes = (ctypes.c_long * len(outs))(*[int(np.prod(d.shape[1:])) for d in outs])
    assert sum(sizes) * batch == delta.size
    ptrs = (_D * len(outs))(*[_p(d) for d in outs])
    lib().orc_route_backward(batch, len(outs), sizes, _p(delta), ptrs)
    return outs


def upsample_forward(x, scale: int = 2) -> np.ndarray:
    x = _f64(x)
    n, c, h, w = x.shape
    y = np.empty((n, c, h * scale, w * scale))
    lib().orc_upsample_forward(n, c, h, w, scale, _p(x), _p(y))
    return y


def upsample_backward(delta, scale: int = 2, dx=None) -> np.ndarray:
    delta = _f64(delta)
    n, c, hh, ww = delta.shape
    assert hh % scale == 0 and ww % scale == 0
    h, w = hh // scale, ww // scale
    dx = np.zeros((n, c, h, w)) if dx is None else _f64(dx).copy()
    lib().orc_upsample_backward(n, c, h, w, scale, _p(delta), _p(dx))
    return dx


def sgd_update(w, dw, batch: int, lr: float, momentum: float, decay: float):
    """One parameter update (orc_sgd_update): returns the new (w, dw)."""
    w = _f64(w).copy()
    dw = _f64(dw).copy()
    lib().orc_sgd_update(w.size, batch, lr, momentum, decay, _p(w), _p(dw))
    return w, dw
