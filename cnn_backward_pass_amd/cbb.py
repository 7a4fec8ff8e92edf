"""Thin ctypes binding of libcbb.so (C ABI in include/cbb.h).

Argument marshalling only: every function here checks that tensors are CUDA
(HIP) float32/int32 contiguous tensors, passes their device pointers and the
current HIP stream to the ``cbb_*`` entry point of the same name, and raises
``CbbError`` on a non-zero status.  No arithmetic of the backward pass runs in
Python; there is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcbb.so")

ACT = {"linear": 0, "leaky": 1, "logistic": 2, "relu": 3, "tanh": 4, "elu": 5, "selu": 6, "plse": 7,
       "lhtan": 8, "hardtan": 9, "stair": 10, "ramp": 11, "relie": 12, "loggy": 13}
BN_NONE, BN_BATCH, BN_FIXED = 0, 1, 2
STATUS = {0: "CBB_OK", -1: "CBB_EINVAL", -2: "CBB_ESHAPE", -3: "CBB_EUNSUPPORTED",
          -4: "CBB_EWORKSPACE", -5: "CBB_EHIP", -6: "CBB_ESCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024
WORKSPACE_ALIGN = 256


class CbbError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({text})")
        self.status = status


class ConvDesc(ctypes.Structure):
    """cbb_conv_desc."""
    _fields_ = [("batch", ctypes.c_int32), ("in_c", ctypes.c_int32), ("in_h", ctypes.c_int32),
                ("in_w", ctypes.c_int32), ("out_c", ctypes.c_int32), ("ksize", ctypes.c_int32),
                ("stride", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("batch_normalize", ctypes.c_int32), ("act", ctypes.c_int32),
                ("slope", ctypes.c_float), ("bn_eps", ctypes.c_float),
                ("groups", ctypes.c_int32), ("dilation", ctypes.c_int32)]

    def _span(self) -> int:
        return max(1, self.dilation) * (self.ksize - 1) + 1

    @property
    def out_h(self) -> int:
        return (self.in_h + 2 * self.pad - self._span()) // self.stride + 1

    @property
    def out_w(self) -> int:
        return (self.in_w + 2 * self.pad - self._span()) // self.stride + 1


class BlockOpts(ctypes.Structure):
    """cbb_block_opts."""
    _fields_ = [("sums", ctypes.c_void_p), ("below_sums", ctypes.c_void_p),
                ("below_y", ctypes.c_void_p), ("below_x_norm", ctypes.c_void_p),
                ("below_act", ctypes.c_int32), ("below_slope", ctypes.c_float),
                ("below_apply_act", ctypes.c_int32)]


def conv_desc(batch, in_c, in_h, in_w, out_c, ksize, stride, pad, batch_normalize, act,
              slope=0.1, bn_eps=1e-5, groups=1, dilation=1) -> ConvDesc:
    a = ACT[act] if isinstance(act, str) else int(act)
    return ConvDesc(batch, in_c, in_h, in_w, out_c, ksize, stride, pad, int(batch_normalize), a,
                    slope, bn_eps, groups, dilation)


_P = ctypes.c_void_p
_i32, _i64, _f, _sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "cbb_abi_version": ([], _i32),
    "cbb_status_string": ([_i32], ctypes.c_char_p),
    "cbb_last_error": ([], ctypes.c_char_p),
    "cbb_conv_block_workspace_size": ([ctypes.POINTER(ConvDesc), ctypes.POINTER(_sz)], _i32),
    "cbb_conv_block_backward": ([ctypes.POINTER(ConvDesc)] + [_P] * 12 + [_i32, _P, _sz, _P], _i32),
    "cbb_conv_block_backward_noalloc": ([ctypes.POINTER(ConvDesc)] + [_P] * 12 + [_i32, _P], _i32),
    "cbb_conv_block_backward_ex": ([ctypes.POINTER(ConvDesc)] + [_P] * 12 +
                                   [_i32, ctypes.POINTER(BlockOpts), _P, _sz, _P], _i32),
    "cbb_conv_backward_data_ex": ([ctypes.POINTER(ConvDesc), _P, _P, _P, _i32,
                                   ctypes.POINTER(BlockOpts), _P, _sz, _P], _i32),
    "cbb_conv_fuses_below_sums": ([ctypes.POINTER(ConvDesc)], _i32),
    "cbb_conv_act_bn_backward": ([ctypes.POINTER(ConvDesc)] + [_P] * 8 + [_P, _sz, _P], _i32),
    "cbb_conv_backward_weights": ([ctypes.POINTER(ConvDesc), _P, _P, _P, _P, _sz, _P], _i32),
    "cbb_conv_backward_data": ([ctypes.POINTER(ConvDesc), _P, _P, _P, _i32, _P, _sz, _P], _i32),
    "cbb_conv_backward_weights_data": ([ctypes.POINTER(ConvDesc)] + [_P] * 5 + [_i32, _P, _sz, _P],
                                       _i32),
    "cbb_conv_fused_weights_data": ([ctypes.POINTER(ConvDesc)], _i32),
    "cbb_conv_dw_forms_dz": ([ctypes.POINTER(ConvDesc)], _i32),
    "cbb_conv_block_forward_workspace_size": ([ctypes.POINTER(ConvDesc), ctypes.POINTER(_sz)],
                                              _i32),
    "cbb_conv_block_forward": ([ctypes.POINTER(ConvDesc)] + [_P] * 9 + [_P, _sz, _P], _i32),
    "cbb_act_backward": ([_i32, _f, _P, _P, _P, _i64, _P], _i32),
    "cbb_bn_backward_workspace_size": ([_i32, _i32, _i64, ctypes.POINTER(_sz)], _i32),
    "cbb_bn_backward": ([_i32, _i32, _i64, _f] + [_P] * 7 + [_P, _sz, _P], _i32),
    "cbb_bn_backward_fixed": ([_i32, _i32, _i64, _f] + [_P] * 7 + [_P, _sz, _P], _i32),
    "cbb_fc_backward": ([_i32, _i32, _i32] + [_P] * 6 + [_i32, _P], _i32),
    "cbb_softmax_loss_backward": ([_i32, _i32, _P, _P, _f, _P, _P, _P], _i32),
    "cbb_fc_softmax_backward": ([_i32, _i32, _i32, _P, _P, _f] + [_P] * 7 + [_P], _i32),
    "cbb_shortcut_backward": ([_i64, _f, _f, _P, _P, _P, _P], _i32),
    "cbb_softmax_backward": ([_i32, _i32, _i64, _P, _P, _P, _P], _i32),
    "cbb_shortcut_backward_resize": ([_i32] * 7 + [_f, _f, _P, _P, _P, _P], _i32),
    "cbb_route_backward": ([_i32, _i32, ctypes.POINTER(_i64), _P, ctypes.POINTER(_P), _P], _i32),
    "cbb_upsample_backward": ([_i32] * 5 + [_P, _P, _P], _i32),
    "cbb_maxpool_backward": ([_i32] * 6 + [_P, _P, _P, _P], _i32),
    "cbb_get_device_error": ([_P, ctypes.POINTER(_i32)], _i32),
    "cbb_sgd_update": ([_i64, _i32, _f, _f, _f, _P, _P, _P], _i32),
    "cbb_set_launch_hook": ([_P, _P], _i32),
}
DEVERR_LABEL = 1
# void (*)(void* user, const char* kernel, void* stream)
LAUNCH_HOOK = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_char_p, ctypes.c_void_p)
EXPORTS = tuple(_SIGS)

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libcbb.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m cnn_backward_pass_amd.build` (hipcc, gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        text = (lib().cbb_status_string(rc) or b"").decode()
        raise CbbError(fn, rc, text)


def _ptr(t: torch.Tensor | None, dtype=torch.float32, name: str = "tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must live on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _sized(fn: str, **spec) -> None:
    """Check each named tensor against the element count (or shape) its call implies:
    a tensor too small for what the kernels read or write would be accessed out of
    bounds on the device.  spec maps name -> (tensor or None, expected numel or shape)."""
    for name, (t, want) in spec.items():
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{fn}: {name}: expected a torch.Tensor")
        if isinstance(want, tuple):
            if tuple(t.shape) != want:
                raise ValueError(f"{fn}: {name} has shape {tuple(t.shape)}, expected {want}")
        elif t.numel() != int(want):
            raise ValueError(f"{fn}: {name} has {t.numel()} elements, expected {int(want)}")


def _conv_sizes(fn: str, desc: "ConvDesc", **tensors) -> None:
    """Sizes of a conv block's tensors from its descriptor: x, dx [N,C,H,W]; y, x_norm,
    delta, dz [N,O,OH,OW]; w, dw [O,C/groups,k,k]; per-channel vectors [O]."""
    g = max(1, desc.groups)
    if desc.in_c % g or desc.out_c % g or desc.out_h < 1 or desc.out_w < 1:
        return  # the library rejects the descriptor itself with a status code
    xs = (desc.batch, desc.in_c, desc.in_h, desc.in_w)
    ys = (desc.batch, desc.out_c, desc.out_h, desc.out_w)
    ws = (desc.out_c, desc.in_c // g, desc.ksize, desc.ksize)
    kind = {"x": xs, "dx": xs, "y": ys, "x_norm": ys, "delta": ys, "dz": ys, "w": ws, "dw": ws}
    spec = {}
    for name, t in tensors.items():
        want = kind.get(name, desc.out_c)
        if isinstance(want, tuple) and t is not None and t.dim() != 4:
            want = int(torch.Size(want).numel())
        spec[name] = (t, want)
    _sized(fn, **spec)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def abi_version() -> int:
    return lib().cbb_abi_version()


def status_string(status: int) -> str:
    return (lib().cbb_status_string(status) or b"").decode()


def last_error() -> str:
    return (lib().cbb_last_error() or b"").decode()


def workspace(nbytes: int, device="cuda") -> torch.Tensor | None:
    """A device byte buffer usable as a cbb workspace (torch allocations are 256-byte aligned)."""
    if nbytes == 0:
        return None
    buf = torch.empty(int(nbytes), dtype=torch.uint8, device=device)
    assert buf.data_ptr() % WORKSPACE_ALIGN == 0
    return buf


def _ws(buf: torch.Tensor | None):
    if buf is None:
        return None, 0
    return _ptr(buf, torch.uint8, "workspace"), buf.numel()


# ----------------------------------------------------------------------------- entry points
def conv_block_workspace_size(desc: ConvDesc) -> int:
    n = ctypes.c_size_t(0)
    _check("cbb_conv_block_workspace_size",
           lib().cbb_conv_block_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def conv_block_backward(desc: ConvDesc, x, w, y, x_norm, var, gamma, delta, dz, dw, db, dgamma,
                        dx, dx_accumulate: bool = False, workspace=None, stream=None) -> None:
    _conv_sizes("conv_block_backward", desc, x=x, w=w, y=y, x_norm=x_norm, var=var, gamma=gamma,
                delta=delta, dz=dz, dw=dw, db=db, dgamma=dgamma, dx=dx)
    wsp, wsb = _ws(workspace)
    _check("cbb_conv_block_backward", lib().cbb_conv_block_backward(
        ctypes.byref(desc), _ptr(x, name="x"), _ptr(w, name="w"), _ptr(y, name="y"),
        _ptr(x_norm, name="x_norm"), _ptr(var, name="var"), _ptr(gamma, name="gamma"),
        _ptr(delta, name="delta"), _ptr(dz, name="dz"), _ptr(dw, name="dw"),
        _ptr(db, name="db"), _ptr(dgamma, name="dgamma"), _ptr(dx, name="dx"),
        int(dx_accumulate), wsp, wsb, _stream(stream)))


def _block_opts(fn: str, desc: ConvDesc, sums, below) -> BlockOpts:
    """cbb_block_opts from `sums` (float32 [2*O]) and `below` (dict: "sums" [2*C] out,
    "y" (None under linear) and "x_norm" [N,C,H,W] of the block below, "act", "slope",
    and "apply_act": True to leave g = dx * act'(y) in dx)."""
    xs = (desc.batch, desc.in_c, desc.in_h, desc.in_w)
    opts = BlockOpts()
    if sums is not None:
        _sized(fn, sums=(sums, 2 * desc.out_c))
        opts.sums = _ptr(sums, name="sums").value
    if below is not None:
        by, bxn = below.get("y"), below.get("x_norm")
        shape = lambda t: xs if t is None or t.dim() == 4 else int(torch.Size(xs).numel())
        _sized(fn, below_sums=(below["sums"], 2 * desc.in_c), below_y=(by, shape(by)),
               below_x_norm=(bxn, shape(bxn)))
        opts.below_sums = _ptr(below["sums"], name="below.sums").value
        opts.below_y = None if by is None else _ptr(by, name="below.y").value
        opts.below_x_norm = None if bxn is None else _ptr(bxn, name="below.x_norm").value
        act = below["act"]
        opts.below_act = ACT[act] if isinstance(act, str) else int(act)
        opts.below_slope = float(below.get("slope", 0.1))
        opts.below_apply_act = int(bool(below.get("apply_act", False)))
    return opts


def conv_block_backward_ex(desc: ConvDesc, x, w, y, x_norm, var, gamma, delta, dz, dw, db, dgamma,
                           dx, dx_accumulate: bool = False, sums=None, below=None, workspace=None,
                           stream=None) -> None:
    """conv_block_backward with this block's act/BN sums given (`sums`: (sum g,
    sum g*x_norm) per channel from the call of the block above) and/or the act/BN sums of
    the block below produced on the way (`below`, see _block_opts)."""
    _conv_sizes("conv_block_backward_ex", desc, x=x, w=w, y=y, x_norm=x_norm, var=var,
                gamma=gamma, delta=delta, dz=dz, dw=dw, db=db, dgamma=dgamma, dx=dx)
    opts = _block_opts("conv_block_backward_ex", desc, sums, below)
    wsp, wsb = _ws(workspace)
    _check("cbb_conv_block_backward_ex", lib().cbb_conv_block_backward_ex(
        ctypes.byref(desc), _ptr(x, name="x"), _ptr(w, name="w"), _ptr(y, name="y"),
        _ptr(x_norm, name="x_norm"), _ptr(var, name="var"), _ptr(gamma, name="gamma"),
        _ptr(delta, name="delta"), _ptr(dz, name="dz"), _ptr(dw, name="dw"),
        _ptr(db, name="db"), _ptr(dgamma, name="dgamma"), _ptr(dx, name="dx"),
        int(dx_accumulate), ctypes.byref(opts), wsp, wsb, _stream(stream)))


def conv_backward_data_ex(desc: ConvDesc, w, dz, dx, dx_accumulate: bool = False, below=None,
                          workspace=None, stream=None) -> None:
    """conv_backward_data producing the act/BN sums of the block below on the way."""
    _conv_sizes("conv_backward_data_ex", desc, w=w, dz=dz, dx=dx)
    opts = _block_opts("conv_backward_data_ex", desc, None, below)
    wsp, wsb = _ws(workspace)
    _check("cbb_conv_backward_data_ex", lib().cbb_conv_backward_data_ex(
        ctypes.byref(desc), _ptr(w, name="w"), _ptr(dz, name="dz"), _ptr(dx, name="dx"),
        int(dx_accumulate), ctypes.byref(opts), wsp, wsb, _stream(stream)))


def conv_fuses_below_sums(desc: ConvDesc) -> bool:
    rc = lib().cbb_conv_fuses_below_sums(ctypes.byref(desc))
    if rc < 0:
        _check("cbb_conv_fuses_below_sums", rc)
    return rc == 1


def conv_block_backward_noalloc(desc: ConvDesc, x, w, y, x_norm, var, gamma, delta, dz, dw, db,
                                dgamma, dx, dx_accumulate: bool = False, stream=None) -> None:
    """conv_block_backward with the library's static scratch buffer (no workspace)."""
    _conv_sizes("conv_block_backward_noalloc", desc, x=x, w=w, y=y, x_norm=x_norm, var=var,
                gamma=gamma, delta=delta, dz=dz, dw=dw, db=db, dgamma=dgamma, dx=dx)
    _check("cbb_conv_block_backward_noalloc", lib().cbb_conv_block_backward_noalloc(
        ctypes.byref(desc), _ptr(x, name="x"), _ptr(w, name="w"), _ptr(y, name="y"),
        _ptr(x_norm, name="x_norm"), _ptr(var, name="var"), _ptr(gamma, name="gamma"),
        _ptr(delta, name="delta"), _ptr(dz, name="dz"), _ptr(dw, name="dw"),
        _ptr(db, name="db"), _ptr(dgamma, name="dgamma"), _ptr(dx, name="dx"),
        int(dx_accumulate), _stream(stream)))


def conv_block_forward_workspace_size(desc: ConvDesc) -> int:
    b = ctypes.c_size_t(0)
    _check("cbb_conv_block_forward_workspace_size",
           lib().cbb_conv_block_forward_workspace_size(ctypes.byref(desc), ctypes.byref(b)))
    return b.value


def conv_block_forward(desc: ConvDesc, x, w, bias, gamma, beta, mean, var, x_norm, y,
                       workspace=None, stream=None) -> None:
    _conv_sizes("conv_block_forward", desc, x=x, w=w, bias=bias, gamma=gamma, beta=beta,
                mean=mean, var=var, x_norm=x_norm, y=y)
    wsp, wsb = _ws(workspace)
    _check("cbb_conv_block_forward", lib().cbb_conv_block_forward(
        ctypes.byref(desc), _ptr(x, name="x"), _ptr(w, name="w"), _ptr(bias, name="bias"),
        _ptr(gamma, name="gamma"), _ptr(beta, name="beta"), _ptr(mean, name="mean"),
        _ptr(var, name="var"), _ptr(x_norm, name="x_norm"), _ptr(y, name="y"), wsp, wsb,
        _stream(stream)))


def conv_act_bn_backward(desc: ConvDesc, y, x_norm, var, gamma, delta, dz, db, dgamma,
                         workspace=None, stream=None) -> None:
    _conv_sizes("conv_act_bn_backward", desc, y=y, x_norm=x_norm, var=var, gamma=gamma,
                delta=delta, dz=dz, db=db, dgamma=dgamma)
    wsp, wsb = _ws(workspace)
    _check("cbb_conv_act_bn_backward", lib().cbb_conv_act_bn_backward(
        ctypes.byref(desc), _ptr(y, name="y"), _ptr(x_norm, name="x_norm"), _ptr(var, name="var"),
        _ptr(gamma, name="gamma"), _ptr(delta, name="delta"), _ptr(dz, name="dz"),
        _ptr(db, name="db"), _ptr(dgamma, name="dgamma"), wsp, wsb, _stream(stream)))


def conv_backward_weights(desc: ConvDesc, x, dz, dw, workspace=None, stream=None) -> None:
    _conv_sizes("conv_backward_weights", desc, x=x, dz=dz, dw=dw)
    wsp, wsb = _ws(workspace)
    _check("cbb_conv_backward_weights", lib().cbb_conv_backward_weights(
        ctypes.byref(desc), _ptr(x, name="x"), _ptr(dz, name="dz"), _ptr(dw, name="dw"), wsp, wsb,
        _stream(stream)))


def conv_backward_data(desc: ConvDesc, w, dz, dx, dx_accumulate: bool = False, workspace=None,
                       stream=None) -> None:
    _conv_sizes("conv_backward_data", desc, w=w, dz=dz, dx=dx)
    wsp, wsb = _ws(workspace)
    _check("cbb_conv_backward_data", lib().cbb_conv_backward_data(
        ctypes.byref(desc), _ptr(w, name="w"), _ptr(dz, name="dz"), _ptr(dx, name="dx"),
        int(dx_accumulate), wsp, wsb, _stream(stream)))


def conv_backward_weights_data(desc: ConvDesc, x, w, dz, dw, dx=None, dx_accumulate: bool = False,
                               workspace=None, stream=None) -> None:
    _conv_sizes("conv_backward_weights_data", desc, x=x, w=w, dz=dz, dw=dw, dx=dx)
    wsp, wsb = _ws(workspace)
    _check("cbb_conv_backward_weights_data", lib().cbb_conv_backward_weights_data(
        ctypes.byref(desc), _ptr(x, name="x"), _ptr(w, name="w"), _ptr(dz, name="dz"),
        _ptr(dw, name="dw"), _ptr(dx, name="dx"), int(dx_accumulate), wsp, wsb, _stream(stream)))


def conv_fused_weights_data(desc: ConvDesc) -> bool:
    rc = lib().cbb_conv_fused_weights_data(ctypes.byref(desc))
    if rc < 0:
        _check("cbb_conv_fused_weights_data", rc)
    return rc == 1


def conv_dw_forms_dz(desc: ConvDesc) -> bool:
    rc = lib().cbb_conv_dw_forms_dz(ctypes.byref(desc))
    if rc < 0:
        _check("cbb_conv_dw_forms_dz", rc)
    return rc == 1


def act_backward(act, slope: float, y, delta, g, stream=None) -> None:
    a = ACT[act] if isinstance(act, str) else int(act)
    if not (y.numel() == delta.numel() == g.numel()):
        raise ValueError("act_backward: y, delta, g must have the same number of elements")
    _check("cbb_act_backward", lib().cbb_act_backward(
        a, slope, _ptr(y, name="y"), _ptr(delta, name="delta"), _ptr(g, name="g"), delta.numel(),
        _stream(stream)))


def bn_backward_workspace_size(n: int, c: int, hw: int) -> int:
    b = ctypes.c_size_t(0)
    _check("cbb_bn_backward_workspace_size",
           lib().cbb_bn_backward_workspace_size(n, c, hw, ctypes.byref(b)))
    return b.value


def bn_backward(g, x_norm, var, gamma, dz, dgamma, dbeta, eps: float = 1e-5, workspace=None,
                stream=None) -> None:
    n, c = g.shape[0], g.shape[1]
    hw = g.numel() // (n * c)
    _sized("bn_backward", x_norm=(x_norm, g.numel()), dz=(dz, g.numel()), var=(var, c),
           gamma=(gamma, c), dgamma=(dgamma, c), dbeta=(dbeta, c))
    wsp, wsb = _ws(workspace)
    _check("cbb_bn_backward", lib().cbb_bn_backward(
        n, c, hw, eps, _ptr(g, name="g"), _ptr(x_norm, name="x_norm"), _ptr(var, name="var"),
        _ptr(gamma, name="gamma"), _ptr(dz, name="dz"), _ptr(dgamma, name="dgamma"),
        _ptr(dbeta, name="dbeta"), wsp, wsb, _stream(stream)))


def bn_backward_fixed(g, x_norm, var, gamma, dz, dgamma, dbeta, eps: float = 1e-5, workspace=None,
                stream=None) -> None:
    n, c = g.shape[0], g.shape[1]
    hw = g.numel() // (n * c)
    _sized("bn_backward_fixed", x_norm=(x_norm, g.numel()), dz=(dz, g.numel()), var=(var, c),
           gamma=(gamma, c), dgamma=(dgamma, c), dbeta=(dbeta, c))
    wsp, wsb = _ws(workspace)
    _check("cbb_bn_backward_fixed", lib().cbb_bn_backward_fixed(
        n, c, hw, eps, _ptr(g, name="g"), _ptr(x_norm, name="x_norm"), _ptr(var, name="var"),
        _ptr(gamma, name="gamma"), _ptr(dz, name="dz"), _ptr(dgamma, name="dgamma"),
        _ptr(dbeta, name="dbeta"), wsp, wsb, _stream(stream)))


def fc_backward(x, w, delta, dw, db, dx, dx_accumulate: bool = False, stream=None) -> None:
    batch, in_dim = x.shape
    out_dim = w.shape[0]
    _sized("fc_backward", w=(w, (out_dim, in_dim)), delta=(delta, batch * out_dim),
           dw=(dw, out_dim * in_dim), db=(db, out_dim), dx=(dx, batch * in_dim))
    _check("cbb_fc_backward", lib().cbb_fc_backward(
        batch, in_dim, out_dim, _ptr(x, name="x"), _ptr(w, name="w"), _ptr(delta, name="delta"),
        _ptr(dw, name="dw"), _ptr(db, name="db"), _ptr(dx, name="dx"), int(dx_accumulate),
        _stream(stream)))


def softmax_loss_backward(prob, labels, dlogits, loss_weight: float = 1.0, bad_labels=None,
                          stream=None) -> None:
    batch, classes = prob.shape
    _sized("softmax_loss_backward", labels=(labels, batch), dlogits=(dlogits, batch * classes),
           bad_labels=(bad_labels, 1))
    _check("cbb_softmax_loss_backward", lib().cbb_softmax_loss_backward(
        batch, classes, _ptr(prob, name="prob"), _ptr(labels, torch.int32, "labels"), loss_weight,
        _ptr(dlogits, name="dlogits"), _ptr(bad_labels, torch.int32, "bad_labels"),
        _stream(stream)))


def fc_softmax_backward(prob, labels, x, w, dlogits, dw, db, dx, loss_weight: float = 1.0,
                        bad_labels=None, stream=None) -> None:
    batch, classes = prob.shape
    in_dim = x.shape[1]
    _sized("fc_softmax_backward", labels=(labels, batch), x=(x, batch * in_dim),
           w=(w, classes * in_dim), dlogits=(dlogits, batch * classes),
           dw=(dw, classes * in_dim), db=(db, classes), dx=(dx, batch * in_dim),
           bad_labels=(bad_labels, 1))
    _check("cbb_fc_softmax_backward", lib().cbb_fc_softmax_backward(
        batch, in_dim, classes, _ptr(prob, name="prob"), _ptr(labels, torch.int32, "labels"),
        loss_weight, _ptr(x, name="x"), _ptr(w, name="w"), _ptr(dlogits, name="dlogits"),
        _ptr(dw, name="dw"), _ptr(db, name="db"), _ptr(dx, name="dx"),
        _ptr(bad_labels, torch.int32, "bad_labels"), _stream(stream)))


def softmax_backward(y, dy, dx, stream=None) -> None:
    """Softmax backward along axis 1 of y ([outer, channels, ...])."""
    outer, channels = y.shape[0], y.shape[1]
    inner = y.numel() // (outer * channels)
    if tuple(dy.shape) != tuple(y.shape) or tuple(dx.shape) != tuple(y.shape):
        raise ValueError("y, dy and dx must have one shape")
    _check("cbb_softmax_backward", lib().cbb_softmax_backward(
        outer, channels, inner, _ptr(y, name="y"), _ptr(dy, name="dy"), _ptr(dx, name="dx"),
        _stream(stream)))


def shortcut_backward(delta, d_main, d_from, alpha: float = 1.0, beta: float = 1.0,
                      stream=None) -> None:
    if not (delta.numel() == d_main.numel() == d_from.numel()):
        raise ValueError("shortcut_backward: equal shapes only")
    _check("cbb_shortcut_backward", lib().cbb_shortcut_backward(
        delta.numel(), alpha, beta, _ptr(delta, name="delta"), _ptr(d_main, name="d_main"),
        _ptr(d_from, name="d_from"), _stream(stream)))


def shortcut_backward_resize(delta, d_main, d_from, alpha: float = 1.0, beta: float = 1.0,
                             stream=None) -> None:
    """delta [b, c1, h1, w1], d_from [b, c2, h2, w2], d_main like delta or None."""
    b, c1, h1, w1 = delta.shape
    b2, c2, h2, w2 = d_from.shape
    if b2 != b:
        raise ValueError("delta and d_from differ in batch")
    if d_main is not None and tuple(d_main.shape) != tuple(delta.shape):
        raise ValueError("d_main must have delta's shape")
    _check("cbb_shortcut_backward_resize", lib().cbb_shortcut_backward_resize(
        b, w1, h1, c1, w2, h2, c2, alpha, beta, _ptr(delta, name="delta"),
        None if d_main is None else _ptr(d_main, name="d_main"), _ptr(d_from, name="d_from"),
        _stream(stream)))


def route_backward(delta, d_ins: Sequence[torch.Tensor], stream=None) -> None:
    batch = delta.shape[0]
    if any(t.numel() % batch for t in d_ins):
        raise ValueError("route_backward: every input must hold `batch` images")
    _sized("route_backward", delta=(delta, sum(t.numel() for t in d_ins)))
    sizes = (ctypes.c_int64 * len(d_ins))(*[t.numel() // batch for t in d_ins])
    ptrs = (ctypes.c_void_p * len(d_ins))(*[_ptr(t, name="d_in").value for t in d_ins])
    _check("cbb_route_backward", lib().cbb_route_backward(
        batch, len(d_ins), sizes, _ptr(delta, name="delta"), ptrs, _stream(stream)))


def upsample_backward(delta, dx, scale: int = 2, stream=None) -> None:
    n, c, h, w = dx.shape
    if tuple(delta.shape) != (n, c, h * scale, w * scale):
        raise ValueError("upsample_backward: delta must be dx's shape times scale")
    _check("cbb_upsample_backward", lib().cbb_upsample_backward(
        n, c, h, w, scale, _ptr(delta, name="delta"), _ptr(dx, name="dx"), _stream(stream)))


def maxpool_backward(idx, delta, dx, ksize: int = 2, stride: int = 2, stream=None) -> None:
    n, c, ih, iw = dx.shape
    oh, ow = (ih - ksize) // stride + 1, (iw - ksize) // stride + 1
    if tuple(delta.shape) != (n, c, oh, ow) or tuple(idx.shape) != (n, c, oh, ow):
        raise ValueError("maxpool_backward: delta/idx shape does not match the pooled shape")
    _check("cbb_maxpool_backward", lib().cbb_maxpool_backward(
        n, c, ih, iw, ksize, stride, _ptr(idx, torch.int32, "idx"), _ptr(delta, name="delta"),
        _ptr(dx, name="dx"), _stream(stream)))


def get_device_error(stream=None) -> int:
    """Wait for the stream, then read and clear the GPU's error word (CBB_DEVERR_* bits
    raised by kernels since the previous read; 0 when none)."""
    code = ctypes.c_int(0)
    _check("cbb_get_device_error", lib().cbb_get_device_error(_stream(stream), ctypes.byref(code)))
    return code.value


_hook_ref = None  # keeps the ctypes callback alive while the library holds it


def set_launch_hook(fn) -> None:
    """fn(kernel_name: str, stream_handle: int) after each kernel the library enqueues;
    None removes the hook.  Process-wide (tracing and per-kernel event timing)."""
    global _hook_ref
    if fn is None:
        _check("cbb_set_launch_hook", lib().cbb_set_launch_hook(None, None))
        _hook_ref = None
        return
    cb = LAUNCH_HOOK(lambda user, name, st: fn(name.decode(), st or 0))
    _check("cbb_set_launch_hook", lib().cbb_set_launch_hook(ctypes.cast(cb, ctypes.c_void_p), None))
    _hook_ref = cb


def sgd_update(w, dw, batch: int, learning_rate: float, momentum: float = 0.0,
               decay: float = 0.0, stream=None) -> None:
    """Parameter update in place: u = dw + decay*batch*w; w -= lr/batch*u; dw = momentum*u."""
    _sized("sgd_update", dw=(dw, w.numel()))
    _check("cbb_sgd_update", lib().cbb_sgd_update(
        w.numel(), batch, learning_rate, momentum, decay, _ptr(w, name="w"), _ptr(dw, name="dw"),
        _stream(stream)))
