"""The C ABI on a host without a GPU: the library loads, exports every symbol
include/cbb.h declares, and rejects bad arguments with status codes before any
HIP call.  No call here passes arguments that would reach a kernel launch."""
import ctypes
import os
import re

import pytest

from cnn_backward_pass_amd import cbb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cbb.h")

pytestmark = pytest.mark.skipif(not os.path.exists(cbb.LIB_PATH),
                                reason="libcbb.so not built (run __graft_entry__.build())")

BOGUS = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(cbb_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert len(names) >= 14
    lib = cbb.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(cbb.EXPORTS)


def test_version_and_status_strings():
    assert cbb.abi_version() == 2
    for code in (0, -1, -2, -3, -4):
        assert cbb.status_string(code)
    assert cbb.status_string(123) == "unknown status"


def _desc(**kw):
    base = dict(batch=2, in_c=3, in_h=8, in_w=8, out_c=4, ksize=3, stride=1, pad=1,
                batch_normalize=1, act="leaky")
    base.update(kw)
    return cbb.conv_desc(**base)


def ws_size(desc):
    n = ctypes.c_size_t(0)
    rc = cbb.lib().cbb_conv_block_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    return rc, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), -1), (dict(in_c=0), -1), (dict(out_c=-2), -1), (dict(ksize=0), -1),
    (dict(stride=0), -1), (dict(pad=-1), -1), (dict(act=14), -1), (dict(act=-1), -1),
    (dict(batch_normalize=3), -1), (dict(batch_normalize=-1), -1),
    (dict(groups=3), -1), (dict(groups=-1), -1), (dict(dilation=-2), -1),
    (dict(dilation=17, pad=0), -3), (dict(ksize=3, pad=3, dilation=1), -3),
    (dict(in_h=4, in_w=4, ksize=3, pad=0, dilation=3), -2),
    (dict(ksize=9, pad=4), -3), (dict(stride=5), -3), (dict(ksize=3, pad=3), -3),
    (dict(in_h=1, in_w=1, ksize=5, pad=1), -2),
    (dict(batch=4096, in_c=512, in_h=1024, in_w=1024), -3),
])
def test_conv_desc_validation(kw, code):
    assert ws_size(_desc(**kw))[0] == code


def test_workspace_size_query_is_host_only():
    rc, n = ws_size(_desc())
    assert rc == 0 and n > 0 and n % 256 == 0
    # larger problems never need less scratch
    rc2, n2 = ws_size(_desc(batch=16, in_h=64, in_w=64))
    assert rc2 == 0 and n2 >= n


def _call_conv(desc, **ptrs):
    names = ["x", "w", "y", "x_norm", "var", "gamma", "delta", "dz", "dw", "db", "dgamma", "dx"]
    args = [ptrs.get(k, BOGUS) for k in names]
    ws = ptrs.get("ws", BOGUS)
    wsb = ptrs.get("wsb", 1 << 30)
    return cbb.lib().cbb_conv_block_backward(ctypes.byref(desc), *args, ptrs.get("acc", 0), ws,
                                             wsb, None)


@pytest.mark.parametrize("missing", ["x", "w", "delta", "dw", "db", "y", "x_norm", "var", "gamma",
                                     "dgamma", "dz"])
def test_conv_null_required_pointer(missing):
    # 5 input channels: not a fused first layer, where dz = NULL is a valid request
    assert _call_conv(_desc(in_c=5), **{missing: None}) == -1


def test_dw_forms_dz_query():
    """Host-only query: which layers' weight-gradient kernel forms dz itself."""
    q = lambda d: cbb.lib().cbb_conv_dw_forms_dz(ctypes.byref(d))
    assert q(_desc(in_c=32, in_h=20, in_w=104, out_c=64, stride=2)) == 1
    assert q(_desc(in_c=32, in_h=11, in_w=52, out_c=128)) == 1
    assert q(_desc(in_c=64, in_h=11, in_w=52, out_c=128)) == 0      # more than one input block
    assert q(_desc(in_c=32, in_h=20, in_w=104, out_c=64, stride=2, batch_normalize=2)) == 0
    assert q(_desc(in_c=32, in_h=20, in_w=104, out_c=64, stride=2, batch_normalize=0)) == 0
    assert q(_desc(in_c=32, in_h=26, in_w=26, out_c=64)) == 0       # width not a multiple of 4
    assert q(_desc(in_c=48, in_h=20, in_w=104, out_c=64)) == 0      # input channels
    assert q(_desc(in_c=32, in_h=20, in_w=104, out_c=96)) == 0      # output channels
    assert q(_desc(ksize=3, in_c=0)) < 0


def test_conv_formed_dz_rules():
    """dz = NULL asks the fused first-layer kernel to form dz itself: only valid on
    such a layer, with dx given and 16-byte aligned saved tensors."""
    d = _desc()
    assert cbb.lib().cbb_conv_fused_weights_data(ctypes.byref(d)) == 1
    assert _call_conv(d, dz=None, dx=None) == -1
    misaligned = ctypes.c_void_p(0x1004)
    for name in ("x", "delta", "y", "x_norm"):
        assert _call_conv(d, dz=None, **{name: misaligned}) == -1
    for kw in (dict(in_c=4), dict(ksize=5, pad=2), dict(stride=2), dict(in_w=10),
               dict(out_c=33)):
        dn = _desc(**kw)
        assert cbb.lib().cbb_conv_fused_weights_data(ctypes.byref(dn)) == 0
        assert _call_conv(dn, dz=None) == -1


def test_conv_pointer_rules_without_bn():
    d = _desc(batch_normalize=0)
    # BN tensors must be NULL when there is no BN
    assert _call_conv(d, dgamma=BOGUS, x_norm=None, var=None, gamma=None) == -1
    # linear without BN: y may be NULL but the other pointer rules still hold
    dl = _desc(batch_normalize=0, act="linear")
    assert _call_conv(dl, y=None, x_norm=None, var=None, gamma=None, dgamma=None, dz=None,
                      x=None) == -1


def test_conv_workspace_and_flags():
    d = _desc()
    _, need = ws_size(d)
    assert _call_conv(d, wsb=need - 1) == -4
    assert _call_conv(d, ws=None) == -4
    assert _call_conv(d, ws=ctypes.c_void_p(0x1004)) == -4     # not 256-byte aligned
    assert _call_conv(d, acc=2) == -1


def test_weights_data_entry_points_validate():
    L = cbb.lib()
    d = _desc()
    _, need = ws_size(d)
    call = lambda *a: L.cbb_conv_backward_weights_data(ctypes.byref(d), *a, None)
    for i in range(4):  # x, w, dz, dw are required
        args = [BOGUS] * 5
        args[i] = None
        assert call(*args, 0, BOGUS, need) == -1
    assert call(*[BOGUS] * 5, 2, BOGUS, need) == -1            # dx_accumulate not 0/1
    assert call(*[BOGUS] * 5, 0, BOGUS, need - 1) == -4        # workspace too small
    assert call(*[BOGUS] * 5, 0, ctypes.c_void_p(0x1004), need) == -4
    # which descriptors take the fused kernel (a host-side query)
    fused = lambda **kw: L.cbb_conv_fused_weights_data(ctypes.byref(_desc(**kw)))
    assert fused() == 1 and fused(out_c=32) == 1 and fused(in_c=1) == 1
    assert fused(out_c=33) == 0 and fused(in_c=4) == 0 and fused(stride=2) == 0
    assert fused(ksize=5, pad=2) == 0 and fused(pad=0) == 0 and fused(in_w=9) == 0
    assert fused(batch=0) == -1
    assert L.cbb_conv_fused_weights_data(None) == -1


def test_other_entry_points_validate():
    L = cbb.lib()
    sz = ctypes.c_size_t(0)
    assert L.cbb_act_backward(14, 0.1, BOGUS, BOGUS, BOGUS, 10, None) == -1
    assert L.cbb_act_backward(-1, 0.1, BOGUS, BOGUS, BOGUS, 10, None) == -1
    assert L.cbb_act_backward(1, 0.1, None, BOGUS, BOGUS, 10, None) == -1
    assert L.cbb_act_backward(1, 0.1, BOGUS, BOGUS, BOGUS, -1, None) == -1
    assert L.cbb_act_backward(1, 0.1, BOGUS, BOGUS, BOGUS, 0, None) == 0      # empty: no launch
    assert L.cbb_bn_backward_workspace_size(0, 4, 16, ctypes.byref(sz)) == -1
    assert L.cbb_bn_backward_workspace_size(2, 4, 16, ctypes.byref(sz)) == 0 and sz.value > 0
    assert L.cbb_bn_backward(2, 4, 16, 1e-5, *[BOGUS] * 7, BOGUS, 0, None) == -4
    assert L.cbb_bn_backward(2, 4, 16, 0.0, *[BOGUS] * 7, BOGUS, 1 << 20, None) == -1
    assert L.cbb_bn_backward_fixed(2, 4, 16, 1e-5, *[BOGUS] * 7, BOGUS, 0, None) == -4
    assert L.cbb_bn_backward_fixed(2, 4, 16, 0.0, *[BOGUS] * 7, BOGUS, 1 << 20, None) == -1
    assert L.cbb_bn_backward_fixed(2, 4, 16, 1e-5, *[BOGUS] * 6, None, BOGUS, 1 << 20, None) == -1
    assert L.cbb_fc_backward(0, 8, 8, *[BOGUS] * 6, 0, None) == -1
    assert L.cbb_fc_backward(4, 8, 8, None, *[BOGUS] * 5, 0, None) == -1
    assert L.cbb_softmax_loss_backward(4, 0, BOGUS, BOGUS, 1.0, BOGUS, None, None) == -1
    assert L.cbb_fc_softmax_backward(4, 8, 10, BOGUS, None, 1.0, *[BOGUS] * 6, None, None) == -1
    assert L.cbb_shortcut_backward(16, 1.0, 1.0, BOGUS, BOGUS, BOGUS, None) == -1  # aliasing
    X = ctypes.c_void_p(0x3000)
    d = _desc()                       # BN, leaky
    F = L.cbb_conv_block_forward
    Y, XN = ctypes.c_void_p(0x4000), ctypes.c_void_p(0x5000)
    assert F(ctypes.byref(d), BOGUS, BOGUS, None, None, BOGUS, BOGUS, BOGUS, XN, Y, BOGUS,
             1 << 30, None) == -1                                   # BN without gamma
    assert F(ctypes.byref(d), BOGUS, BOGUS, BOGUS, BOGUS, BOGUS, BOGUS, BOGUS, XN, Y, BOGUS,
             1 << 30, None) == -1                                   # bias with BN
    assert F(ctypes.byref(d), BOGUS, BOGUS, None, BOGUS, BOGUS, BOGUS, BOGUS, Y, Y, BOGUS,
             1 << 30, None) == -1                                   # x_norm aliases y
    assert F(ctypes.byref(d), BOGUS, BOGUS, None, BOGUS, BOGUS, BOGUS, BOGUS, XN, Y, BOGUS,
             0, None) == -4                                         # workspace too small
    dl = _desc(batch_normalize=0, act="linear")
    assert F(ctypes.byref(dl), BOGUS, BOGUS, None, BOGUS, None, None, None, None, Y, BOGUS,
             1 << 30, None) == -1                                   # gamma without BN
    assert L.cbb_softmax_backward(0, 10, 1, BOGUS, X, X, None) == -1
    assert L.cbb_softmax_backward(4, 10, 1, BOGUS, X, BOGUS, None) == -1       # dx aliases y
    assert L.cbb_softmax_backward(4, 10, 0, BOGUS, X, X, None) == -1
    assert L.cbb_shortcut_backward_resize(2, 8, 8, 4, 4, 8, 4, 1.0, 1.0, BOGUS, X, BOGUS,
                                          None) == -1                  # d_from aliases delta
    assert L.cbb_shortcut_backward_resize(2, 8, 8, 4, 4, 6, 4, 1.0, 1.0, BOGUS, None, X,
                                          None) == -2                  # aspect differs
    assert L.cbb_shortcut_backward_resize(2, 4, 8, 4, 8, 8, 4, 1.0, 1.0, BOGUS, None, X,
                                          None) == -2
    assert L.cbb_shortcut_backward_resize(0, 8, 8, 4, 4, 4, 4, 1.0, 1.0, BOGUS, None, X,
                                          None) == -1
    assert L.cbb_shortcut_backward(0, 1.0, 1.0, BOGUS, ctypes.c_void_p(0x2000),
                                   ctypes.c_void_p(0x3000), None) == 0
    sizes = (ctypes.c_int64 * 2)(10, 0)
    ptrs = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    assert L.cbb_route_backward(2, 2, sizes, BOGUS, ptrs, None) == -1
    assert L.cbb_route_backward(2, 9, sizes, BOGUS, ptrs, None) == -1
    assert L.cbb_upsample_backward(2, 3, 4, 4, 9, BOGUS, BOGUS, None) == -3
    assert L.cbb_upsample_backward(2, 3, 0, 4, 2, BOGUS, BOGUS, None) == -1
    assert L.cbb_maxpool_backward(2, 3, 4, 4, 5, 2, BOGUS, BOGUS, BOGUS, None) == -2
    assert L.cbb_maxpool_backward(2, 3, 4, 4, 2, 0, BOGUS, BOGUS, BOGUS, None) == -1


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    t = torch.zeros(4)
    with pytest.raises(ValueError):
        cbb.act_backward("leaky", 0.1, t, t, t)


def test_device_error_and_hook_validate():
    """cbb_get_device_error rejects a NULL result pointer before touching the GPU; the
    launch hook is set and removed on the host."""
    L = cbb.lib()
    assert L.cbb_get_device_error(None, None) == -1
    calls = []
    cbb.set_launch_hook(lambda name, st: calls.append(name))
    cbb.set_launch_hook(None)
    assert calls == []          # nothing was launched
    assert cbb.DEVERR_LABEL == 1


def test_binding_checks_sizes_against_the_descriptor():
    """The binding compares every tensor with the sizes its call implies before any
    pointer reaches the library: an undersized tensor would be read or written out of
    bounds by the kernels."""
    torch = pytest.importorskip("torch")
    d = cbb.conv_desc(2, 3, 8, 8, 4, 3, 1, 1, 1, "leaky")
    z = lambda *s: torch.zeros(*s)
    ok = dict(x=z(2, 3, 8, 8), w=z(4, 3, 3, 3), y=z(2, 4, 8, 8), x_norm=z(2, 4, 8, 8),
              var=z(4), gamma=z(4), delta=z(2, 4, 8, 8), dz=z(2, 4, 8, 8), dw=z(4, 3, 3, 3),
              db=z(4), dgamma=z(4), dx=z(2, 3, 8, 8))
    for name, bad in (("dx", z(2, 3, 8, 7)), ("dx", z(2 * 3 * 8 * 8 - 1)), ("delta", z(1, 4, 8, 8)),
                      ("w", z(4, 3, 3, 2)), ("var", z(3)), ("dgamma", z(5)), ("x", z(2, 3, 8))):
        kw = dict(ok, **{name: bad})
        with pytest.raises(ValueError, match=name):
            cbb.conv_block_backward(d, **kw)
    with pytest.raises(ValueError, match="dw"):
        cbb.conv_backward_weights(d, ok["x"], ok["dz"], z(4, 3, 3, 3 - 1))
    with pytest.raises(ValueError, match="dx"):
        cbb.conv_backward_data(d, ok["w"], ok["dz"], z(2, 3, 4, 8))
    with pytest.raises(ValueError, match="y"):
        cbb.conv_block_forward(d, ok["x"], ok["w"], None, z(4), z(4), z(4), z(4), z(2, 4, 8, 8),
                               z(2, 4, 8, 9))
    # inner product, batch norm, softmax loss, route
    with pytest.raises(ValueError, match="dw"):
        cbb.fc_backward(z(4, 8), z(5, 8), z(4, 5), z(5, 7), z(5), z(4, 8))
    with pytest.raises(ValueError, match="dx"):
        cbb.fc_backward(z(4, 8), z(5, 8), z(4, 5), z(5, 8), z(5), z(4, 7))
    with pytest.raises(ValueError, match="dz"):
        cbb.bn_backward(z(2, 4, 16), z(2, 4, 16), z(4), z(4), z(2, 4, 15), z(4), z(4))
    with pytest.raises(ValueError, match="gamma"):
        cbb.bn_backward_fixed(z(2, 4, 16), z(2, 4, 16), z(4), z(3), z(2, 4, 16), z(4), z(4))
    with pytest.raises(ValueError, match="labels"):
        cbb.softmax_loss_backward(z(4, 10), torch.zeros(3, dtype=torch.int32), z(4, 10))
    with pytest.raises(ValueError, match="dlogits"):
        cbb.fc_softmax_backward(z(4, 10), torch.zeros(4, dtype=torch.int32), z(4, 8), z(10, 8),
                                z(4, 9), z(10, 8), z(10), None)
    with pytest.raises(ValueError, match="delta"):
        cbb.route_backward(z(2, 7, 4, 4), [z(2, 4, 4, 4), z(2, 2, 4, 4)])


def test_noalloc_entry_point_validates_on_the_host():
    """The no-allocation variant rejects, before any HIP call, a layer whose scratch
    would not fit its static buffer (CBB_ESCRATCH) and every argument error of the
    workspace entry point."""
    L = cbb.lib()
    big = _desc(batch=16, in_c=256, in_h=26, in_w=26, out_c=512)
    _, need = ws_size(big)
    assert need > cbb.NOALLOC_SCRATCH_BYTES
    names = ["x", "w", "y", "x_norm", "var", "gamma", "delta", "dz", "dw", "db", "dgamma", "dx"]
    call = lambda d, **kw: L.cbb_conv_block_backward_noalloc(
        ctypes.byref(d), *[kw.get(k, BOGUS) for k in names], kw.get("acc", 0), None)
    assert call(big) == -6
    assert "static buffer" in cbb.status_string(-6)
    d = _desc(in_c=5)
    for missing in ("x", "w", "delta", "dw", "db", "x_norm", "gamma"):
        assert call(d, **{missing: None}) == -1
    assert call(d, acc=2) == -1
    assert call(_desc(batch=0)) == -1


def test_sgd_update_validates():
    L = cbb.lib()
    X, Y = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000)
    assert L.cbb_sgd_update(-1, 1, 0.1, 0.9, 0.0, X, Y, None) == -1
    assert L.cbb_sgd_update(10, 0, 0.1, 0.9, 0.0, X, Y, None) == -1
    assert L.cbb_sgd_update(10, 1, -0.1, 0.9, 0.0, X, Y, None) == -1
    assert L.cbb_sgd_update(10, 1, 0.1, float("nan"), 0.0, X, Y, None) == -1
    assert L.cbb_sgd_update(10, 1, 0.1, 0.9, -1.0, X, Y, None) == -1
    assert L.cbb_sgd_update(10, 1, 0.1, 0.9, 0.0, X, X, None) == -1
    assert L.cbb_sgd_update(10, 1, 0.1, 0.9, 0.0, None, Y, None) == -1
    assert L.cbb_sgd_update(0, 1, 0.1, 0.9, 0.0, X, Y, None) == 0     # empty: no launch
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError, match="dw"):
        cbb.sgd_update(torch.zeros(10), torch.zeros(9), 1, 0.1)


def test_block_options_validate_on_the_host():
    """cbb_block_opts: sums only with batch statistics, below sums need dx, the block
    below's x_norm (and y unless it is linear) and a valid activation; tensors of the
    block below without a place for its sums are refused, and so is the apply flag
    (0 or 1) without them; the data-only call takes no sums of its own.  All refused before any HIP call."""
    L = cbb.lib()
    names = ["x", "w", "y", "x_norm", "var", "gamma", "delta", "dz", "dw", "db", "dgamma", "dx"]

    def call(d, opts, **kw):
        return L.cbb_conv_block_backward_ex(ctypes.byref(d), *[kw.get(k, BOGUS) for k in names],
                                            kw.get("acc", 0), ctypes.byref(opts), BOGUS, 1 << 30,
                                            None)

    nobn = _desc(in_c=5, batch_normalize=0)
    o = cbb.BlockOpts(sums=0x2000)
    assert call(nobn, o, x_norm=None, var=None, gamma=None, dgamma=None) == -1
    fixed = _desc(in_c=5, batch_normalize=2)
    assert call(fixed, o) == -1
    d = _desc(in_c=5)
    o = cbb.BlockOpts(below_sums=0x2000, below_x_norm=0x3000, below_act=1)
    assert call(d, o) == -1                       # leaky below without its y
    o.below_y = 0x4000
    assert call(d, o, dx=None) == -1              # the sums below need dx
    assert call(d, cbb.BlockOpts(below_sums=0x2000, below_y=0x4000, below_act=1)) == -1
    assert call(d, cbb.BlockOpts(below_sums=0x2000, below_x_norm=0x3000, below_act=14)) == -1
    assert call(d, cbb.BlockOpts(below_y=0x4000, below_x_norm=0x3000)) == -1
    assert call(d, cbb.BlockOpts(sums=0x2000, below_sums=0x2000, below_x_norm=0x3000)) == -1
    # dx left holding g only where the sums below are made, and the flag is 0 or 1
    assert call(d, cbb.BlockOpts(below_apply_act=1)) == -1
    assert call(d, cbb.BlockOpts(below_sums=0x2000, below_y=0x4000, below_x_norm=0x3000,
                                 below_act=1, below_apply_act=2)) == -1
    o4 = cbb.BlockOpts(sums=0x2000)
    assert L.cbb_conv_backward_data_ex(ctypes.byref(d), BOGUS, BOGUS, BOGUS, 0, ctypes.byref(o4),
                                       BOGUS, 1 << 30, None) == -1
    # which layers add the sums up in their input-gradient kernel
    assert cbb.conv_fuses_below_sums(cbb.conv_desc(16, 32, 416, 416, 64, 3, 2, 1, 1, "leaky"))
    assert cbb.conv_fuses_below_sums(cbb.conv_desc(2, 32, 40, 72, 64, 3, 2, 1, 1, "leaky"))
    # 128 output channels on a small image: the input gradient is split over them
    assert not cbb.conv_fuses_below_sums(cbb.conv_desc(2, 32, 40, 72, 128, 3, 2, 1, 1, "leaky"))
    assert not cbb.conv_fuses_below_sums(cbb.conv_desc(8, 128, 52, 52, 256, 3, 1, 1, 1, "leaky"))
    assert not cbb.conv_fuses_below_sums(cbb.conv_desc(2, 64, 40, 72, 64, 3, 2, 1, 1, "leaky"))
    assert L.cbb_conv_fuses_below_sums(ctypes.byref(_desc(batch=0))) == -1
