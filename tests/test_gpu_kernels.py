"""GPU parity of each entry point on small and ragged shapes, plus the bit-exact
cases (coverage counts, one-hot probes, copies and single adds)."""
import types

import numpy as np
import pytest

import oracle as O
import oracle.model as M
from gpu_common import announce, assert_close, assert_exact, require_gpu

pytestmark = pytest.mark.gpu


def _layer(c, oc, k, s, p, bn, act, h, w, groups=1, dilation=1):
    return types.SimpleNamespace(in_c=c, out_c=oc, k=k, stride=s, pad=p, bn=bn, act=act,
                                 in_h=h, in_w=w, groups=groups, dilation=dilation)


def _t(torch, a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(dtype if dtype is not None else torch.float32).cuda()


CONV_CASES = [  # n, c, h, w, oc, k, s, p, bn, act
    (2, 3, 32, 32, 16, 3, 1, 1, True, "leaky"),
    (1, 5, 13, 11, 7, 3, 2, 1, True, "leaky"),
    (3, 2, 9, 17, 33, 5, 1, 2, True, "logistic"),
    (2, 70, 10, 9, 65, 1, 1, 0, True, "relu"),
    (1, 1, 28, 28, 20, 5, 1, 0, False, "linear"),
    (2, 20, 12, 12, 50, 5, 1, 0, False, "linear"),
    (2, 33, 15, 15, 40, 3, 2, 0, False, "leaky"),
    (1, 4, 17, 19, 3, 7, 3, 3, True, "leaky"),
    (2, 8, 7, 7, 96, 1, 2, 0, True, "leaky"),
    (4, 129, 6, 6, 130, 3, 1, 1, True, "leaky"),
    (1, 3, 5, 5, 1, 5, 1, 0, False, "linear"),
    (2, 16, 21, 21, 8, 4, 2, 1, True, "leaky"),
    (2, 64, 13, 13, 128, 3, 1, 1, True, "leaky"),    # dX: tap-aligned K, split over K
    (2, 32, 20, 20, 256, 3, 2, 1, True, "leaky"),    # dX: stride-2 phases, tap-aligned, split
    (4, 3, 128, 128, 8, 3, 1, 1, True, "leaky"),     # dW: many splits (two-level reduce)
    (2, 2, 19, 70, 5, 7, 1, 3, False, "relu"),       # dX: 2-channel direct kernel, k = 7
    (3, 4, 9, 9, 6, 1, 1, 0, True, "logistic"),      # dX: 4-channel direct kernel, k = 1
    (1, 64, 17, 23, 32, 3, 1, 1, True, "leaky"),     # dX: 3x3 tile-direct, ragged width
    (2, 32, 19, 37, 16, 3, 2, 1, True, "leaky"),     # dX: 3x3 stride-2 tile-direct, odd sizes
    (1, 64, 9, 62, 16, 3, 1, 1, False, "linear"),    # dX: tile-direct at the widest image
    (3, 32, 7, 8, 48, 3, 1, 1, True, "relu"),        # dX: tile-direct at the narrowest image
    (2, 64, 12, 130, 64, 3, 2, 1, True, "leaky"),    # dX: stride-2, width beyond one region
    (2, 32, 20, 104, 64, 3, 2, 1, True, "leaky"),    # dW row-streaming: stride 2, split runs
    (1, 32, 15, 121, 64, 3, 2, 1, True, "leaky"),    # dW row-streaming: odd sizes, ragged strip
    (2, 64, 11, 52, 128, 3, 1, 1, True, "leaky"),    # dW row-streaming: stride 1, 2x2 (o, i) blocks
    (3, 32, 9, 26, 64, 3, 1, 1, False, "linear"),    # dW row-streaming: 26-wide strip
    (1, 96, 5, 62, 64, 3, 1, 1, True, "relu"),       # dW row-streaming: 64-wide strip, one split
    (4, 32, 64, 52, 64, 3, 1, 1, True, "leaky"),     # dW row-streaming: many runs, two-level sum
    (1, 32, 1, 30, 64, 3, 1, 1, True, "leaky"),      # dW row-streaming: a single output row
    (2, 32, 2, 60, 64, 3, 2, 1, True, "leaky"),      # dW row-streaming: stride 2, one output row
    (1, 32, 12, 416, 64, 3, 2, 1, True, "leaky"),    # dW row-streaming: 104-wide strips, stride 2
    (1, 32, 5, 208, 64, 3, 1, 1, False, "linear"),   # dW row-streaming: 104-wide strips, stride 1
    (2, 64, 12, 12, 96, 1, 1, 0, True, "leaky"),     # 1x1 GEMMs with 16-byte staging, ragged o
    (3, 20, 6, 10, 70, 1, 1, 0, False, "linear"),    # 1x1 GEMMs: ragged i and o tiles
    (4, 32, 64, 64, 48, 1, 1, 0, True, "leaky"),     # 1x1 dW: 64 K splits, two-level sum
    (2, 128, 26, 26, 255, 1, 1, 0, False, "linear"), # 1x1: 255 output channels (ragged K of dX)
    (2, 16, 12, 12, 32, 3, 1, 1, True, "tanh"),      # the other activations, batch BN
    (2, 24, 10, 10, 40, 3, 1, 1, 2, "selu"),         # BN with fixed statistics
    (3, 20, 9, 9, 24, 1, 1, 0, 2, "loggy"),          # fixed statistics, 1x1
    (2, 8, 11, 13, 16, 3, 2, 1, False, "stair"),     # no BN, run-time activation switch
    (2, 64, 12, 12, 64, 3, 1, 1, 2, "leaky"),        # fixed statistics, 3x3 tile-direct
    (2, 64, 40, 31, 24, 3, 1, 1, True, "leaky"),     # dX: 128-pixel tile-direct, ragged plane
    (2, 3, 24, 40, 32, 3, 1, 1, True, "logistic"),   # first layer, logistic
    (1, 2, 17, 36, 12, 3, 1, 1, False, "relu"),      # first layer, bias only
    (2, 1, 20, 16, 5, 3, 1, 1, True, "linear"),      # first layer, BN, no activation
    (1, 3, 13, 132, 30, 3, 1, 1, False, "leaky"),    # first layer, two column strips
    (6, 32, 200, 264, 64, 3, 2, 1, True, "leaky"),   # stride-2 dX: persistent, 1-2 tiles per WG
    (2, 32, 36, 136, 128, 3, 2, 1, False, "relu"),   # stride-2 dX: persistent, 8 chunks per tile
]


def run_conv(torch, case, seed, dx_accumulate=False, in_place=False, want_dx=True, form_dz=False):
    from cnn_backward_pass_amd import cbb
    n, c, h, w, oc, k, s, p, bn, act = case[:10]
    groups, dil = case[10:12] if len(case) > 10 else (1, 1)
    L = _layer(c, oc, k, s, p, bn, act, h, w, groups, dil)
    r = np.random.default_rng(seed)
    x = r.normal(size=(n, c, h, w)).astype(np.float32)
    wt = (r.normal(size=(oc, c // groups, k, k)) * 0.2).astype(np.float32)
    gamma = (1.0 + 0.3 * r.normal(size=oc)) if bn else None
    beta = r.normal(size=oc) if bn else None
    bias = None if bn else r.normal(size=oc)
    # fixed statistics (bn = 2): the stored mean and variance
    mean, var = (r.normal(size=oc), r.uniform(0.5, 2.0, size=oc)) if bn == 2 else (None, None)
    saved = M.round_saved_to_f32(M.conv_block_forward(L, x, wt, bias=bias, gamma=gamma, beta=beta,
                                                      mean=mean, var=var))
    delta = r.normal(size=saved["y"].shape).astype(np.float32)
    dx0 = r.normal(size=x.shape).astype(np.float32)
    ref = M.conv_block_backward(L, saved, delta, want_dx=want_dx,
                                dx_init=dx0 if dx_accumulate else None)
    desc = cbb.conv_desc(n, c, h, w, oc, k, s, p, bn, act, groups=groups, dilation=dil)
    T = lambda a: None if a is None else _t(torch, a)
    d_delta = T(delta)
    d_dz = d_delta if in_place else (torch.empty_like(d_delta) if (bn or act != "linear") else None)
    if form_dz:   # dz not stored: the fused kernel forms it from delta, y and x_hat
        d_dz = None
    dw = T(np.ones_like(wt) * 0.5)              # accumulation target with a known start
    db = T(np.full(oc, 0.25, np.float32))
    dg = T(np.full(oc, -0.5, np.float32)) if bn else None
    dx = T(dx0) if want_dx else None
    ws = cbb.workspace(cbb.conv_block_workspace_size(desc))
    cbb.conv_block_backward(desc, T(saved["x_in"]), T(wt), T(saved["y"]) if act != "linear" else None,
                            T(saved.get("xhat")) if bn else None, T(saved.get("var")) if bn else None,
                            T(saved.get("gamma")) if bn else None, d_delta, d_dz, dw, db, dg, dx,
                            dx_accumulate, ws)
    torch.cuda.synchronize()
    h_ = lambda t: t.cpu().double().numpy()
    got = {"dw": h_(dw) - 0.5, "db": h_(db) - 0.25}
    if bn:
        got["dgamma"] = h_(dg) + 0.5
    if d_dz is not None:
        got["dz"] = h_(d_dz)
    if want_dx:
        got["dx"] = h_(dx)
    return ref, got


@pytest.mark.parametrize("case", CONV_CASES)
def test_conv_block_backward_parity(case):
    torch = require_gpu()
    announce(f"conv_block {case}")
    ref, got = run_conv(torch, case, seed=100 + CONV_CASES.index(case))
    for k in ("dw", "db", "dz", "dx", "dgamma"):
        if k in got:
            assert_close(k, got[k], ref[k] if k != "dgamma" else ref["dgamma"])


FORM_DZ_CASES = [  # first layers whose dz the fused dW + dX kernel forms as it stages delta
    (2, 3, 32, 32, 16, 3, 1, 1, True, "leaky"),
    (2, 3, 24, 40, 32, 3, 1, 1, True, "logistic"),
    (1, 2, 17, 36, 12, 3, 1, 1, False, "relu"),      # bias only: dz = g
    (2, 1, 20, 16, 5, 3, 1, 1, True, "linear"),      # BN without activation: no y
    (1, 3, 13, 132, 30, 3, 1, 1, False, "leaky"),    # two column strips
    (2, 3, 12, 16, 32, 3, 1, 1, 2, "tanh"),          # fixed statistics: dz = a g
    (4, 3, 128, 128, 8, 3, 1, 1, True, "leaky"),     # many work-groups, two-level dW sum
    (1, 3, 30, 8, 17, 3, 1, 1, True, "loggy"),       # run-time activation switch
    (1, 3, 1, 60, 32, 3, 1, 1, True, "leaky"),       # a single row
    (3, 2, 2, 28, 9, 3, 1, 1, True, "relu"),         # two rows
    (2, 3, 33, 56, 32, 3, 1, 1, True, "leaky"),      # an odd row count
    (2, 3, 40, 416, 32, 3, 1, 1, True, "leaky"),     # the stem's width: four strips
]


@pytest.mark.parametrize("acc", [False, True])
@pytest.mark.parametrize("case", FORM_DZ_CASES)
def test_conv_block_backward_forms_dz(case, acc):
    """dz = NULL on a fused first layer: dz is formed inside the dW + dX kernel from
    delta, y and x_hat with the BN backward's per-channel map; dW, db, dgamma and dx
    match the oracle as on the stored-dz route."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    n, c, h, w, oc, k, s, p, bn, act = case
    assert cbb.conv_fused_weights_data(cbb.conv_desc(n, c, h, w, oc, k, s, p, bn, act)) == 1
    announce(f"conv_block forming dz {case} accumulate={acc}")
    ref, got = run_conv(torch, case, seed=500 + FORM_DZ_CASES.index(case), dx_accumulate=acc,
                        form_dz=True)
    assert "dz" not in got
    for key in ("dw", "db", "dx", "dgamma"):
        if key in got:
            assert_close(key, got[key], ref[key])


DW_FORMS_DZ_CASES = [  # batch statistics on the row-streaming 3x3 dW kernel's 16-byte path
    (2, 32, 20, 104, 64, 3, 2, 1, True, "leaky"),    # stride 2, 52-wide strips
    (2, 32, 11, 52, 128, 3, 1, 1, True, "logistic"), # run-time activation, two output blocks
    (1, 32, 9, 64, 64, 3, 1, 1, True, "linear"),     # no activation: y not read
    (2, 32, 12, 416, 64, 3, 2, 1, True, "relu"),     # four strips per row
    (1, 32, 7, 32, 64, 3, 1, 1, True, "tanh"),       # 32-wide strip
]


@pytest.mark.parametrize("acc", [False, True])
@pytest.mark.parametrize("case", DW_FORMS_DZ_CASES)
def test_dw_kernel_forms_and_writes_dz(case, acc):
    """The weight-gradient kernel forms dz from delta, y and x_hat, writes it (each element
    once) and dX reads it: dz, dW, db, dgamma, dx match the
    oracle.  In place (dz = delta) the stored-dz route runs instead."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    n, c, h, w, oc, k, s, p, bn, act = case
    assert cbb.conv_dw_forms_dz(cbb.conv_desc(n, c, h, w, oc, k, s, p, bn, act))
    announce(f"dW forming dz {case} accumulate={acc}")
    ref, got = run_conv(torch, case, seed=700 + DW_FORMS_DZ_CASES.index(case), dx_accumulate=acc)
    for key in ("dz", "dw", "db", "dx", "dgamma"):
        assert_close(key, got[key], ref[key])
    ref, got = run_conv(torch, case, seed=701, in_place=True)
    for key in ("dz", "dw", "dx"):
        assert_close(key + " (in place)", got[key], ref[key])


GD_CASES = [  # n, c, h, w, oc, k, s, p, bn, act, groups, dilation
    (2, 8, 13, 13, 12, 3, 1, 1, True, "leaky", 2, 1),       # grouped 3x3
    (2, 16, 12, 12, 16, 3, 1, 2, True, "leaky", 16, 2),     # depthwise, dilated
    (2, 6, 15, 14, 9, 3, 2, 2, False, "linear", 3, 2),      # stride 2, dilation 2, 3 groups
    (1, 4, 17, 16, 8, 5, 1, 4, True, "relu", 1, 2),         # dilated 5x5
    (2, 12, 10, 12, 24, 1, 1, 0, True, "leaky", 4, 1),      # grouped 1x1
    (2, 64, 20, 20, 64, 3, 1, 1, True, "leaky", 2, 1),      # grouped, channels of the 3x3 kernels
    (1, 6, 19, 19, 6, 3, 3, 3, False, "leaky", 2, 3),       # stride 3, dilation 3
    (2, 64, 8, 8, 256, 3, 1, 1, True, "leaky", 2, 1),       # dX split over K across the groups
    (2, 32, 13, 13, 32, 3, 2, 1, True, "leaky", 32, 1),     # depthwise, stride 2
    (3, 24, 17, 15, 24, 5, 1, 2, False, "relu", 24, 1),     # depthwise 5x5
    # depthwise 1x1, no BN: with BN its dW would be sum dz * x, a multiple of sum dz * x_norm
    # (x_norm is affine in x per channel) -- zero up to an eps-sized residue
    (2, 8, 9, 9, 8, 1, 1, 0, False, "leaky", 8, 1),
    (8, 64, 52, 52, 64, 3, 1, 1, True, "leaky", 64, 1),     # depthwise, many segments per channel
    (2, 16, 12, 12, 32, 3, 1, 1, True, "leaky", 16, 1),     # two filters per channel (general)
    (2, 64, 10, 52, 128, 3, 1, 1, True, "leaky", 2, 1),     # grouped dW on the row-streaming kernel
    (2, 64, 40, 104, 128, 3, 2, 1, False, "relu", 2, 1),    # the same at stride 2, 5 row runs
    # grouped row-streaming dW with more than 32 splits per group: the two-level
    # ordered reduction (dw_reduce_l1 / l2) on tap-major partials, stride 1 and 2
    (4, 64, 64, 104, 128, 3, 1, 1, True, "leaky", 2, 1),
    (4, 64, 64, 208, 128, 3, 2, 1, False, "relu", 2, 1),
    (1, 4, 96, 96, 4, 3, 1, 1, True, "leaky", 4, 1),        # depthwise, plane beyond LDS: streaming
    # grouped 3x3 dX on the tile-direct kernel (one grid row per group): 32-channel tiles
    # split over K, the same at stride 2, and 64-channel tiles split four ways
    (2, 64, 32, 32, 128, 3, 1, 1, True, "leaky", 2, 1),
    (2, 64, 16, 64, 256, 3, 2, 1, True, "leaky", 2, 1),
    (2, 128, 16, 16, 256, 3, 1, 1, False, "linear", 2, 1),
    (2, 8, 90, 91, 8, 5, 2, 2, False, "relu", 8, 1),        # depthwise, 8190-pixel plane in LDS, s2
    # dilation-2 3x3 (pad 2) dX on the stride-1 tile-direct kernel: 256-pixel tiles with
    # 16-byte tile copies, 128-pixel tiles, and 4-byte copies (width not a multiple of 4);
    # dilation 3 stays on the general kernel
    (2, 64, 12, 20, 16, 3, 1, 2, True, "leaky", 1, 2),
    (1, 32, 40, 36, 24, 3, 1, 2, False, "relu", 1, 2),
    (2, 64, 9, 18, 8, 3, 1, 2, True, "linear", 1, 2),
    (1, 32, 40, 36, 24, 3, 1, 3, False, "relu", 1, 3),
]


@pytest.mark.parametrize("case", GD_CASES)
def test_grouped_dilated_conv_block(case):
    """Grouped and dilated layers (all groups in one launch: the general kernels, the
    row-streaming 3x3 dW kernel for grouped 3x3 layers with 32k input and 64k output
    channels per group, the tile-direct 3x3 dX kernel for grouped 3x3 pad-1 layers,
    streaming kernels for depthwise layers) against the oracle's grouped / dilated
    loops; overwrite, then accumulate in place."""
    torch = require_gpu()
    announce(f"grouped/dilated conv_block {case}")
    ref, got = run_conv(torch, case, seed=300 + GD_CASES.index(case))
    for k in ("dw", "db", "dz", "dx", "dgamma"):
        if k in got:
            assert_close(k, got[k], ref[k])
    ref, got = run_conv(torch, case, seed=7, dx_accumulate=True, in_place=True)
    for k in ("dw", "db", "dx"):
        assert_close(k + " (accumulate)", got[k], ref[k])


@pytest.mark.parametrize("case", [CONV_CASES[0], CONV_CASES[1], CONV_CASES[3], CONV_CASES[5],
                                  CONV_CASES[6], CONV_CASES[12], CONV_CASES[13], CONV_CASES[17],
                                  CONV_CASES[18], CONV_CASES[22], CONV_CASES[26], CONV_CASES[33],
                                  CONV_CASES[35],
                                  CONV_CASES[-2]])
def test_conv_block_accumulate_inplace_and_no_dx(case):
    torch = require_gpu()
    announce(f"conv_block accumulate/in-place {case}")
    ref, got = run_conv(torch, case, seed=7, dx_accumulate=True, in_place=True)
    for k in ("dw", "db", "dx"):
        assert_close(k, got[k], ref[k])
    if "dz" in got:
        assert_close("dz in place", got["dz"], ref["dz"])
    ref, got = run_conv(torch, case, seed=8, want_dx=False)
    assert_close("dw (no dx)", got["dw"], ref["dw"])


@pytest.mark.parametrize("case", [CONV_CASES[0], CONV_CASES[-4], CONV_CASES[-1]])
def test_first_layer_accumulate(case):
    """First layers (one streaming kernel for dW and dX) with dx accumulation and dz
    in its own buffer."""
    torch = require_gpu()
    announce(f"first layer, accumulate {case}")
    ref, got = run_conv(torch, case, seed=9, dx_accumulate=True)
    for k in ("dw", "db", "dz", "dx"):
        assert_close(k, got[k], ref[k])


@pytest.mark.parametrize("case", [(2, 3, 32, 32, 16, 3, 1, 1), (1, 4, 41, 41, 6, 3, 2, 1),
                                  (2, 5, 9, 10, 3, 5, 2, 2), (3, 6, 8, 8, 70, 1, 1, 0),
                                  (1, 33, 19, 23, 65, 3, 1, 1), (2, 3, 30, 30, 32, 3, 1, 1),
                                  (1, 32, 9, 60, 64, 3, 2, 1), (2, 64, 8, 52, 128, 3, 1, 1)])
def test_conv_coverage_bit_exact(case):
    """W = 1, delta = 1 (linear, no BN): dx counts covering windows times C_out; with x = 1,
    dW counts valid taps times N; db = N*OH*OW.  Integers below 2^24: exact in fp32."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    announce(f"coverage {case}")
    n, c, h, w, oc, k, s, p = case
    desc = cbb.conv_desc(n, c, h, w, oc, k, s, p, 0, "linear")
    oh, ow = desc.out_h, desc.out_w
    ones_w = np.ones((oc, c, k, k), np.float32)
    ones_x = np.ones((n, c, h, w), np.float32)
    ones_d = np.ones((n, oc, oh, ow), np.float32)
    dw = torch.zeros(oc, c, k, k, device="cuda")
    db = torch.zeros(oc, device="cuda")
    dx = torch.zeros(n, c, h, w, device="cuda")
    ws = cbb.workspace(cbb.conv_block_workspace_size(desc))
    cbb.conv_block_backward(desc, _t(torch, ones_x), _t(torch, ones_w), None, None, None, None,
                            _t(torch, ones_d), None, dw, db, None, dx, False, ws)
    torch.cuda.synchronize()
    assert_exact("dx", dx.cpu().double().numpy(),
                 O.conv_backward_data(ones_w, ones_d, (h, w), s, p))
    assert_exact("dw", dw.cpu().double().numpy(), O.conv_backward_weights(ones_x, ones_d, k, s, p))
    assert_exact("db", db.cpu().double().numpy(), np.full(oc, n * oh * ow, np.float64))


@pytest.mark.parametrize("case", [  # n, c, h, w, oc, k, s, p
    (2, 3, 32, 32, 16, 3, 1, 1),    # fused: the single-block layer
    (3, 3, 19, 44, 32, 3, 1, 1),    # fused: ragged tiles in both directions, 32 outputs
    (1, 1, 9, 12, 7, 3, 1, 1),      # fused: one input channel, one partial tile
    (2, 2, 40, 68, 20, 3, 1, 1),    # fused: two input channels
    (1, 3, 1, 4, 5, 3, 1, 1),       # fused: one image row
    (1, 3, 37, 244, 32, 3, 1, 1),   # fused: three column strips, runs of one row
    (8, 3, 100, 256, 32, 3, 1, 1),  # fused: ragged last strip, runs of four rows
    (2, 3, 20, 20, 40, 3, 1, 1),    # not fused: more than 32 outputs
    (1, 3, 9, 9, 8, 3, 1, 1),       # not fused: width not a multiple of 4
    (2, 4, 12, 12, 8, 3, 1, 1),     # not fused: four inputs
    (2, 32, 20, 104, 64, 3, 2, 1),  # not fused: row-streaming dW, tile-direct dX
])
def test_conv_backward_weights_data(case):
    """dW and dX from one call (fused where the library reports it) against the oracle,
    with and without dx, overwrite and accumulate."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    n, c, h, w, oc, k, s, p = case
    announce(f"weights_data {case}")
    r = np.random.default_rng(500 + c * 7 + oc)
    oh, ow = O.conv_out_dim(h, k, s, p), O.conv_out_dim(w, k, s, p)
    x = r.normal(size=(n, c, h, w)).astype(np.float32)
    wt = (r.normal(size=(oc, c, k, k)) * 0.3).astype(np.float32)
    dz = r.normal(size=(n, oc, oh, ow)).astype(np.float32)
    dx0 = r.normal(size=x.shape).astype(np.float32)
    desc = cbb.conv_desc(n, c, h, w, oc, k, s, p, False, "linear")
    expect_fused = c <= 3 and k == 3 and p == 1 and s == 1 and oc <= 32 and w % 4 == 0
    assert cbb.conv_fused_weights_data(desc) == expect_fused
    ref_dw = O.conv_backward_weights(x, dz, k, s, p)
    ref_dx = O.conv_backward_data(wt, dz, (h, w), s, p)
    ws = cbb.workspace(cbb.conv_block_workspace_size(desc))
    for accumulate in (False, True):
        dw = _t(torch, np.full(wt.shape, 0.5, np.float32))
        dx = _t(torch, dx0)
        cbb.conv_backward_weights_data(desc, _t(torch, x), _t(torch, wt), _t(torch, dz), dw, dx,
                                       accumulate, ws)
        torch.cuda.synchronize()
        assert_close("dw", dw.cpu().double().numpy() - 0.5, ref_dw)
        assert_close("dx", dx.cpu().double().numpy(), ref_dx + (dx0 if accumulate else 0.0))
    dw = _t(torch, np.zeros(wt.shape, np.float32))
    cbb.conv_backward_weights_data(desc, _t(torch, x), _t(torch, wt), _t(torch, dz), dw, None,
                                   False, ws)
    torch.cuda.synchronize()
    assert_close("dw (no dx)", dw.cpu().double().numpy(), ref_dw)


@pytest.mark.parametrize("case", [(2, 64, 12, 12, 96, 1, 1, 0), (1, 3, 9, 12, 8, 3, 1, 1),
                                  (1, 64, 9, 20, 16, 3, 1, 1), (1, 32, 40, 30, 16, 3, 1, 1),
                                  (2, 32, 12, 70, 32, 3, 2, 1)])
def test_misaligned_tensors_take_the_general_kernels(case):
    """Tensors that are not 16-byte aligned (a view one float into a buffer) go through
    the general kernels, or the 3x3 input-gradient kernels staged through registers
    (same tiles, same workspace), and give the same gradients."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    n, c, h, w, oc, k, s, p = case
    announce(f"misaligned {case}")
    r = np.random.default_rng(77)
    oh, ow = O.conv_out_dim(h, k, s, p), O.conv_out_dim(w, k, s, p)
    x = r.normal(size=(n, c, h, w)).astype(np.float32)
    wt = (r.normal(size=(oc, c, k, k)) * 0.3).astype(np.float32)
    dz = r.normal(size=(n, oc, oh, ow)).astype(np.float32)

    def shifted(a):  # contiguous view starting 4 bytes after a 256-byte aligned allocation
        buf = torch.empty(a.size + 1, dtype=torch.float32, device="cuda")
        v = buf[1:].view(a.shape)
        v.copy_(torch.from_numpy(a))
        return v

    desc = cbb.conv_desc(n, c, h, w, oc, k, s, p, False, "linear")
    ws = cbb.workspace(cbb.conv_block_workspace_size(desc))
    dw = _t(torch, np.zeros(wt.shape, np.float32))
    dx = shifted(np.zeros(x.shape, np.float32))
    cbb.conv_backward_weights_data(desc, shifted(x), shifted(wt), shifted(dz), dw, dx, False, ws)
    torch.cuda.synchronize()
    assert_close("dw", dw.cpu().double().numpy(), O.conv_backward_weights(x, dz, k, s, p))
    assert_close("dx", dx.cpu().double().numpy(), O.conv_backward_data(wt, dz, (h, w), s, p))


def test_conv_one_hot_probes_bit_exact():
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    n, c, h, w, oc, k, s, p = 2, 5, 9, 9, 4, 3, 2, 1
    announce("one-hot probes")
    desc = cbb.conv_desc(n, c, h, w, oc, k, s, p, 0, "linear")
    oh, ow = desc.out_h, desc.out_w
    r = np.random.default_rng(5)
    x = r.normal(size=(n, c, h, w)).astype(np.float32)
    wt = r.normal(size=(oc, c, k, k)).astype(np.float32)
    ws = cbb.workspace(cbb.conv_block_workspace_size(desc))
    for (b, o, y0, x0) in [(0, 0, 0, 0), (1, 3, oh - 1, ow - 1), (0, 2, 0, ow - 1),
                           (1, 1, oh - 1, 0), (0, 0, oh // 2, ow // 2), (1, 2, 1, 2)]:
        d = np.zeros((n, oc, oh, ow), np.float32)
        d[b, o, y0, x0] = 1.0
        dw = torch.zeros(oc, c, k, k, device="cuda")
        db = torch.zeros(oc, device="cuda")
        dx = torch.zeros(n, c, h, w, device="cuda")
        cbb.conv_block_backward(desc, _t(torch, x), _t(torch, wt), None, None, None, None,
                                _t(torch, d), None, dw, db, None, dx, False, ws)
        torch.cuda.synchronize()
        assert_exact("probe dx", dx.cpu().double().numpy(), O.conv_backward_data(wt, d, (h, w), s, p))
        assert_exact("probe dw", dw.cpu().double().numpy(), O.conv_backward_weights(x, d, k, s, p))


@pytest.mark.parametrize("shape", [
    (2, 16, 32, 32), (8, 256, 26, 26),          # one pass, 256-thread work-groups
    (1, 8, 96, 64),                             # one pass at its 256 x 6 float4 limit
    (1, 8, 96, 68), (8, 32, 52, 52),            # one pass, 1024-thread work-groups
    (6, 4, 64, 64),                             # one pass at its 1024 x 6 float4 limit
    (6, 4, 64, 68), (2, 4, 128, 128),           # two streaming passes (16-byte loads)
    (3, 5, 7, 9), (2, 3, 1, 1)])                # two passes, element loads
def test_bn_backward_entry_point(shape):
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    announce(f"bn_backward {shape}")
    r = np.random.default_rng(11)
    n, c = shape[:2]
    z = r.normal(size=shape) * 1.5 + 0.2
    gamma = 1 + 0.2 * r.normal(size=c)
    _, var, xhat, _ = O.bn_forward(z, gamma, np.zeros(c), 1e-5)
    g = r.normal(size=shape).astype(np.float32)
    xhat32, var32, gamma32 = (a.astype(np.float32) for a in (xhat, var, gamma))
    dz_ref, dg_ref, dbeta_ref = O.bn_backward(g, xhat32, var32, gamma32, 1e-5)
    hw = int(np.prod(shape[2:]))
    ws = cbb.workspace(cbb.bn_backward_workspace_size(n, c, hw))
    dz = torch.empty(shape, device="cuda")
    dg = torch.zeros(c, device="cuda")
    dbeta = torch.zeros(c, device="cuda")
    cbb.bn_backward(_t(torch, g), _t(torch, xhat32), _t(torch, var32), _t(torch, gamma32), dz, dg,
                    dbeta, 1e-5, ws)
    torch.cuda.synchronize()
    # Two samples per channel: dz is the difference of terms of size |gamma g|/sigma that
    # cancel to ~1e-4 of themselves, so fp32 reaches it only to ~eps32 of the terms.
    terms = np.abs(gamma32[None, :, None, None] / np.sqrt(var32 + 1e-5)[None, :, None, None]
                   * g).max()
    if n * hw > 2:
        assert_close("dz", dz.cpu().double().numpy(), dz_ref)
    else:
        err = np.abs(dz.cpu().double().numpy() - dz_ref).max()
        assert err <= 1e-5 * terms, (err, terms)
    assert_close("dgamma", dg.cpu().double().numpy(), dg_ref)
    assert_close("dbeta", dbeta.cpu().double().numpy(), dbeta_ref)
    # invariant of a consistent forward: sum dz ~ 0 per channel
    s = dz.cpu().double().numpy().sum(axis=tuple(i for i in range(len(shape)) if i != 1))
    scale = np.abs(dz.cpu().double().numpy()).sum(axis=tuple(i for i in range(len(shape)) if i != 1))
    if n * hw > 2:
        assert np.all(np.abs(s) <= 1e-5 * scale + 1e-30)
    else:  # the degenerate two-sample case: bounded by the size of the cancelling terms
        assert np.all(np.abs(s) <= 1e-5 * terms)


@pytest.mark.parametrize("shape", [(2, 16, 32, 32), (4, 64, 13, 13), (3, 5, 7, 9), (1, 3, 1, 1),
                                   (6, 4, 64, 64),      # one pass at its 1024 x 6 float4 limit
                                   (2, 4, 128, 128)])   # the streaming pass
def test_bn_backward_fixed_entry_point(shape):
    """Fixed statistics: dz = gamma g / sqrt(var + eps) in the streaming pass, dgamma /
    dbeta from the per-segment sums, added onto non-zero values."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    announce(f"bn_backward_fixed {shape}")
    r = np.random.default_rng(17)
    n, c = shape[:2]
    z = r.normal(size=shape)
    gamma = (1 + 0.2 * r.normal(size=c)).astype(np.float32)
    mean, var = r.normal(size=c), r.uniform(0.5, 2.0, size=c).astype(np.float32)
    xhat, _ = O.bn_forward_fixed(z, mean, var, gamma, np.zeros(c), 1e-5)
    g = r.normal(size=shape).astype(np.float32)
    xhat32 = xhat.astype(np.float32)
    dz_ref, dg_ref, dbeta_ref = O.bn_backward_fixed(g, xhat32, var, gamma, 1e-5)
    hw = int(np.prod(shape[2:]))
    ws = cbb.workspace(cbb.bn_backward_workspace_size(n, c, hw))
    dz = torch.empty(shape, device="cuda")
    dg = _t(torch, np.full(c, 0.5, np.float32))
    dbeta = _t(torch, np.full(c, -0.25, np.float32))
    cbb.bn_backward_fixed(_t(torch, g), _t(torch, xhat32), _t(torch, var), _t(torch, gamma), dz,
                          dg, dbeta, 1e-5, ws)
    torch.cuda.synchronize()
    assert_close("dz", dz.cpu().double().numpy(), dz_ref)
    assert_close("dgamma", dg.cpu().double().numpy() - 0.5, dg_ref)
    assert_close("dbeta", dbeta.cpu().double().numpy() + 0.25, dbeta_ref)


@pytest.mark.parametrize("shape", [(16, 32, 104, 104), (2, 300, 16, 16), (1, 7, 1, 4)])
def test_bn_backward_in_place_accumulating(shape):
    """dz written over g, dgamma / dbeta added to non-zero values, workspace holding
    garbage on entry: a large plane, many short channels, one tiny plane."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    announce(f"bn_backward in place {shape}")
    r = np.random.default_rng(12)
    n, c = shape[:2]
    z = r.normal(size=shape) * 0.7 - 0.3
    gamma = 1 + 0.2 * r.normal(size=c)
    _, var, xhat, _ = O.bn_forward(z, gamma, np.zeros(c), 1e-5)
    g = r.normal(size=shape).astype(np.float32)
    xhat32, var32, gamma32 = (a.astype(np.float32) for a in (xhat, var, gamma))
    dz_ref, dg_ref, dbeta_ref = O.bn_backward(g, xhat32, var32, gamma32, 1e-5)
    hw = int(np.prod(shape[2:]))
    ws = cbb.workspace(cbb.bn_backward_workspace_size(n, c, hw))
    ws.fill_(0xAB)
    dg = torch.full((c,), 0.5, device="cuda")
    dbeta = torch.full((c,), -0.25, device="cuda")
    gt = _t(torch, g)
    cbb.bn_backward(gt, _t(torch, xhat32), _t(torch, var32), _t(torch, gamma32), gt, dg, dbeta,
                    1e-5, ws)   # dz written over g
    torch.cuda.synchronize()
    assert_close("dz", gt.cpu().double().numpy(), dz_ref)
    assert_close("dgamma", dg.cpu().double().numpy(), dg_ref + 0.5)
    assert_close("dbeta", dbeta.cpu().double().numpy(), dbeta_ref - 0.25)


# activations whose derivative is a function of y (rounded differently in fp32), not a constant
SMOOTH_ACTS = ("logistic", "tanh", "elu", "selu", "loggy")


@pytest.mark.parametrize("act", ["linear", "leaky", "logistic", "relu", "tanh", "elu", "selu",
                                 "plse", "lhtan", "hardtan", "stair", "ramp", "relie", "loggy"])
@pytest.mark.parametrize("count", [1, 7, 4096, 1000003])
def test_act_backward_exact(act, count):
    """g = delta * act'(y): where act' is piecewise constant, one fp32 multiply by the
    page's constant, equal to the oracle's product rounded to fp32; otherwise within 1e-6."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    announce(f"act {act} {count}")
    r = np.random.default_rng(count)
    y = (1.5 * r.normal(size=count)).astype(np.float32)
    if act == "logistic":
        y = r.uniform(0, 1, size=count).astype(np.float32)
    elif act in ("tanh", "loggy"):
        y = r.uniform(-1, 1, size=count).astype(np.float32)
    elif act == "elu":
        y = np.maximum(y, -0.999).astype(np.float32)
    elif act == "stair":   # outputs on and off the integers
        y = np.where(r.uniform(size=count) < 0.5, np.round(y), y).astype(np.float32)
    y[: min(count, 3)] = 0.0                       # the kink value goes to the slope branch
    for v, at in ((1.0, 3), (-1.0, 4)):            # breakpoints of hardtan, lhtan, plse
        if count > at:
            y[at] = v
    d = r.normal(size=count).astype(np.float32)
    g = torch.empty(count, device="cuda")
    cbb.act_backward(act, 0.1, _t(torch, y), _t(torch, d), g)
    torch.cuda.synchronize()
    ref = O.act_backward(O.ACT_NAMES[act], np.float32(0.1), y, d)
    if act in SMOOTH_ACTS:
        assert_close("g", g.cpu().double().numpy(), ref, tol=1e-6)
    else:
        ref32 = (d.astype(np.float64) * O.act_backward(O.ACT_NAMES[act], np.float32(0.1), y,
                                                       np.ones_like(d)).astype(np.float32)).astype(np.float32)
        assert_exact("g", g.cpu().numpy(), ref32)


@pytest.mark.parametrize("dshape,sshape,alpha,beta", [
    ((2, 64, 52, 52), (2, 32, 26, 26), 1.0, 1.0),     # source smaller: every second row/col
    ((2, 32, 26, 26), (2, 64, 52, 52), 0.5, 2.0),     # source larger: strided targets
    ((3, 5, 9, 9), (3, 7, 9, 9), 1.0, 1.0),           # equal size, channels differ
    ((1, 8, 12, 6), (1, 8, 4, 2), 1.0, 0.25),         # ratio 3, no d_main
])
def test_shortcut_backward_resize_exact(dshape, sshape, alpha, beta):
    """Single adds of a power-of-two multiple into distinct targets: bit-exact."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    announce(f"shortcut resize {dshape} -> {sshape}")
    r = np.random.default_rng(41)
    delta = r.normal(size=dshape).astype(np.float32)
    m0 = r.normal(size=dshape).astype(np.float32)
    f0 = r.normal(size=sshape).astype(np.float32)
    use_main = beta != 0.25
    dm = _t(torch, m0) if use_main else None
    df = _t(torch, f0)
    cbb.shortcut_backward_resize(_t(torch, delta), dm, df, alpha, beta)
    torch.cuda.synchronize()
    rm, rf = O.shortcut_backward_resize(delta, m0 if use_main else None, f0, alpha, beta)
    assert_exact("d_from", df.cpu().numpy(), rf.astype(np.float32))
    if use_main:
        assert_exact("d_main", dm.cpu().numpy(), rm.astype(np.float32))


@pytest.mark.parametrize("shape", [(64, 10), (1000, 513), (3, 5, 4, 6), (16, 80, 13, 13)])
def test_softmax_backward(shape):
    """Generic softmax backward: rows (one wave each) and the strided form; in place too."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    announce(f"softmax backward {shape}")
    r = np.random.default_rng(61)
    logits = r.normal(size=shape)
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    y = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    dy = r.normal(size=shape).astype(np.float32)
    ref = O.softmax_backward(y, dy)
    dx = torch.empty(shape, device="cuda")
    cbb.softmax_backward(_t(torch, y), _t(torch, dy), dx)
    d_in = _t(torch, dy)
    cbb.softmax_backward(_t(torch, y), d_in, d_in)
    torch.cuda.synchronize()
    assert_close("dx", dx.cpu().double().numpy(), ref)
    assert_close("dx in place", d_in.cpu().double().numpy(), ref)


def test_shortcut_route_upsample_maxpool_exact():
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    announce("shortcut/route/upsample/maxpool")
    r = np.random.default_rng(3)
    d = r.normal(size=(2, 6, 5, 7)).astype(np.float32)
    m0 = r.normal(size=d.shape).astype(np.float32)
    f0 = r.normal(size=d.shape).astype(np.float32)
    dm, df = _t(torch, m0), _t(torch, f0)
    cbb.shortcut_backward(_t(torch, d), dm, df, 1.0, 1.0)
    rm, rf = O.shortcut_backward(d, m0, f0, 1.0, 1.0)
    torch.cuda.synchronize()
    assert_exact("d_main", dm.cpu().numpy(), rm.astype(np.float32))
    assert_exact("d_from", df.cpu().numpy(), rf.astype(np.float32))
    # route: 3 inputs, ragged sizes (not multiples of 4)
    dr = r.normal(size=(3, 9, 3, 3)).astype(np.float32)
    ins0 = [r.normal(size=(3, cc, 3, 3)).astype(np.float32) for cc in (2, 4, 3)]
    ins = [_t(torch, a) for a in ins0]
    cbb.route_backward(_t(torch, dr), ins)
    refs = O.route_backward(dr, ins0)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(ins, refs)):
        assert_exact(f"route{i}", a.cpu().numpy(), b.astype(np.float32))
    # route: the most inputs a call takes (8, one launch), 16-byte pieces (sizes multiples
    # of 4) and ragged sizes, each added onto nonzero deltas
    for chans, hw in (((4, 8, 4, 12, 4, 4, 8, 4), 2), ((1, 3, 2, 5, 1, 1, 2, 3), 3)):
        dr = r.normal(size=(2, sum(chans), hw, hw)).astype(np.float32)
        ins0 = [r.normal(size=(2, cc, hw, hw)).astype(np.float32) for cc in chans]
        ins = [_t(torch, a) for a in ins0]
        cbb.route_backward(_t(torch, dr), ins)
        refs = O.route_backward(dr, [a.copy() for a in ins0])
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ins, refs)):
            assert_exact(f"route{len(chans)}.{hw}.{i}", a.cpu().numpy(), b.astype(np.float32))
    # upsample with integer deltas: exact; random deltas: tolerance
    du = r.integers(-20, 20, size=(2, 3, 8, 6)).astype(np.float32)
    dsrc = torch.zeros(2, 3, 4, 3, device="cuda")
    cbb.upsample_backward(_t(torch, du), dsrc, 2)
    torch.cuda.synchronize()
    assert_exact("upsample int", dsrc.cpu().numpy(), O.upsample_backward(du, 2))
    du = r.normal(size=(8, 128, 26, 26)).astype(np.float32)
    dsrc = torch.zeros(8, 128, 13, 13, device="cuda")
    cbb.upsample_backward(_t(torch, du), dsrc, 2)
    torch.cuda.synchronize()
    assert_close("upsample", dsrc.cpu().double().numpy(), O.upsample_backward(du, 2), tol=1e-6)
    # max pool: indices from the oracle's forward; every pixel receives at most one delta
    xp = r.normal(size=(4, 5, 12, 12))
    _, idx = O.maxpool_forward(xp, 2, 2)
    dp = r.normal(size=idx.shape).astype(np.float32)
    dx = torch.full((4, 5, 12, 12), 7.0, device="cuda")   # overwritten
    cbb.maxpool_backward(_t(torch, idx, torch.int32), _t(torch, dp), dx, 2, 2)
    torch.cuda.synchronize()
    assert_exact("maxpool", dx.cpu().numpy(), O.maxpool_backward(idx, dp, (12, 12)).astype(np.float32))
    # overlapping windows (k=3, s=2): several deltas may land on one pixel
    xp = r.normal(size=(2, 3, 11, 11))
    _, idx = O.maxpool_forward(xp, 3, 2)
    dp = r.normal(size=idx.shape).astype(np.float32)
    dx = torch.empty(2, 3, 11, 11, device="cuda")
    cbb.maxpool_backward(_t(torch, idx, torch.int32), _t(torch, dp), dx, 3, 2)
    torch.cuda.synchronize()
    assert_close("maxpool overlap", dx.cpu().double().numpy(), O.maxpool_backward(idx, dp, (11, 11)),
                 tol=1e-6)


def test_fc_and_softmax_loss():
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    announce("fc / softmax loss")
    r = np.random.default_rng(4)
    for (b, din, dout) in [(64, 800, 500), (64, 500, 10), (5, 37, 3), (1, 1, 1), (70, 65, 129),
                           (3, 300, 700)]:
        x = r.normal(size=(b, din)).astype(np.float32)
        w = r.normal(size=(dout, din)).astype(np.float32)
        d = r.normal(size=(b, dout)).astype(np.float32)
        dw0 = r.normal(size=(dout, din)).astype(np.float32)
        dw, db, dx = _t(torch, dw0), torch.zeros(dout, device="cuda"), torch.zeros(b, din, device="cuda")
        cbb.fc_backward(_t(torch, x), _t(torch, w), _t(torch, d), dw, db, dx)
        torch.cuda.synchronize()
        rdw, rdb, rdx = O.fc_backward(x, w, d, dw=dw0)
        assert_close(f"fc dw {b,din,dout}", dw.cpu().double().numpy(), rdw)
        assert_close(f"fc db {b,din,dout}", db.cpu().double().numpy(), rdb)
        assert_close(f"fc dx {b,din,dout}", dx.cpu().double().numpy(), rdx)
    prob = O.softmax_forward(r.normal(size=(64, 10)) * 2).astype(np.float32)
    labels = r.integers(0, 10, size=64).astype(np.int32)
    dl = torch.empty(64, 10, device="cuda")
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    cbb.get_device_error()   # start from a clear error word
    cbb.softmax_loss_backward(_t(torch, prob), _t(torch, labels, torch.int32), dl, 1.0, bad)
    torch.cuda.synchronize()
    assert_close("dlogits", dl.cpu().double().numpy(), O.softmax_loss_backward(prob, labels), tol=1e-6)
    assert int(bad.item()) == 0
    assert cbb.get_device_error() == 0
    # out-of-range labels: row keeps prob * scale, counted once per bad sample, and the
    # GPU's error word carries the label bit until it is read
    lab2 = labels.copy()
    lab2[[3, 9]] = [10, -1]
    cbb.softmax_loss_backward(_t(torch, prob), _t(torch, lab2, torch.int32), dl, 1.0, bad)
    assert cbb.get_device_error() == cbb.DEVERR_LABEL
    assert cbb.get_device_error() == 0
    got = dl.cpu().double().numpy()
    assert int(bad.item()) == 2
    np.testing.assert_allclose(got[3], prob[3].astype(np.float64) / 64, rtol=1e-6)
    ok = np.ones(64, bool)
    ok[[3, 9]] = False
    assert_close("dlogits valid rows", got[ok], O.softmax_loss_backward(prob[ok], labels[ok]) * ok.sum() / 64,
                 tol=1e-6)


def test_launch_hook_names_each_kernel():
    """The tracing hook sees every kernel of a call, in launch order, on the call's stream
    (the one-pass act/BN kernel, then the gradient kernels)."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    announce("launch hook")
    d = cbb.conv_desc(2, 8, 12, 12, 16, 3, 1, 1, 1, "leaky")
    g = torch.Generator(device="cuda").manual_seed(5)
    rn = lambda *s: torch.randn(*s, device="cuda", generator=g)
    x, w, y, xn, dl = rn(2, 8, 12, 12), rn(16, 8, 3, 3), rn(2, 16, 12, 12), rn(2, 16, 12, 12), rn(2, 16, 12, 12)
    var, gam = torch.rand(16, device="cuda") + 0.5, torch.ones(16, device="cuda")
    dz, dw, db, dg, dx = (torch.empty_like(dl), torch.zeros_like(w), torch.zeros(16, device="cuda"),
                          torch.zeros(16, device="cuda"), torch.empty_like(x))
    ws = cbb.workspace(cbb.conv_block_workspace_size(d))
    seen = []
    stream = torch.cuda.current_stream()
    cbb.set_launch_hook(lambda name, st: seen.append((name, st)))
    try:
        cbb.conv_block_backward(d, x, w, y, xn, var, gam, dl, dz, dw, db, dg, dx, False, ws)
    finally:
        cbb.set_launch_hook(None)
    torch.cuda.synchronize()
    names = [n for n, _ in seen]
    assert names[0] == "actbn_channel", names     # a channel fits one work-group
    assert len(names) >= 3 and all(st == stream.cuda_stream for _, st in seen)
    assert any(n.startswith("conv_dw") for n in names) and any(n.startswith("conv_dx") for n in names)
    cbb.conv_block_backward(d, x, w, y, xn, var, gam, dl, dz, dw, db, dg, dx, False, ws)
    torch.cuda.synchronize()
    assert len(seen) == len(names)   # removed: no more calls


@pytest.mark.parametrize("n,batch,lr,mom,decay,off", [
    (294912, 8, 0.1, 0.9, 5e-4, 0),      # the residual 3x3 layer's weights, 16-byte path
    (1001, 64, 0.01, 0.0, 0.0, 0),       # ragged tail
    (777, 3, 0.5, 0.5, 1e-2, 1),         # misaligned: element path only
    (1, 1, 1.0, 0.9, 0.0, 0)])
def test_sgd_update(n, batch, lr, mom, decay, off):
    """The parameter update against the oracle's, over three steps with new gradients
    added onto the buffer in between (as a backward pass accumulates)."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    announce(f"sgd_update n={n} batch={batch} off={off}")
    r = np.random.default_rng(n)
    w0 = r.normal(size=n).astype(np.float32)
    wb = torch.zeros(n + off, device="cuda")
    db = torch.zeros(n + off, device="cuda")
    w, d = wb[off:], db[off:]
    w.copy_(torch.from_numpy(w0))
    rw, rd = w0.astype(np.float64), np.zeros(n)
    for step in range(3):
        g = (r.normal(size=n) * batch).astype(np.float32)
        d.add_(torch.from_numpy(g).cuda())
        rd = rd + g
        cbb.sgd_update(w, d, batch, lr, mom, decay)
        rw, rd = O.sgd_update(rw, rd.astype(np.float32), batch, lr, mom, decay)
        torch.cuda.synchronize()
        assert_close(f"w step {step}", w.cpu().double().numpy(), rw, tol=1e-6)
        assert_close(f"dw step {step}", d.cpu().double().numpy(), rd, tol=1e-6)
        rw, rd = w.cpu().double().numpy(), d.cpu().double().numpy()


@pytest.mark.parametrize("act", ["leaky", "linear"])
@pytest.mark.parametrize("n,oc,h,w", [(4, 3, 96, 104),     # one pass, 1024 threads x 10 float4
                                      (4, 3, 104, 104),    # beyond it: the streaming pass
                                      (3, 7, 9, 12)])      # one pass, 256 threads
def test_bias_only_act_stage(n, oc, h, w, act):
    """The act stage of a conv without BN: db += sum g and, with an activation, dz = g,
    on both sides of the one-pass size limit."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    announce(f"bias-only act stage {(n, oc, h, w)} {act}")
    r = np.random.default_rng(oc * h + w)
    y = r.normal(size=(n, oc, h, w)).astype(np.float32)
    d = r.normal(size=(n, oc, h, w)).astype(np.float32)
    desc = cbb.conv_desc(n, 3, h, w, oc, 1, 1, 0, 0, act)
    ws = cbb.workspace(cbb.conv_block_workspace_size(desc))
    db0 = r.normal(size=oc).astype(np.float32)
    db = _t(torch, db0)
    dz = torch.empty(n, oc, h, w, device="cuda") if act != "linear" else None
    cbb.conv_act_bn_backward(desc, _t(torch, y) if act != "linear" else None, None, None, None,
                             _t(torch, d), dz, db, None, ws)
    torch.cuda.synchronize()
    g = O.act_backward(cbb.ACT[act], 0.1, y, d)
    assert_close("db", db.cpu().double().numpy(), db0 + g.sum(axis=(0, 2, 3)), tol=1e-5)
    if dz is not None:
        assert_close("dz", dz.cpu().double().numpy(), g, tol=1e-6)
