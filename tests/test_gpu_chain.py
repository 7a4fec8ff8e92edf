"""Two consecutive conv blocks in one chain of calls (cbb_block_opts): the upper call
also produces the lower block's act/BN sums (in the stride-2 input-gradient kernel's
epilogue where it can, else by a reduction pass over dx) and the lower call takes them
instead of reducing its delta.  With below_apply_act the upper call leaves
g = dx * act'(y) of the block below in dx, and the lower call runs with a linear
activation on it.  Both blocks are compared with the oracle's blocks run one after the
other (the lower block's delta is the upper block's dx)."""
import types

import numpy as np
import pytest

import oracle.model as M
from gpu_common import announce, assert_close, require_gpu

pytestmark = pytest.mark.gpu


def _layer(c, oc, k, s, p, act, h, w):
    return types.SimpleNamespace(in_c=c, out_c=oc, k=k, stride=s, pad=p, bn=True, act=act,
                                 in_h=h, in_w=w, groups=1, dilation=1)


def _act_grad(act, y):
    """The three activation gradients the cases use, read from the output (the pages'
    leaky: 1 above zero, else the slope 0.1; relu: 1 above zero, else 0; linear: 1)."""
    if act == "linear":
        return np.ones_like(y)
    return np.where(y > 0, 1.0, 0.1 if act == "leaky" else 0.0)


def _t(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32).cuda()


# (n, lower: c_in -> c_mid act, upper: c_mid -> c_out stride, h, w, dx_accumulate, fused)
CHAIN_CASES = [
    (2, 3, 32, "leaky", 64, 2, 40, 72, False, True),    # the stem's pair: fused sums, ragged tile
    (2, 3, 32, "relu", 64, 2, 24, 64, False, True),     # run-time activation of the block below
    (1, 3, 32, "leaky", 64, 2, 16, 136, False, True),   # three tile columns
    (1, 3, 32, "leaky", 128, 2, 16, 136, False, False), # split input gradient: a reduction pass
    (2, 16, 32, "leaky", 64, 2, 20, 40, False, True),   # lower block on the general route
    (2, 3, 32, "leaky", 64, 2, 20, 36, False, False),   # output width not a multiple of 4
    (2, 3, 32, "leaky", 64, 2, 24, 40, True, True),     # the upper dx added onto a prior delta
    (2, 3, 32, "leaky", 64, 1, 12, 20, False, False),   # stride 1: a reduction pass over dx
    (1, 3, 32, "linear", 64, 2, 16, 64, False, True),   # no activation below (y not read)
]


@pytest.mark.parametrize("apply_act", [False, True])
@pytest.mark.parametrize("case", CHAIN_CASES)
def test_chained_blocks_match_oracle(case, apply_act):
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    n, c0, c1, act0, c2, s1, h, w, acc, fused = case
    announce(f"chained blocks {case} apply_act {apply_act}")
    r = np.random.default_rng(4000 + CHAIN_CASES.index(case))
    L0 = _layer(c0, c1, 3, 1, 1, act0, h, w)
    L1 = _layer(c1, c2, 3, s1, 1, "leaky", h, w)
    x0 = r.normal(size=(n, c0, h, w)).astype(np.float32)
    w0 = (r.normal(size=(c1, c0, 3, 3)) * 0.3).astype(np.float32)
    w1 = (r.normal(size=(c2, c1, 3, 3)) * 0.1).astype(np.float32)
    g0, b0 = 1.0 + 0.3 * r.normal(size=c1), r.normal(size=c1)
    g1, b1 = 1.0 + 0.3 * r.normal(size=c2), r.normal(size=c2)
    s0 = M.round_saved_to_f32(M.conv_block_forward(L0, x0, w0, gamma=g0, beta=b0))
    x1 = s0["y"].astype(np.float32)
    s1_ = M.round_saved_to_f32(M.conv_block_forward(L1, x1, w1, gamma=g1, beta=b1))
    delta1 = r.normal(size=s1_["y"].shape).astype(np.float32)
    prior = r.normal(size=x1.shape).astype(np.float32)   # dx_accumulate: the delta so far
    ref1 = M.conv_block_backward(L1, s1_, delta1, want_dx=True,
                                 dx_init=prior if acc else None)
    ref0 = M.conv_block_backward(L0, s0, ref1["dx"], want_dx=True)

    # the lower call: its own activation, or linear when dx already holds its g
    d0 = cbb.conv_desc(n, c0, h, w, c1, 3, 1, 1, 1, "linear" if apply_act else act0)
    d1 = cbb.conv_desc(n, c1, h, w, c2, 3, s1, 1, 1, "leaky")
    assert cbb.conv_fuses_below_sums(d1) == fused
    T = lambda a: _t(torch, a)
    y0 = T(s0["y"]) if act0 != "linear" else None
    xn0 = T(s0["xhat"])
    sums = torch.full((2 * c1,), float("nan"), device="cuda")   # every entry is written
    dw1, db1, dg1 = torch.zeros(c2, c1, 3, 3, device="cuda"), torch.zeros(c2, device="cuda"), \
        torch.zeros(c2, device="cuda")
    dz1 = torch.empty(s1_["y"].shape, device="cuda")
    dx1 = T(prior) if acc else torch.empty(x1.shape, device="cuda")
    ws = cbb.workspace(max(cbb.conv_block_workspace_size(d0), cbb.conv_block_workspace_size(d1)))
    seen = []
    cbb.set_launch_hook(lambda name, st: seen.append(name))
    try:
        cbb.conv_block_backward_ex(d1, T(s1_["x_in"]), T(w1), T(s1_["y"]), T(s1_["xhat"]),
                                   T(s1_["var"]), T(s1_["gamma"]), T(delta1), dz1, dw1, db1, dg1,
                                   dx1, acc, below={"sums": sums, "y": y0, "x_norm": xn0,
                                                    "act": act0, "slope": 0.1,
                                                    "apply_act": apply_act},
                                   workspace=ws)
        upper = list(seen)
        form_dz = cbb.conv_fused_weights_data(d0)
        dw0, db0, dg0 = torch.zeros(c1, c0, 3, 3, device="cuda"), torch.zeros(c1, device="cuda"), \
            torch.zeros(c1, device="cuda")
        dz0 = None if form_dz else torch.empty(s0["y"].shape, device="cuda")
        dx0 = torch.empty(x0.shape, device="cuda")
        cbb.conv_block_backward_ex(d0, T(x0), T(w0), None if apply_act else y0, xn0,
                                   T(s0["var"]), T(s0["gamma"]), dx1, dz0, dw0, db0, dg0, dx0,
                                   False, sums=sums, workspace=ws)
        lower = seen[len(upper):]
    finally:
        cbb.set_launch_hook(None)
    torch.cuda.synchronize()
    assert ("conv_dx3_s2p (act/BN sums below)" in upper) == fused, upper
    assert "actbn_reduce" not in lower and "actbn_channel" not in lower, lower
    h_ = lambda t: t.cpu().double().numpy()
    assert_close("upper dw", h_(dw1), ref1["dw"])
    assert_close("upper db", h_(db1), ref1["db"])
    assert_close("upper dgamma", h_(dg1), ref1["dgamma"])
    assert_close("upper dz", h_(dz1), ref1["dz"])
    # the sums the upper call left for the lower block: sum g, sum g * x_hat per channel
    g = ref1["dx"] * _act_grad(act0, s0["y"])
    assert_close("upper dx", h_(dx1), g if apply_act else ref1["dx"])
    want = np.stack([g.sum(axis=(0, 2, 3)), (g * s0["xhat"]).sum(axis=(0, 2, 3))], axis=1)
    assert_close("below sums", h_(sums).reshape(-1, 2), want)
    assert_close("lower dw", h_(dw0), ref0["dw"])
    assert_close("lower db", h_(db0), ref0["db"])
    assert_close("lower dgamma", h_(dg0), ref0["dgamma"])
    assert_close("lower dx", h_(dx0), ref0["dx"])
    if dz0 is not None:
        assert_close("lower dz", h_(dz0), ref0["dz"])


def test_backward_data_with_sums_below():
    """The input-gradient call alone produces the same sums as the block call."""
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    announce("backward data with sums below")
    g = torch.Generator(device="cuda").manual_seed(11)
    rn = lambda *s: torch.randn(*s, device="cuda", generator=g)
    d = cbb.conv_desc(2, 32, 24, 48, 64, 3, 2, 1, 1, "leaky")
    w, dz = rn(64, 32, 3, 3), rn(2, 64, 12, 24)
    y, xn = rn(2, 32, 24, 48), rn(2, 32, 24, 48)
    ws = cbb.workspace(cbb.conv_block_workspace_size(d))
    dx, sums = torch.empty(2, 32, 24, 48, device="cuda"), torch.empty(64, device="cuda")
    cbb.conv_backward_data_ex(d, w, dz, dx, False,
                              below={"sums": sums, "y": y, "x_norm": xn, "act": "leaky"},
                              workspace=ws)
    ref = torch.empty_like(dx)
    cbb.conv_backward_data(d, w, dz, ref, False, ws)
    torch.cuda.synchronize()
    assert torch.equal(dx, ref)    # the epilogue's sums change nothing it stores
    gf = ref * torch.where(y > 0, 1.0, 0.1)
    gg = gf.double()
    want = torch.stack([gg.sum(dim=(0, 2, 3)), (gg * xn.double()).sum(dim=(0, 2, 3))], dim=1)
    assert_close("sums", sums.view(-1, 2).double().cpu().numpy(), want.cpu().numpy())
    # dx left holding g: one fp32 product per element, as the activation step makes it
    dx2, sums2 = torch.empty_like(dx), torch.empty_like(sums)
    cbb.conv_backward_data_ex(d, w, dz, dx2, False,
                              below={"sums": sums2, "y": y, "x_norm": xn, "act": "leaky",
                                     "apply_act": True},
                              workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(dx2, gf)
    assert torch.equal(sums2, sums)
