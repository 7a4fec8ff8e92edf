"""cbb_conv_block_backward_noalloc (scratch memory in the library's static device
buffer, no workspace argument) against cbb_conv_block_backward with a caller's
workspace, on the same inputs, through the C ABI: three calls in a row on one GPU,
each smaller than the one before (the buffer keeps the previous call's contents),
covering the split-K input gradient, the dW kernel that forms dz, and the fused
first-layer kernel that forms dz without storing it."""
import pytest

from gpu_common import announce, assert_exact, require_gpu

pytestmark = pytest.mark.gpu

CASES = [  # n, c, h, w, oc, stride, bn, act, dz stored
    (8, 256, 26, 26, 512, 1, 1, "leaky", True),    # 58 MiB of scratch: dX split over K
    (2, 32, 40, 104, 64, 2, 1, "leaky", True),     # dW forms dz and writes it
    (2, 3, 32, 32, 16, 1, 1, "leaky", False),      # fused first layer, dz never stored
]


def _tensors(torch, desc, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    rn = lambda *s: torch.randn(*s, device="cuda", generator=g)
    n, c, h, w, oc = desc.batch, desc.in_c, desc.in_h, desc.in_w, desc.out_c
    oh, ow = desc.out_h, desc.out_w
    return dict(x=rn(n, c, h, w), w=rn(oc, c, 3, 3) * 0.05, y=rn(n, oc, oh, ow),
                x_norm=rn(n, oc, oh, ow), var=torch.rand(oc, device="cuda", generator=g) + 0.5,
                gamma=rn(oc), delta=rn(n, oc, oh, ow))


def _outputs(torch, desc, stored):
    n, c, h, w, oc = desc.batch, desc.in_c, desc.in_h, desc.in_w, desc.out_c
    z = lambda *s: torch.zeros(*s, device="cuda")
    return dict(dz=z(n, oc, desc.out_h, desc.out_w) if stored else None, dw=z(oc, c, 3, 3),
                db=z(oc), dgamma=z(oc), dx=z(n, c, h, w))


def test_noalloc_matches_workspace_entry_point_on_shrinking_calls():
    torch = require_gpu()
    from cnn_backward_pass_amd import cbb
    for k, (n, c, h, w, oc, s, bn, act, stored) in enumerate(CASES):
        announce(f"noalloc case {k}: n={n} c={c} {h}x{w} -> {oc} stride {s} dz stored {stored}")
        desc = cbb.conv_desc(n, c, h, w, oc, 3, s, 1, bn, act)
        need = cbb.conv_block_workspace_size(desc)
        assert need <= cbb.NOALLOC_SCRATCH_BYTES
        t = _tensors(torch, desc, 900 + k)
        ref, got = _outputs(torch, desc, stored), _outputs(torch, desc, stored)
        ws = cbb.workspace(need)
        args = (t["x"], t["w"], t["y"], t["x_norm"], t["var"], t["gamma"], t["delta"])
        cbb.conv_block_backward(desc, *args, ref["dz"], ref["dw"], ref["db"], ref["dgamma"],
                                ref["dx"], False, ws)
        cbb.conv_block_backward_noalloc(desc, *args, got["dz"], got["dw"], got["db"],
                                        got["dgamma"], got["dx"], False)
        torch.cuda.synchronize()
        for key in ("dz", "dw", "db", "dgamma", "dx"):
            if ref[key] is not None:
                assert_exact(f"case {k} {key}", got[key].cpu().numpy(), ref[key].cpu().numpy())
        del ws
