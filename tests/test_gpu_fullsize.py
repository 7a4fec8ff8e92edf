"""Every workload at its full size, in the launch configuration the benchmark times
(same Runner, same full batch, same fp32 stand-in forward tensors), against the oracle
run on the same inputs at the same size: every output tensor, every element, within the
fp32 bound.  The oracle's full pass takes a few seconds per workload on the GPU host.
"""
import pytest

import oracle.model as M
from cnn_backward_pass_amd import synth
from gpu_common import announce, assert_close, expected_d_in, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["single_block", "lenet", "darknet53_residual", "yolov3_stem",
                                  "yolov3_head"])
def test_full_size_workload_against_oracle(name):
    torch = require_gpu()
    from cnn_backward_pass_amd.workloads import Runner
    wl = synth.WORKLOADS[name]
    announce(f"full-size {name} batch {wl.batch}")
    inp = synth.inputs(name)
    saved = synth.saved_standins(name)
    r = Runner(name, inp, saved)
    r.reset()
    r.step()
    torch.cuda.synchronize()
    got = r.results()
    del r
    ref = M.workload_backward(wl, inp, saved, inp.get("delta"))
    errs = {}
    for li, c in enumerate(wl.convs):
        errs[f"{c.name}.dw"] = assert_close(f"{c.name}.dw", got["dw"][li], ref["dw"][li])
        errs[f"{c.name}.db"] = assert_close(f"{c.name}.db", got["db"][li], ref["db"][li])
        if c.bn:
            errs[f"{c.name}.dgamma"] = assert_close(f"{c.name}.dgamma", got["dgamma"][li],
                                                    ref["dgamma"][li])
        if c.bn and got["dz"][li] is not None:   # not stored where the fused kernel forms it
            errs[f"{c.name}.dz"] = assert_close(f"{c.name}.dz", got["dz"][li], ref["dz"][li])
        if ref["d_in"][li] is not None:
            errs[f"{c.name}.dx"] = assert_close(f"{c.name}.dx", got["d_in"][li],
                                                  expected_d_in(got, ref, saved, li))
    announce("max|err|/max|ref|: " + ", ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    if name == "lenet":
        for i in range(2):
            assert_close(f"ip{i + 1}.dw", got["fc_dw"][i], ref["fc_dw"][i])
            assert_close(f"ip{i + 1}.db", got["fc_db"][i], ref["fc_db"][i])
        assert_close("d_c1", got["d_c1"], ref["d_c1"])
    elif name == "yolov3_head":
        assert_close("d_route_a", got["d_route_a"], ref["d_route_a"])
        assert_close("d_up_src", got["d_up_src"], ref["d_up_src"])
