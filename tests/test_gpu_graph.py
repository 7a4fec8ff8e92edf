"""A backward step captured as a HIP graph (torch.cuda.CUDAGraph) and replayed gives
the eager step's results bit for bit, replay after replay, with eager work and
synchronisations between the replays (the library issues no memset or allocation
inside a step, so the graph holds kernel nodes only)."""
import pytest

from cnn_backward_pass_amd import synth
from gpu_common import announce, assert_exact, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,batch", [("single_block", 2), ("lenet", 64),
                                        ("darknet53_residual", 1), ("yolov3_stem", 1),
                                        ("yolov3_head", 1)])
def test_graph_replay_matches_eager(name, batch):
    torch = require_gpu()
    from cnn_backward_pass_amd.workloads import Runner
    announce(f"graph replay {name} batch {batch}")
    inp = synth.inputs(name, scale_batch=batch)
    saved = synth.saved_standins(name, scale_batch=batch)
    r = Runner(name, inp, saved)
    r.reset()
    r.step()
    torch.cuda.synchronize()
    eager = r.results()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        g.capture_begin()
        r.step()
        g.capture_end()
    torch.cuda.synchronize()
    for rep in range(3):
        r.reset()            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = r.results()
        for key in ("dw", "db", "dgamma", "d_in", "dz"):
            for a, b in zip(eager[key], got[key]):
                if a is not None:
                    assert_exact(f"replay {rep} {key}", b, a)
        r.step()             # an eager step after the replay (accumulates on top)
        torch.cuda.synchronize()
