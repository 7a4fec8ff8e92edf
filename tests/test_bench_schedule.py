"""Host logic of the benchmark's two-stream step (bench.enqueue_step), run on the CPU with
stand-ins for torch's streams and events: every workload is enqueued exactly once, on the
stream the schedule gives it, the second stream waits for the start event before the early
workloads and for the event recorded right after the FORK kernel before the late ones, and
the current stream waits for the second stream's final event."""
import contextlib

import bench


class FakeEvent:
    def __init__(self, log):
        self.log, self.where = log, None

    def record(self, stream=None):
        self.where = (stream or FakeTorch.current).name
        self.log.append(("record", self.where, id(self)))


class FakeStream:
    def __init__(self, name, log):
        self.name, self.log = name, log

    def wait_event(self, ev):
        self.log.append(("wait", self.name, id(ev)))


class FakeTorch:
    current = None

    def __init__(self):
        self.log = []
        FakeTorch.current = FakeStream("main", self.log)
        outer = self

        class Cuda:
            @staticmethod
            def current_stream():
                return FakeTorch.current

            @staticmethod
            def Event(**kw):
                return FakeEvent(outer.log)

            @staticmethod
            @contextlib.contextmanager
            def stream(s):
                prev, FakeTorch.current = FakeTorch.current, s
                try:
                    yield
                finally:
                    FakeTorch.current = prev
        self.cuda = Cuda


class FakeRunner:
    def __init__(self, name, kernels, log):
        self.name, self.kernels, self.log = name, kernels, log

    def step(self, hook=None):
        for k in self.kernels:
            self.log.append(("kernel", FakeTorch.current.name, self.name, k))
            if hook is not None:
                hook("call", k)


def _run(fork_kernel_runs=True, hook_for=None):
    torch = FakeTorch()
    fork_name, fork_kernel = bench.FORK
    runners = {}
    for n in bench.ORDER:
        ks = [f"{n}.k0", f"{n}.k1"]
        if n == fork_name:
            ks = ["sums", "dw"] + ([fork_kernel] if fork_kernel_runs else []) + ["first", "fold"]
        runners[n] = FakeRunner(n, ks, torch.log)
    side = FakeStream("side", torch.log)
    bench.enqueue_step(runners, torch, side, hook_for)
    return torch.log


def test_each_workload_once_on_its_stream():
    log = _run()
    ran = [(e[1], e[2]) for e in log if e[0] == "kernel"]
    for n in bench.ORDER:
        streams = {s for s, w in ran if w == n}
        assert streams == {"side" if n in bench.SIDE else "main"}, (n, streams)
    # every kernel of every workload exactly once
    kernels = [e[3] for e in log if e[0] == "kernel"]
    assert len(kernels) == len(set(kernels))


def test_side_waits_for_start_then_for_the_fork_kernel():
    log = _run()
    fork_name, fork_kernel = bench.FORK
    idx = {e: i for i, e in enumerate(log)}
    waits = [(i, e) for i, e in enumerate(log) if e[0] == "wait" and e[1] == "side"]
    assert len(waits) == 2
    (i0, w0), (i1, w1) = waits
    # the first wait is on an event recorded on main before anything else
    rec0 = next(i for i, e in enumerate(log) if e[0] == "record" and e[2] == w0[2])
    assert log[rec0][1] == "main" and rec0 < i0
    assert not any(e[0] == "kernel" for e in log[:rec0])
    # the early workloads follow the first wait on the side stream
    early = [i for i, e in enumerate(log) if e[0] == "kernel" and e[2] in bench.SIDE_EARLY]
    assert early and min(early) > i0 and max(early) < i1
    # the second wait is on the event recorded on main right after the FORK kernel
    rec1 = next(i for i, e in enumerate(log) if e[0] == "record" and e[2] == w1[2])
    assert log[rec1][1] == "main"
    assert log[rec1 - 1][0] == "kernel" and log[rec1 - 1][3] == fork_kernel
    late = [i for i, e in enumerate(log) if e[0] == "kernel" and e[2] in bench.SIDE_LATE]
    assert late and min(late) > i1
    # the current stream joins the side stream last
    assert log[-1][0] == "wait" and log[-1][1] == "main"
    rec_j = next(i for i, e in enumerate(log) if e[0] == "record" and e[2] == log[-1][2])
    assert log[rec_j][1] == "side" and rec_j > max(late)


def test_fork_falls_back_to_the_end_of_the_fork_workload():
    log = _run(fork_kernel_runs=False)
    fork_name, _ = bench.FORK
    waits = [e for e in log if e[0] == "wait" and e[1] == "side"]
    rec1 = next(i for i, e in enumerate(log) if e[0] == "record" and e[2] == waits[1][2])
    last_fork_kernel = max(i for i, e in enumerate(log) if e[0] == "kernel" and e[2] == fork_name)
    assert rec1 > last_fork_kernel


def test_one_stream_when_side_is_none():
    torch = FakeTorch()
    runners = {n: FakeRunner(n, [f"{n}.k"], torch.log) for n in bench.ORDER}
    bench.enqueue_step(runners, torch, None)
    assert [e[2] for e in torch.log if e[0] == "kernel"] == bench.ORDER
    assert all(e[0] == "kernel" and e[1] == "main" for e in torch.log)


def test_hooks_reach_their_workload_on_its_stream():
    seen = []

    def hook_for(name):
        if name not in ("lenet", bench.FORK[0]):
            return None
        return lambda call, kernel: seen.append((name, FakeTorch.current.name, kernel))
    _run(hook_for=hook_for)
    assert {(n, s) for n, s, _ in seen} == {("lenet", "side"), (bench.FORK[0], "main")}
    assert bench.FORK[1] in [k for n, _, k in seen if n == bench.FORK[0]]
