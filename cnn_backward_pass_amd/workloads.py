"""GPU-side composition of each workload's backward pass through the C ABI.

A ``Runner`` owns the device copies of one workload's inputs and the forward
tensors a backward pass reads, the gradient buffers and the workspace, and
enqueues one full backward pass (``step``) as a sequence of ``cbb_*`` calls on
one stream, layer by layer from the loss side, in the order of Darknet's
backward_network / Caffe's Net::Backward.  All arithmetic happens in libcbb.

Buffers that receive gradients by accumulation (parameter gradients, the
shortcut/route/upsample targets, the residual block's input gradient) are
cleared by ``reset``; a step run again without a reset adds on top, which the
benchmark relies on (every step costs the same and values only scale).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import cbb, synth


def _dev(a, device, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device).contiguous()


@dataclass
class KernelWork:
    """Algorithmic work of one conv / fc gradient (for GFLOP/s and roofline accounting)."""
    name: str
    flops: float
    bytes: float


class Runner:
    def __init__(self, name: str, inputs: dict, saved: dict, device: str = "cuda"):
        self.name = name
        self._probe = None
        self._ctx = None
        self.wl = synth.WORKLOADS[name]
        self.device = device
        self.inp = inputs
        d = lambda a, dt=None: _dev(a, device, dt)
        f32 = torch.float32
        wl = self.wl
        L = saved["layers"]
        self.convs = []
        for li, c in enumerate(wl.convs):
            n = L[li]["x_in"].shape[0] if "x_in" in L[li] else wl.batch
            desc = cbb.conv_desc(n, c.in_c, c.in_h, c.in_w, c.out_c, c.k, c.stride, c.pad, c.bn,
                                 c.act, synth.LEAKY_SLOPE, synth.BN_EPS)
            ent = {"desc": desc, "x": d(L[li]["x_in"], f32), "w": d(inputs["w"][li], f32)}
            oshape = (n, c.out_c, c.out_h, c.out_w)
            ent["y"] = d(L[li]["y"], f32) if c.act != "linear" else None
            if c.bn:
                ent["xhat"] = d(L[li]["xhat"], f32)
                ent["var"] = d(L[li]["var"], f32)
                ent["gamma"] = d(L[li]["gamma"], f32)
                ent["dz"] = torch.empty(oshape, dtype=f32, device=device)
                ent["dgamma"] = torch.zeros(c.out_c, dtype=f32, device=device)
            else:
                ent["xhat"] = ent["var"] = ent["gamma"] = ent["dgamma"] = None
                ent["dz"] = None if c.act == "linear" else torch.empty(oshape, dtype=f32,
                                                                       device=device)
            ent["fused"] = cbb.conv_fused_weights_data(desc)
            # a fused dW + dX layer with an act/BN stage: dz is not stored, the fused
            # kernel forms it from delta, y and x_hat (conv_block_backward with dz=None)
            has_dx = not (name == "lenet" and li == 0)
            ent["form_dz"] = bool(ent["fused"]) and has_dx and (c.bn or c.act != "linear")
            # batch statistics on a 3x3 row-streaming layer: the dW kernel forms dz and
            # writes it for dX (the act/BN stage stops after the channel sums)
            ent["dw_forms_dz"] = bool(cbb.conv_dw_forms_dz(desc))
            ent["dw"] = torch.zeros_like(ent["w"])
            ent["db"] = torch.zeros(c.out_c, dtype=f32, device=device)
            ent["ws_bytes"] = cbb.conv_block_workspace_size(desc)
            self.convs.append(ent)
        # Consecutive blocks whose upper input-gradient kernel adds up the lower block's
        # act/BN sums (batch statistics) as it writes that block's delta: the lower
        # call takes the sums instead of reducing its delta again (cbb_block_opts).
        # The same epilogue reads the lower block's y, so it also leaves that block's
        # g = delta * act'(y) in the delta (the in-place activation step done), and
        # the lower call runs with a linear activation and reads no y.
        for e in self.convs:
            e["below"] = None
            e["sums_in"] = None
        self.d_in_act = [None] * len(self.convs)   # d_in[li] holds g of this activation
        if name not in ("lenet", "darknet53_residual"):   # layer li-1's delta is li's dx
            for li in range(1, len(self.convs)):
                lo, c_lo = self.convs[li - 1], wl.convs[li - 1]
                if c_lo.bn and cbb.conv_fuses_below_sums(
                        self.convs[li]["desc"]):
                    lo["sums_in"] = torch.empty(2 * c_lo.out_c, dtype=f32, device=device)
                    apply = c_lo.act != "linear"
                    self.convs[li]["below"] = {"sums": lo["sums_in"], "y": lo["y"],
                                               "x_norm": lo["xhat"], "act": c_lo.act,
                                               "slope": synth.LEAKY_SLOPE, "apply_act": apply}
                    if apply:
                        self.d_in_act[li] = c_lo.act
                        dl = lo["desc"]
                        lo["desc"] = cbb.conv_desc(dl.batch, c_lo.in_c, c_lo.in_h, c_lo.in_w,
                                                   c_lo.out_c, c_lo.k, c_lo.stride, c_lo.pad,
                                                   c_lo.bn, "linear", synth.LEAKY_SLOPE,
                                                   synth.BN_EPS)
                        lo["y"] = None
        self.workspace = cbb.workspace(max(e["ws_bytes"] for e in self.convs), device)
        self.batch = self.convs[0]["desc"].batch
        n = self.batch
        # inter-layer deltas: d_in[li] = gradient w.r.t. conv li's input
        self.d_in = [torch.zeros((n, c.in_c, c.in_h, c.in_w), dtype=f32, device=device)
                     for c in wl.convs]
        if name == "lenet":
            self.idx = [d(saved["pool_idx"][0], torch.int32), d(saved["pool_idx"][1], torch.int32)]
            self.relu_y = d(saved["relu_y"], f32)
            self.pool2_out = d(saved["pool2_out"], f32).reshape(n, -1).contiguous()
            self.prob = d(saved["prob"], f32)
            self.labels = d(inputs["labels"], torch.int32)
            self.fc_w = [d(w, f32) for w in inputs["fc_w"]]
            self.fc_dw = [torch.zeros_like(w) for w in self.fc_w]
            self.fc_db = [torch.zeros(w.shape[0], dtype=f32, device=device) for w in self.fc_w]
            self.dlogits = torch.empty_like(self.prob)
            self.d_relu = torch.empty_like(self.relu_y)
            self.g_relu = torch.empty_like(self.relu_y)
            c1, c2 = wl.convs
            self.d_pool2 = torch.empty((n, c2.out_c, c2.out_h // 2, c2.out_w // 2), dtype=f32,
                                       device=device)
            self.d_c2 = torch.zeros((n, c2.out_c, c2.out_h, c2.out_w), dtype=f32, device=device)
            self.d_c1 = torch.zeros((n, c1.out_c, c1.out_h, c1.out_w), dtype=f32, device=device)
            self.bad_labels = torch.zeros(1, dtype=torch.int32, device=device)
        else:
            self.delta = d(inputs["delta"], f32)
        if name == "darknet53_residual":
            self.d_main = torch.zeros_like(self.delta)
        if name == "yolov3_head":
            up_c = inputs["up_src"].shape[1]
            a_c = wl.convs[0].in_c - up_c
            hw = wl.convs[0].in_h
            self.d_route_a = torch.zeros((n, a_c, hw, hw), dtype=f32, device=device)
            self.d_up = torch.zeros((n, up_c, hw, hw), dtype=f32, device=device)
            self.d_up_src = torch.zeros((n, up_c, hw // 2, hw // 2), dtype=f32, device=device)

    # ------------------------------------------------------------------ enqueue
    def reset(self) -> None:
        for e in self.convs:
            e["dw"].zero_()
            e["db"].zero_()
            if e["dgamma"] is not None:
                e["dgamma"].zero_()
        for t in self.d_in:
            t.zero_()
        if self.name == "lenet":
            for t in self.fc_dw + self.fc_db:
                t.zero_()
            self.bad_labels.zero_()
        if self.name == "darknet53_residual":
            self.d_main.zero_()
        if self.name == "yolov3_head":
            self.d_route_a.zero_()
            self.d_up.zero_()
            self.d_up_src.zero_()

    def _conv(self, li: int, delta, dx, dx_accumulate: bool, stream) -> None:
        e = self.convs[li]
        self._ctx = self.wl.convs[li].name
        probe = self._probe
        form_dz = e["form_dz"] and dx is not None
        if probe is None or probe[0] != li or form_dz:
            # a fused-dz layer is one stage, "block" (its dz is never stored)
            target = probe is not None and probe[0] == li and probe[1] == "block"
            if target:
                probe[2](True, True)
            cbb.conv_block_backward_ex(e["desc"], e["x"], e["w"], e["y"], e["xhat"], e["var"],
                                       e["gamma"], delta, None if form_dz else e["dz"], e["dw"],
                                       e["db"], e["dgamma"], dx, dx_accumulate,
                                       sums=e["sums_in"], below=e["below"] if dx is not None
                                       else None, workspace=self.workspace, stream=stream)
            if target:
                probe[2](True, False)
            return
        # The same stages conv_block_backward runs, called one by one so that
        # events can bracket one of them ("act_bn", "dW", "dX", or "dWdX" where
        # the library computes both gradients in one fused kernel).
        _, stage, mark = probe
        dz = delta if e["dz"] is None else e["dz"]
        if e["dw_forms_dz"]:
            # the block without dx (act/BN sums, then dW forming and writing dz), then dX
            mark(stage == "actbn_dW", True)
            cbb.conv_block_backward_ex(e["desc"], e["x"], e["w"], e["y"], e["xhat"], e["var"],
                                       e["gamma"], delta, e["dz"], e["dw"], e["db"], e["dgamma"],
                                       None, False, sums=e["sums_in"], workspace=self.workspace,
                                       stream=stream)
            mark(stage == "actbn_dW", False)
            if dx is not None:
                mark(stage == "dX", True)
                cbb.conv_backward_data_ex(e["desc"], e["w"], e["dz"], dx, dx_accumulate,
                                          below=e["below"], workspace=self.workspace,
                                          stream=stream)
                mark(stage == "dX", False)
            return
        if e["sums_in"] is not None or e["below"] is not None:
            raise RuntimeError("a chained layer is timed stage by stage only on the routes "
                               "above")
        mark(stage == "act_bn", True)
        cbb.conv_act_bn_backward(e["desc"], e["y"], e["xhat"], e["var"], e["gamma"], delta,
                                 e["dz"], e["db"], e["dgamma"], self.workspace, stream)
        mark(stage == "act_bn", False)
        if dx is not None and e["fused"]:
            mark(stage == "dWdX", True)
            cbb.conv_backward_weights_data(e["desc"], e["x"], e["w"], dz, e["dw"], dx,
                                           dx_accumulate, self.workspace, stream)
            mark(stage == "dWdX", False)
            return
        mark(stage == "dW", True)
        cbb.conv_backward_weights(e["desc"], e["x"], dz, e["dw"], self.workspace, stream)
        mark(stage == "dW", False)
        if dx is not None:
            mark(stage == "dX", True)
            cbb.conv_backward_data(e["desc"], e["w"], dz, dx, dx_accumulate, self.workspace,
                                   stream)
            mark(stage == "dX", False)

    def layer_delta(self, li: int):
        """The gradient buffer a step feeds into conv layer li (its output's delta)."""
        if self.name == "lenet":
            return self.d_c2 if li == 1 else self.d_c1
        if self.name == "darknet53_residual":
            return self.d_main if li == 1 else self.d_in[1]
        return self.delta if li == len(self.convs) - 1 else self.d_in[li + 1]

    def stages(self, li: int) -> list[str]:
        """The separately timed stages of conv layer li (see step's probe)."""
        has_dx = not (self.name == "lenet" and li == 0)
        if self.convs[li]["form_dz"]:
            return ["block"]
        if self.convs[li]["dw_forms_dz"]:
            return ["actbn_dW", "dX"] if has_dx else ["actbn_dW"]
        if has_dx and self.convs[li]["fused"]:
            return ["act_bn", "dWdX"]
        return ["act_bn", "dW", "dX"] if has_dx else ["act_bn", "dW"]

    def run_stage(self, li: int, stage: str, stream=None) -> None:
        """Enqueue one stage ("act_bn", "dW" or "dX") of conv layer li on its own, on the
        buffers as they stand (for profiling; dX overwrites the layer's input gradient)."""
        e = self.convs[li]
        delta = self.layer_delta(li)
        dz = delta if e["dz"] is None else e["dz"]
        if stage == "act_bn":
            cbb.conv_act_bn_backward(e["desc"], e["y"], e["xhat"], e["var"], e["gamma"], delta,
                                     e["dz"], e["db"], e["dgamma"], self.workspace, stream)
        elif stage == "dW":
            cbb.conv_backward_weights(e["desc"], e["x"], dz, e["dw"], self.workspace, stream)
        elif stage == "dX":
            if self.name == "lenet" and li == 0:
                raise ValueError("the first LeNet conv has no input gradient")
            cbb.conv_backward_data_ex(e["desc"], e["w"], dz, self.d_in[li], False,
                                      below=e["below"], workspace=self.workspace, stream=stream)
        elif stage == "actbn_dW":
            cbb.conv_block_backward_ex(e["desc"], e["x"], e["w"], e["y"], e["xhat"], e["var"],
                                       e["gamma"], delta, e["dz"], e["dw"], e["db"], e["dgamma"],
                                       None, False, sums=e["sums_in"], workspace=self.workspace,
                                       stream=stream)
        elif stage == "block":
            cbb.conv_block_backward_ex(e["desc"], e["x"], e["w"], e["y"], e["xhat"], e["var"],
                                       e["gamma"], delta, None, e["dw"], e["db"], e["dgamma"],
                                       self.d_in[li], False, sums=e["sums_in"],
                                       below=e["below"], workspace=self.workspace,
                                       stream=stream)
        elif stage == "dWdX":
            cbb.conv_backward_weights_data(e["desc"], e["x"], e["w"], dz, e["dw"], self.d_in[li],
                                           False, self.workspace, stream)
        else:
            raise ValueError(f"unknown stage {stage!r}")

    def _dz_of(self, li: int, delta):
        e = self.convs[li]
        return delta if e["dz"] is None else e["dz"]

    def step(self, stream=None, probe=None, hook=None) -> None:
        """Enqueue one backward pass.  ``probe = (layer, stage, mark)`` runs that conv layer
        stage by stage and calls ``mark(is_target_stage, before)`` around each stage.
        ``hook(call, kernel)`` is called right after each kernel the library enqueues
        (cbb_set_launch_hook), with ``call`` the step's current call: a conv layer's name
        or the other layer's ("ip2+loss", "relu", "ip1", "pool2", "pool1", "shortcut",
        "route", "upsample")."""
        self._probe = probe
        self._ctx = None
        if hook is not None:
            cbb.set_launch_hook(lambda kernel, st: hook(self._ctx, kernel))
        try:
            self._step(stream)
        finally:
            self._probe = None
            if hook is not None:
                cbb.set_launch_hook(None)

    def _step(self, stream) -> None:
        name = self.name
        if name == "lenet":
            self._ctx = "ip2+loss"
            cbb.fc_softmax_backward(self.prob, self.labels, self.relu_y, self.fc_w[1],
                                    self.dlogits, self.fc_dw[1], self.fc_db[1], self.d_relu,
                                    1.0, self.bad_labels, stream)
            self._ctx = "relu"
            cbb.act_backward("relu", 0.0, self.relu_y, self.d_relu, self.g_relu, stream)
            self._ctx = "ip1"
            cbb.fc_backward(self.pool2_out, self.fc_w[0], self.g_relu, self.fc_dw[0],
                            self.fc_db[0], self.d_pool2.view(self.batch, -1), False, stream)
            self._ctx = "pool2"
            cbb.maxpool_backward(self.idx[1], self.d_pool2, self.d_c2, 2, 2, stream)
            self._conv(1, self.d_c2, self.d_in[1], False, stream)
            self._ctx = "pool1"
            cbb.maxpool_backward(self.idx[0], self.d_in[1], self.d_c1, 2, 2, stream)
            self._conv(0, self.d_c1, None, False, stream)
            return
        if name == "darknet53_residual":
            # shortcut: delta to the last conv's output (alpha) and to the block input (beta)
            self._ctx = "shortcut"
            cbb.shortcut_backward(self.delta, self.d_main, self.d_in[0], 1.0, 1.0, stream)
            self._conv(1, self.d_main, self.d_in[1], False, stream)
            self._conv(0, self.d_in[1], self.d_in[0], True, stream)
            return
        d = self.delta
        for li in range(len(self.convs) - 1, -1, -1):
            self._conv(li, d, self.d_in[li], False, stream)
            d = self.d_in[li]
        if name == "yolov3_head":
            self._ctx = "route"
            cbb.route_backward(self.d_in[0], [self.d_route_a, self.d_up], stream)
            self._ctx = "upsample"
            cbb.upsample_backward(self.d_up, self.d_up_src, 2, stream)

    # ------------------------------------------------------------------ results
    def results(self) -> dict:
        """Device results as float64 numpy arrays, keyed like the oracle's workload_backward."""
        h = lambda t: None if t is None else t.detach().to("cpu", torch.float64).numpy()
        out = {"dw": [h(e["dw"]) for e in self.convs], "db": [h(e["db"]) for e in self.convs],
               "dgamma": [h(e["dgamma"]) for e in self.convs],
               "d_in": [h(t) for t in self.d_in],
               # None, or the activation whose g = delta * act'(y of conv li-1) d_in[li] holds
               "d_in_act": list(self.d_in_act),
               # a layer whose dz the fused kernel forms in place stores none
               "dz": [None if e["form_dz"] else h(e["dz"]) for e in self.convs]}
        if self.name == "lenet":
            out.update(dlogits=h(self.dlogits), fc_dw=[h(t) for t in self.fc_dw],
                       fc_db=[h(t) for t in self.fc_db], d_relu=h(self.d_relu),
                       g_relu=h(self.g_relu), d_pool2=h(self.d_pool2), d_c2=h(self.d_c2),
                       d_c1=h(self.d_c1), bad_labels=int(self.bad_labels.item()))
            out["d_in"][0] = None
        elif self.name == "yolov3_head":
            out.update(d_route=h(self.d_in[0]), d_route_a=h(self.d_route_a), d_up=h(self.d_up),
                       d_up_src=h(self.d_up_src))
        else:
            out["dx"] = h(self.d_in[0])
        return out

    # ------------------------------------------------------------------ accounting
    def work(self) -> list[KernelWork]:
        """Algorithmic FLOPs and touch-once bytes of every conv / fc gradient of one step."""
        ws = []
        for li, (c, e) in enumerate(zip(self.wl.convs, self.convs)):
            n = e["desc"].batch
            macs = n * c.out_c * c.out_h * c.out_w * c.in_c * c.k * c.k
            x_b = 4.0 * n * c.in_c * c.in_h * c.in_w
            d_b = 4.0 * n * c.out_c * c.out_h * c.out_w
            w_b = 4.0 * c.out_c * c.in_c * c.k * c.k
            ws.append(KernelWork(f"{c.name}.dW", 2.0 * macs, x_b + d_b + w_b))
            has_dx = not (self.name == "lenet" and li == 0)
            if has_dx:
                ws.append(KernelWork(f"{c.name}.dX", 2.0 * macs, w_b + d_b + x_b))
            if c.bn or c.act != "linear":
                per = 16.0 if c.bn else 12.0
                ws.append(KernelWork(f"{c.name}.act_bn", 0.0, per * n * c.out_c * c.out_h * c.out_w))
        if self.name == "lenet":
            n = self.batch
            for (din, dout), nm in zip(synth.LENET_FC, ("ip1", "ip2")):
                ws.append(KernelWork(f"{nm}.dW", 2.0 * n * din * dout, 4.0 * (n * din + n * dout + din * dout)))
                ws.append(KernelWork(f"{nm}.dX", 2.0 * n * din * dout, 4.0 * (n * dout + din * dout + n * din)))
        return ws

    def flops(self) -> float:
        return sum(k.flops for k in self.work())
