"""One DSpark decode round on the GPU: gamma draft steps, the confidence head,
the prefix scheduler and verification.

The Round object owns the output tensors and the two workspaces (allocated once,
reused every round) and calls the C-ABI in order; it does no arithmetic itself.
With overlap, the confidence head and the scheduler run on a second stream while
the last position is drafted: the head at position k reads the draft token of
position k - 1 only, so the last position's token is first read by verification,
and the outputs are those of the calls in order.  It pays with the streaming draft
(one launch pair per position); the persistent draft runs every position in one
launch, and splitting that launch costs more than the overlap saves.
"""
from __future__ import annotations

import torch

from . import dsp


class Round:
    def __init__(self, R: int, gamma: int, V: int, r: int, device="cuda"):
        self.R, self.gamma, self.V, self.r = R, gamma, V, r
        dev = torch.device(device)
        i32, f32 = torch.int32, torch.float32
        self.tok = torch.zeros((R, gamma), dtype=i32, device=dev)
        self.q = torch.zeros((R, gamma), dtype=f32, device=dev)
        self.stats = torch.zeros((R, gamma, 2), dtype=torch.float64, device=dev)
        self.c = torch.zeros((R, gamma), dtype=f32, device=dev)
        self.len = torch.zeros((R,), dtype=i32, device=dev)
        self.a = torch.zeros((R, gamma), dtype=f32, device=dev)
        self.B = torch.zeros((1,), dtype=i32, device=dev)
        self.K = torch.zeros((1,), dtype=i32, device=dev)
        self.accept = torch.zeros((R, gamma), dtype=torch.int8, device=dev)
        self.n_accept = torch.zeros((R,), dtype=i32, device=dev)
        self.y = torch.zeros((R,), dtype=i32, device=dev)
        self.p = torch.zeros((R, gamma), dtype=f32, device=dev)
        # zero-filled, so that the workspaces' error words read "no give-up" even
        # before their first call
        self.ws_draft = torch.zeros(max(1, dsp.dsp_workspace_size(dsp.DSP_WS_DRAFT, R, gamma, V, r)),
                                    dtype=torch.uint8, device=dev)
        self.ws_verify = torch.zeros(max(1, dsp.dsp_workspace_size(dsp.DSP_WS_VERIFY, R, gamma, V, r)),
                                     dtype=torch.uint8, device=dev)

    def draft(self, inp, temperature, seed, rnd, stream=None, k=0, n_steps=None):
        n_steps = self.gamma - k if n_steps is None else n_steps
        dsp.dsp_draft_step(inp["base"], inp["E"], inp["W2"], inp["anchor"], self.tok, self.q,
                           self.stats, k, temperature, seed, rnd, self.ws_draft, stream,
                           n_steps=n_steps)

    def confidence(self, inp, stream=None):
        dsp.dsp_confidence(inp["h"], inp["E"], inp["anchor"], self.tok, inp["w"], inp["T"],
                           inp["offset"], self.c, stream)

    def schedule(self, inp, mode=None, tau0=None, stream=None):
        mode = inp["mode"] if mode is None else mode
        tau0 = inp["tau0"] if tau0 is None else tau0
        dsp.dsp_schedule(self.c, inp["sps"], inp["B_max"], tau0, mode, self.len, self.a, self.B,
                         stream)

    def schedule_async(self, inp, c_hist, tau0=None, stream=None):
        """The capacity-barrier scheduler: capacity from c_hist (an earlier round's
        confidences of the same requests), admission by this round's self.c."""
        tau0 = inp["tau0"] if tau0 is None else tau0
        dsp.dsp_schedule_async(self.c, c_hist, inp["sps"], inp["B_max"], tau0, self.len, self.a,
                               self.B, self.K, stream)

    def verify(self, inp, temperature, seed, rnd, stream=None, flags=dsp.DSP_PATH_AUTO):
        dsp.dsp_verify(inp["target"], inp["base"], inp["E"], inp["W2"], inp["anchor"], self.tok,
                       self.q, self.stats, self.len, self.accept, self.n_accept, self.y, self.p,
                       temperature, seed, rnd, self.ws_verify, stream, flags=flags)

    def check(self, stream=None):
        """Wait for the stream and raise DspError(DSP_ERR_TIMEOUT) if a bounded wait
        of the last draft or verify call gave up."""
        args = (self.R, self.gamma, self.V, self.r)
        dsp.dsp_workspace_status(dsp.DSP_WS_DRAFT, self.ws_draft, *args, stream=stream)
        dsp.dsp_workspace_status(dsp.DSP_WS_VERIFY, self.ws_verify, *args, stream=stream)

    def run(self, inp, temperature, seed, rnd, mode=None, tau0=None, stream=None, overlap=False):
        if not overlap or self.gamma < 2:
            self.draft(inp, temperature, seed, rnd, stream)
            self.confidence(inp, stream)
            self.schedule(inp, mode, tau0, stream)
        else:
            s = torch.cuda.current_stream() if stream is None else stream
            if not hasattr(self, "side"):
                self.side = torch.cuda.Stream(device=self.tok.device)
                self.fork, self.join = torch.cuda.Event(), torch.cuda.Event()
            self.draft(inp, temperature, seed, rnd, s, k=0, n_steps=self.gamma - 1)
            self.fork.record(s)
            self.side.wait_event(self.fork)
            self.confidence(inp, self.side)
            self.schedule(inp, mode, tau0, self.side)
            self.draft(inp, temperature, seed, rnd, s, k=self.gamma - 1, n_steps=1)
            self.join.record(self.side)
            s.wait_event(self.join)
        self.verify(inp, temperature, seed, rnd, stream)
        return self
