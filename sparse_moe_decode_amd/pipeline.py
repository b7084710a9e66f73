"""Host-staged decode of a layer stack: expert staging overlapped with compute.

Orchestration only (launch order, streams and events); every step of the
decode and of the slot policy runs in the library's kernels.

The routed experts of the predicted layers live in a pinned host pool; each
such layer has 2K HBM slots. The prerouter head of layer l-1 at token t writes
the set layer l will execute at token t+1 ("The Other Half of the Memory
Wall", §3.2, prediction-as-routing), so that set can be staged while token t
is still running:

* side stream: for each predicted layer l, wait for the launch that holds
  layer l-1 at token t, then stage_experts(l, new = prediction for t+1,
  in_use = set token t executes at l) and record staged[l];
* main stream: one launch for the leading router layers, then one launch per
  predicted layer after waiting for staged[l], then one for the trailing
  router layers.

The slots of the set in use are never overwritten, and a layer's launch
resolves its slots only after its own staging event. The in-use sets are read
from a copy taken on the main stream when token t starts (double-buffered by
token parity): the live routing buffer they come from is rewritten by token
t+1's heads, which may already run while the last layers of token t+1's
staging are still pending. Router layers have no prediction to stage ahead and
keep their pools resident in HBM.
"""

from __future__ import annotations

import torch

from . import api


class StagedStack:
    """Layers `cons` (a contiguous range) read their routed experts through
    slot pools filled by `stager` (stager layer i = cons[i]); the rest of
    `model`'s layers are resident. `state` is the decode state of the stack."""

    def __init__(self, ctx: api.Context, model: api.Model, state: api.State,
                 stager: api.Stager, cons: list[int], n_layers: int,
                 main: torch.cuda.Stream | None = None, side: torch.cuda.Stream | None = None):
        assert cons and cons == list(range(cons[0], cons[-1] + 1)) and cons[0] >= 1
        assert cons[-1] < n_layers
        self.ctx, self.model, self.state, self.stager = ctx, model, state, stager
        self.cons, self.L = cons, n_layers
        self.main = main if main is not None else torch.cuda.current_stream()
        self.side = side if side is not None else torch.cuda.Stream()
        self.staged = {l: torch.cuda.Event() for l in cons}
        self.done = {l: torch.cuda.Event() for l in range(cons[0] - 1, cons[-1])}
        # sets[t & 1] = routing consumed at token t, copied when token t starts
        self.sets = torch.zeros_like(state.route_idx)

    def stage(self, t: int, after_token: bool):
        """Stage token t's predicted sets; after_token: wait per layer for the
        launch of token t-1 that produced the prediction (else wait for
        everything already on the main stream)."""
        st = self.state
        if not after_token:
            self.side.wait_stream(self.main)
        for i, l in enumerate(self.cons):
            if after_token:
                self.side.wait_event(self.done[l - 1])
            in_use = self.sets[(t - 1) & 1][l] if t > 0 else None
            api.stage_experts(self.stager, i, st.route_idx[t & 1][l], in_use,
                              side_stream=self.side, done_event=self.staged[l])

    def run_token(self, t: int, h):
        """Token t through all layers; h fp16 [L+1, d] (h[0] = input). Stages
        token t+1's predicted sets behind it."""
        c0, c1 = self.cons[0], self.cons[-1]
        ctx, model, st, main = self.ctx, self.model, self.state, self.main
        with torch.cuda.stream(main):
            self.sets[t & 1].copy_(st.route_idx[t & 1])
        api.layer_step(ctx, model, 0, c0, st, t, h, main)
        self.done[c0 - 1].record(main)
        for l in self.cons:
            main.wait_event(self.staged[l])
            api.layer_step(ctx, model, l, l + 1, st, t, h[l:], main)
            if l in self.done:
                self.done[l].record(main)
        if c1 + 1 < self.L:
            api.layer_step(ctx, model, c1 + 1, self.L, st, t, h[c1 + 1:], main)
        self.stage(t + 1, after_token=True)
