"""Host-staged decode of a layer stack: expert staging overlapped with compute.

Orchestration only (launch order, streams and events); every step of the
decode and of the slot policy runs in the library's kernels.

The routed experts of the predicted layers live in a pinned host pool; each
such layer has 2K HBM slots. The prerouter head of layer l-1 at token t writes
the set layer l will execute at token t+1 ("The Other Half of the Memory
Wall", §3.2, prediction-as-routing), so that set can be staged while token t
is still running:

* side stream: for each group of predicted layers, wait for the launch of
  token t that holds the heads predicting the group, then stage the group's
  layers in one stage_experts_n call (new = predictions for t+1, in_use =
  the sets token t executes there) and record staged[group];
* main stream: one launch for the leading router layers, then one launch per
  group after waiting for staged[group], then one for the trailing router
  layers.

The persistent layer kernel takes one workgroup per compute unit and fills
it, so staging kernels could otherwise only run between its launches;
reserve_cus leaves that many compute units to them, so copies and layers run
side by side.

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
    `model`'s layers are resident. `state` is the decode state of the stack.

    group: predicted layers per launch. Layer m's prediction comes from head
    m-1, so the staging of a group for token t+1 waits for the launch of token
    t that holds the head predicting the group's last layer (for one-layer
    groups, the previous launch). Larger groups mean fewer launches and fewer
    cross-stream waits per token, and a later start for each group's staging."""

    def __init__(self, ctx: api.Context, model: api.Model, state: api.State,
                 stager: api.Stager, cons: list[int], n_layers: int,
                 main: torch.cuda.Stream | None = None, side: torch.cuda.Stream | None = None,
                 reserve_cus: int = 0, group: int = 1):
        assert cons and cons == list(range(cons[0], cons[-1] + 1)) and cons[0] >= 1
        assert cons[-1] < n_layers and group >= 1
        if reserve_cus > 0:
            cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
            model.set_grid(cus - reserve_cus)
        self.ctx, self.model, self.state, self.stager = ctx, model, state, stager
        self.cons, self.L = cons, n_layers
        self.main = main if main is not None else torch.cuda.current_stream()
        self.side = side if side is not None else torch.cuda.Stream()
        # groups [g0, g1) of predicted layers, one launch each
        self.groups = [(l, min(l + group, cons[-1] + 1)) for l in range(cons[0], cons[-1] + 1, group)]
        self.staged = [torch.cuda.Event() for _ in self.groups]
        self.launched = [torch.cuda.Event() for _ in self.groups]
        self.pre = torch.cuda.Event()  # launch of the layers before the first group
        # sets[t & 1] = routing consumed at token t, copied when token t starts
        self.sets = torch.zeros_like(state.route_idx)

    def _source(self, j: int) -> torch.cuda.Event:
        """Event of the launch holding the head that predicts group j's last
        layer (or, for a one-layer group, its only layer)."""
        g0, g1 = self.groups[j]
        x = g1 - 2 if g1 - 2 >= g0 else g0 - 1
        if x < self.cons[0]:
            return self.pre
        return self.launched[(x - self.cons[0]) // (self.groups[0][1] - self.groups[0][0])]

    def stage(self, t: int, after_token: bool):
        """Stage token t's predicted sets; after_token: wait per group for the
        launch of token t-1 that produced the predictions (else wait for
        everything already on the main stream)."""
        st = self.state
        if not after_token:
            self.side.wait_stream(self.main)
        for j, (g0, g1) in enumerate(self.groups):
            if after_token:
                self.side.wait_event(self._source(j))
            in_use = self.sets[(t - 1) & 1][g0:g1] if t > 0 else None
            api.stage_experts_n(self.stager, g0 - self.cons[0], g1 - g0, st.route_idx[t & 1][g0:g1],
                                in_use, side_stream=self.side, done_event=self.staged[j])

    def run_token(self, t: int, h):
        """Token t through all layers; h fp16 [L+1, d] (h[0] = input). Stages
        token t+1's predicted sets behind it."""
        c0, c1 = self.cons[0], self.cons[-1]
        ctx, model, st, main = self.ctx, self.model, self.state, self.main
        with torch.cuda.stream(main):
            self.sets[t & 1].copy_(st.route_idx[t & 1])
        api.layer_step(ctx, model, 0, c0, st, t, h, main)
        self.pre.record(main)
        for j, (g0, g1) in enumerate(self.groups):
            main.wait_event(self.staged[j])
            api.layer_step(ctx, model, g0, g1, st, t, h[g0:], main)
            self.launched[j].record(main)
        if c1 + 1 < self.L:
            api.layer_step(ctx, model, c1 + 1, self.L, st, t, h[c1 + 1:], main)
        self.stage(t + 1, after_token=True)
