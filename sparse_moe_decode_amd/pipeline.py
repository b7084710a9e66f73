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
    slot pools filled by `stager` (stager layer i = cons[i]), or through the
    entries of a cross-layer hot cache when `stager` is an api.HotCache; the
    rest of `model`'s layers are resident. `state` is the decode state of the
    stack.

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
        cached = isinstance(self.stager, api.HotCache)
        for j, (g0, g1) in enumerate(self.groups):
            if after_token:
                self.side.wait_event(self._source(j))
            if cached:  # the cache keeps the running token's entries by their stamps
                api.stage_experts_cached(self.stager, g0 - self.cons[0], g1 - g0,
                                         st.route_idx[t & 1][g0:g1], t, side_stream=self.side,
                                         done_event=self.staged[j])
                continue
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


class PrefillStack:
    """Prefill-sized batches through layers whose routed experts live in a
    pinned host pool, with layer-ahead whole-layer staging ("The Other Half of
    the Memory Wall", §3.1 Executor paths, whole-layer: a prefill loads every
    expert of a layer at once, and the load of the next layer overlaps the
    current layer's GPU work).

    Two HBM layer buffers alternate: while layer l runs moe_int4_decode on
    buffer l % 2 (main stream), stage_layer copies layer l+1's bundles into
    the other buffer (side stream, DMA), after the main stream has finished
    with it (layer l-1). Events order every copy against the kernels that read
    its buffer.

    host_pool: pinned uint8 [L, E * bundle]; shared: per-layer shared-expert
    dicts of device tensors (resident) or None."""

    def __init__(self, ctx: api.Context, host_pool, shared: list,
                 main: torch.cuda.Stream | None = None, side: torch.cuda.Stream | None = None):
        self.ctx, self.host, self.shared = ctx, host_pool, shared
        self.L = host_pool.shape[0]
        self.bundle = ctx.bundle_bytes()
        assert host_pool.shape[1] == ctx.dims["E"] * self.bundle and host_pool.is_pinned()
        self.hbm = torch.empty((2, host_pool.shape[1]), dtype=torch.uint8, device="cuda")
        self.views = [api.bundle_view(self.hbm[i].data_ptr(), ctx.dims) for i in range(2)]
        self.main = main if main is not None else torch.cuda.current_stream()
        self.side = side if side is not None else torch.cuda.Stream()
        self.staged = [torch.cuda.Event() for _ in range(2)]
        self.free = [torch.cuda.Event() for _ in range(2)]

    def _stage(self, l: int):
        buf = l % 2
        self.side.wait_event(self.free[buf])
        api.stage_layer(self.ctx, self.host[l], self.hbm[buf], stream=self.side,
                        done_event=self.staged[buf])

    def run(self, x, idx, w, y):
        """Layer l maps x[l] (fp16 [B, d], normed) with routing idx[l], w[l]
        ([B, K]) to y[l]; all on the GPU."""
        for i in range(2):  # both buffers start free
            self.free[i].record(self.main)
        self._stage(0)
        for l in range(self.L):
            buf = l % 2
            if l + 1 < self.L:
                self._stage(l + 1)
            self.main.wait_event(self.staged[buf])
            api.moe_int4_decode(self.ctx, self.views[buf], x[l], idx[l], w[l], y=y[l],
                                shared=self.shared[l], stride=self.bundle, stream=self.main)
            self.free[buf].record(self.main)
