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


class StorageStagedStack(StagedStack):
    """StagedStack whose pinned host pool is itself filled from per-layer
    stacked files on disk (api.Store), the pages' weight tier ("The Other
    Half of the Memory Wall", §3.1: experts stay on SSD and stream by byte
    range; §5.3: reads issued one token ahead take the load time off the
    critical path).

    A bundle is read from disk when a staged set needs it and it is neither
    in the previous token's set of its layer (then it holds an HBM slot) nor
    in the RAM tier: an LRU of `ram_bundles` (layer, id) keys over the pinned
    pool (0 keeps nothing beyond what is being staged). Reads land at the
    bundle's own address in the pool, so a re-read rewrites the same bytes.

    arm "prefetch": after token t's launches are queued, each group's
    predicted sets for t+1 are read back as soon as the launch holding the
    heads that predict it has run, and its disk reads are queued at once; the
    GPU staging of each group then waits for its own reads.
    arm "ondemand": no early reads: before each group of token t runs, its
    sets are read back, its disk reads are queued and waited for, then it is
    staged and launched (group = 1 gives per-layer loads, as on-demand
    streaming does).

    Per token, blocked_s sums the time the host waited on disk reads; loads
    lists (bundles, seconds) per read ticket."""

    def __init__(self, ctx, model, state, stager, cons, n_layers, store, host_pool,
                 ram_bundles: int = 0, arm: str = "prefetch", **kw):
        super().__init__(ctx, model, state, stager, cons, n_layers, **kw)
        import collections
        assert arm in ("prefetch", "ondemand")
        self.store, self.host_pool, self.arm = store, host_pool, arm
        self.E = ctx.dims["E"]
        self.bundle = ctx.bundle_bytes()
        self.base = host_pool.data_ptr()
        self.ram = collections.OrderedDict()
        self.ram_bundles = ram_bundles
        self.prev = {}  # layer -> set of ids of the previous staged token
        self.copy_stream = torch.cuda.Stream()
        self.sets_host = torch.empty_like(state.route_idx[0], device="cpu").pin_memory()
        self.blocked_s = 0.0
        self.loads = []

    def _read_group(self, t: int, g0: int, g1: int, after: torch.cuda.Event | None):
        """Queue disk reads for token t's sets of layers [g0, g1); returns the
        ticket list."""
        st = self.state
        with torch.cuda.stream(self.copy_stream):
            if after is not None:
                self.copy_stream.wait_event(after)
            else:
                self.copy_stream.wait_stream(self.main)
            self.sets_host[g0:g1].copy_(st.route_idx[t & 1][g0:g1], non_blocking=True)
        self.copy_stream.synchronize()
        sets = self.sets_host[g0:g1].numpy()
        tickets = []
        for i, l in enumerate(range(g0, g1)):
            ids = []
            prev = self.prev.get(l, set())
            for e in sorted(set(int(v) for v in sets[i])):
                key = (l, e)
                if key in self.ram:
                    self.ram.move_to_end(key)
                    continue
                if e in prev:
                    continue
                ids.append(e)
                self.ram[key] = True
                while len(self.ram) > self.ram_bundles:
                    self.ram.popitem(last=False)
            self.prev[l] = set(int(v) for v in sets[i])
            if ids:
                li = l - self.cons[0]
                dst = [self.base + (li * self.E + e) * self.bundle for e in ids]
                tickets.append((len(ids), self.store.read(li, ids, dst)))
        return tickets

    def _wait(self, tickets):
        for n, tk in tickets:
            blocked, read = self.store.wait(tk)
            self.blocked_s += blocked
            self.loads.append((n, read))

    def stage(self, t: int, after_token: bool):
        if not after_token:  # initial staging: read everything first
            for g0, g1 in self.groups:
                self._wait(self._read_group(t, g0, g1, None))
        super().stage(t, after_token)

    def run_token(self, t: int, h):
        if self.arm == "prefetch":
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
            # predictions for t+1 become readable group by group
            pending = [self._read_group(t + 1, g0, g1, self._source(j))
                       for j, (g0, g1) in enumerate(self.groups)]
            for j, (g0, g1) in enumerate(self.groups):
                self._wait(pending[j])
                self.side.wait_event(self._source(j))
                in_use = self.sets[t & 1][g0:g1]
                api.stage_experts_n(self.stager, g0 - c0, g1 - g0, st.route_idx[(t + 1) & 1][g0:g1],
                                    in_use, side_stream=self.side, done_event=self.staged[j])
            return
        # on demand: each group's reads are queued and waited for just before it runs
        c0, c1 = self.cons[0], self.cons[-1]
        ctx, model, st, main = self.ctx, self.model, self.state, self.main
        with torch.cuda.stream(main):
            self.sets[t & 1].copy_(st.route_idx[t & 1])
        api.layer_step(ctx, model, 0, c0, st, t, h, main)
        for j, (g0, g1) in enumerate(self.groups):
            if t > 0:
                self._wait(self._read_group(t, g0, g1, None))
                self.side.wait_stream(main)
                api.stage_experts_n(self.stager, g0 - c0, g1 - g0, st.route_idx[t & 1][g0:g1],
                                    self.sets[(t - 1) & 1][g0:g1], side_stream=self.side,
                                    done_event=self.staged[j])
            main.wait_event(self.staged[j])
            api.layer_step(ctx, model, g0, g1, st, t, h[g0:], main)
        if c1 + 1 < self.L:
            api.layer_step(ctx, model, c1 + 1, self.L, st, t, h[c1 + 1:], main)
