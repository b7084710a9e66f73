"""GPU parity of layer_step: single layers of every tier and the full stacks,
64-layer launches, and top-K below the kernels' expert slots.

Runs tokens through layer_step exactly as the benchmark does (one call per
token over the layer range) and checks every (token, layer) step against the
oracle, re-anchored on the GPU's own inputs (see stack_check.py).
"""

import numpy as np
import pytest

from gpu_util import announce, dev, host
from stack_check import StackChecker
from sparse_moe_decode_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_moe_decode_amd import api as _api
    return _api


def _run_and_check(api, orc, tier, roles, seed, T, check_layers, rho=0.5, zero_mean=False,
                   path="auto", mutate=None):
    """mutate(l, lw) -> lw, if given, reshapes each layer's host weights
    before upload (the checker sees the same weights)."""
    import torch
    from sparse_moe_decode_amd import workloads as wl
    dm = synth.dims(tier)
    L = len(roles)
    layers, keep = [], {}
    for l, role in enumerate(roles):
        lw = synth.layer(seed, l, dm, role, zero_mean=zero_mean)
        if mutate is not None:
            lw = mutate(l, lw)
        if l in check_layers:
            keep[l] = lw
        if L > 2:
            announce("upload", tier, f"layer {l}/{L}")
        layers.append(dict(routed=wl.tree_to_dev(lw["routed"]), shared=wl.tree_to_dev(lw["shared"]),
                           attn=dev(lw["attn"]),
                           router=None if lw["router"] is None else dev(lw["router"]),
                           router_bias=(None if lw["router_bias"] is None
                                        else dev(lw["router_bias"])),
                           head=wl.tree_to_dev(lw["head"])))
    ctx = api.Context(dm, max_tokens=4)
    model = api.Model(ctx, layers)
    model.set_path({"auto": api.PATH_AUTO, "phases": api.PATH_PHASES, "chain": api.PATH_CHAIN,
                    "persistent": api.PATH_PERSISTENT, "flow": api.PATH_FLOW}[path])
    state = api.State(dm, L)
    idx0, w0 = wl.initial_routing(tier, seed, L)
    state.route_idx[0].copy_(torch.from_numpy(idx0))
    state.route_w[0].copy_(torch.from_numpy(w0))
    toks = wl.token_inputs(tier, seed, T, rho)
    checker = StackChecker(orc, tier, seed, roles, check_layers, keep, zero_mean)
    prev_exec = None
    h = torch.empty((L + 1, dm["d"]), dtype=torch.float16, device="cuda")
    for t in range(T):
        announce("layer_step", tier, path, f"L={L}", f"token {t}")
        h[0].copy_(torch.from_numpy(toks[t]))
        api.layer_step(ctx, model, 0, L, state, t, h)
        assert api.device_status(ctx) == 0
        cur, nxt = t & 1, (t + 1) & 1
        exec_idx = host(state.exec_idx[cur]).copy()
        checker.check(t, host(h).copy(), host(state.x_trace).copy(), exec_idx,
                      host(state.exec_w[cur]).copy(),
                      prev_exec, host(state.route_idx[cur]).copy(),
                      host(state.route_w[cur]).copy(), host(state.route_idx[nxt]).copy(),
                      host(state.route_w[nxt]).copy(),
                      host(state.head_logits).copy())
        prev_exec = exec_idx
    print(f"{tier} {path} L={L}: {checker.steps} layer-steps checked, worst error ratio "
          f"{checker.worst:.3f}, re-anchored router sets {checker.reanchored}, predictions "
          f"{checker.pred_reanchored}, x elements one ulp off {checker.x_ulp_diffs}")
    model.close()
    ctx.close()
    return checker


@pytest.mark.parametrize("tier,T,path", [("tiny", 24, "phases"), ("8b", 5, "phases"),
                                         ("35b", 5, "phases"), ("8b", 5, "chain"),
                                         ("35b", 5, "chain"), ("8b", 5, "persistent"),
                                         ("35b", 5, "persistent"), ("8b", 5, "flow"),
                                         ("35b", 5, "flow")])
def test_layer_step_two_layers(api, orc, tier, T, path):
    """Layer 0 runs its router and owns a head predicting layer 1; layer 1
    consumes that prediction and owns a head with no consumer."""
    roles = [dict(router=True, head=True), dict(router=False, head=True)]
    _run_and_check(api, orc, tier, roles, seed=31, T=T, check_layers=[0, 1], path=path)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("path", ["chain", "flow", "persistent", "phases"])
def test_layer_step_stack_35b(api, orc, path):
    """Full 35B stack (40 layers, heads on 6-38) in the benchmark's launch
    configuration; every layer-step of the first tokens is checked."""
    roles = synth.stack_roles("35b")
    _run_and_check(api, orc, "35b", roles, seed=3, T=3, check_layers=list(range(40)),
                   zero_mean=True, path=path)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("path", ["chain", "flow", "persistent", "phases"])
def test_layer_step_stack_8b(api, orc, path):
    roles = synth.stack_roles("8b")
    _run_and_check(api, orc, "8b", roles, seed=5, T=3, check_layers=list(range(24)),
                   zero_mean=True, path=path)


def _long_stack(api, n_layers, E, seed, tier="8b", K=None):
    import torch
    from sparse_moe_decode_amd import workloads as wl
    dm = synth.dims(tier, E=E) if K is None else synth.dims(tier, E=E, K=K)
    roles = ([dict(router=True, head=True)] +
             [dict(router=False, head=True) for _ in range(n_layers - 2)] +
             [dict(router=True, head=False)])
    layers, keep = [], {}
    for l, role in enumerate(roles):
        lw = synth.layer(seed, l, dm, role, zero_mean=True)
        keep[l] = lw
        if l % 8 == 0:
            announce("upload", tier, f"E={E}", f"layer {l}/{n_layers}")
        layers.append(dict(routed=wl.tree_to_dev(lw["routed"]), shared=wl.tree_to_dev(lw["shared"]),
                           attn=dev(lw["attn"]),
                           router=None if lw["router"] is None else dev(lw["router"]),
                           router_bias=(None if lw["router_bias"] is None
                                        else dev(lw["router_bias"])),
                           head=wl.tree_to_dev(lw["head"])))
    rng = synth.rng_for(seed, 10_000)
    idx0 = np.stack([synth.random_set(rng, E, dm["K"]) for _ in range(n_layers)])
    w0 = np.stack([synth.random_weights(rng, dm["K"]) for _ in range(n_layers)])
    state = api.State(dm, n_layers)
    state.route_idx[0].copy_(torch.from_numpy(idx0))
    state.route_w[0].copy_(torch.from_numpy(w0))
    return dm, roles, layers, keep, state


@pytest.mark.timeout(900)
def test_layer_step_64_layers_flow(api, orc):
    """The largest launch of the streaming kernel: 64 layers (8B shapes, 32
    experts), routers on the first and last layer, heads on all but the
    last; every layer-step of two tokens against the oracle."""
    import torch
    from sparse_moe_decode_amd import workloads as wl
    L, seed = 64, 19
    dm, roles, layers, keep, state = _long_stack(api, L, 32, seed)
    ctx = api.Context(dm, max_tokens=1)
    model = api.Model(ctx, layers)
    model.set_path(api.PATH_FLOW)
    toks = wl.token_inputs("8b", seed, 2, 0.5)
    checker = StackChecker(orc, "8b", seed, roles, list(range(L)), keep, zero_mean=True, dims=dm)
    prev_exec = None
    h = torch.empty((L + 1, dm["d"]), dtype=torch.float16, device="cuda")
    for t in range(2):
        announce("layer_step", "8b", "flow", f"L={L}", f"token {t}")
        h[0].copy_(torch.from_numpy(toks[t]))
        api.layer_step(ctx, model, 0, L, state, t, h)
        assert api.device_status(ctx) == 0
        cur, nxt = t & 1, (t + 1) & 1
        exec_idx = host(state.exec_idx[cur]).copy()
        checker.check(t, host(h).copy(), host(state.x_trace).copy(), exec_idx,
                      host(state.exec_w[cur]).copy(), prev_exec, host(state.route_idx[cur]).copy(),
                      host(state.route_w[cur]).copy(), host(state.route_idx[nxt]).copy(),
                      host(state.route_w[nxt]).copy(), host(state.head_logits).copy())
        prev_exec = exec_idx
    print(f"8b E=32 flow L={L}: {checker.steps} layer-steps checked, worst error ratio "
          f"{checker.worst:.3f}")
    model.close()
    ctx.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("path", ["chain", "persistent"])
def test_layer_step_64_layers_persistent(api, orc, path):
    """The largest launch of the persistent kernels: 64 layers (8B shapes, 32
    experts), routers on the first and last layer, heads on all but the
    last; every layer-step of two tokens against the oracle. A 65-layer range
    cannot be forced onto either kernel (E0_ERR_SHAPE) and runs per phase on
    the automatic path."""
    import torch
    from sparse_moe_decode_amd import workloads as wl
    L, seed = 64, 17
    dm, roles, layers, keep, state = _long_stack(api, L, 32, seed)
    ctx = api.Context(dm, max_tokens=1)
    model = api.Model(ctx, layers)
    pid = {"chain": api.PATH_CHAIN, "persistent": api.PATH_PERSISTENT}[path]
    model.set_path(pid)
    toks = wl.token_inputs("8b", seed, 2, 0.5)
    checker = StackChecker(orc, "8b", seed, roles, list(range(L)), keep, zero_mean=True, dims=dm)
    prev_exec = None
    h = torch.empty((L + 1, dm["d"]), dtype=torch.float16, device="cuda")
    for t in range(2):
        announce("layer_step", "8b", path, f"L={L}", f"token {t}")
        h[0].copy_(torch.from_numpy(toks[t]))
        api.layer_step(ctx, model, 0, L, state, t, h)
        assert api.device_status(ctx) == 0
        cur, nxt = t & 1, (t + 1) & 1
        exec_idx = host(state.exec_idx[cur]).copy()
        checker.check(t, host(h).copy(), host(state.x_trace).copy(), exec_idx,
                      host(state.exec_w[cur]).copy(), prev_exec, host(state.route_idx[cur]).copy(),
                      host(state.route_w[cur]).copy(), host(state.route_idx[nxt]).copy(),
                      host(state.route_w[nxt]).copy(), host(state.head_logits).copy())
        prev_exec = exec_idx
    print(f"8b E=32 {path} L={L}: {checker.steps} layer-steps checked, worst error ratio "
          f"{checker.worst:.3f}")
    model.close()

    L2 = L + 1
    dm2, roles2, layers2, keep2, state2 = _long_stack(api, L2, 32, seed + 1)
    model2 = api.Model(ctx, layers2)
    model2.set_path(pid)
    h2 = torch.zeros((L2 + 1, dm["d"]), dtype=torch.float16, device="cuda")
    announce("layer_step", "8b", f"{path} refused", f"L={L2}")
    with pytest.raises(api.E0Error) as err:
        api.layer_step(ctx, model2, 0, L2, state2, 0, h2)
    assert err.value.code == api.E0_ERR_SHAPE
    model2.set_path(api.PATH_AUTO)
    h2[0].copy_(torch.from_numpy(toks[0]))
    api.layer_step(ctx, model2, 0, L2, state2, 0, h2)
    torch.cuda.synchronize()
    assert api.device_status(ctx) == 0
    assert bool(torch.isfinite(h2.float()).all())
    model2.close()
    ctx.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("path", ["chain", "flow", "persistent", "phases"])
def test_layer_step_bitwise_deterministic(api, path):
    """Two runs of the 35B stack (40 layers, three tokens) from the same
    state give the same bits: every layer's residual, executed set and
    weights, head logits and prediction. The cross-workgroup exchanges are
    where run-to-run variation would enter."""
    import torch
    from sparse_moe_decode_amd import workloads as wl
    tier, seed, T = "35b", 47, 3
    dm = synth.dims(tier)
    roles = synth.stack_roles(tier)
    L = len(roles)
    layers = []
    for l, role in enumerate(roles):
        if l % 8 == 0:
            announce("upload", tier, f"layer {l}/{L}")
        lw = synth.layer(seed, l, dm, role, zero_mean=True)
        layers.append(dict(routed=wl.tree_to_dev(lw["routed"]), shared=wl.tree_to_dev(lw["shared"]),
                           attn=dev(lw["attn"]),
                           router=None if lw["router"] is None else dev(lw["router"]),
                           router_bias=None, head=wl.tree_to_dev(lw["head"])))
    ctx = api.Context(dm, max_tokens=1)
    model = api.Model(ctx, layers)
    model.set_path({"chain": api.PATH_CHAIN, "persistent": api.PATH_PERSISTENT,
                    "flow": api.PATH_FLOW, "phases": api.PATH_PHASES}[path])
    idx0, w0 = wl.initial_routing(tier, seed, L)
    toks = wl.token_inputs(tier, seed, T)
    runs = []
    for run in range(2):
        state = api.State(dm, L)
        state.route_idx[0].copy_(torch.from_numpy(idx0))
        state.route_w[0].copy_(torch.from_numpy(w0))
        h = torch.zeros((T, L + 1, dm["d"]), dtype=torch.float16, device="cuda")
        got = []
        for t in range(T):
            announce("layer_step determinism", tier, path, f"run {run} token {t}")
            h[t, 0].copy_(torch.from_numpy(toks[t]))
            api.layer_step(ctx, model, 0, L, state, t, h[t])
            torch.cuda.synchronize()
            assert api.device_status(ctx) == 0
            cur, nxt = t & 1, (t + 1) & 1
            got.append([host(x).copy() for x in (state.exec_idx[cur], state.exec_w[cur],
                                                  state.route_idx[nxt], state.route_w[nxt],
                                                  state.head_logits, state.x_trace)])
        got.append([host(h).view(np.uint16).copy()])
        runs.append(got)
    for a, b in zip(runs[0], runs[1]):
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{path}: runs differ"
    model.close()
    ctx.close()


@pytest.mark.parametrize("tier,K,path", [("35b", 2, "persistent"), ("35b", 3, "persistent"),
                                         ("8b", 6, "persistent"), ("35b", 3, "chain"),
                                         ("8b", 6, "chain"), ("35b", 3, "flow")])
def test_layer_step_top_k_below_slots(api, orc, tier, K, path):
    """Top-K below the kernels' expert slots (K = 2 and 3 on the five-slot
    instantiation, 6 on the nine-slot one): the slots past K hold no expert
    and the down rows skip them. Four layers (routers first and last, 32
    experts), every layer-step of three tokens against the oracle. (The
    layer-ahead slot kernel takes at most 64 shared-expert owners, so not
    K = 2 on 256 workgroups.)"""
    import torch
    from sparse_moe_decode_amd import workloads as wl
    L, seed = 4, 23 + K
    dm, roles, layers, keep, state = _long_stack(api, L, 32, seed, tier=tier, K=K)
    ctx = api.Context(dm, max_tokens=1)
    model = api.Model(ctx, layers)
    model.set_path({"chain": api.PATH_CHAIN, "persistent": api.PATH_PERSISTENT,
                    "flow": api.PATH_FLOW}[path])
    toks = wl.token_inputs(tier, seed, 3, 0.5)
    checker = StackChecker(orc, tier, seed, roles, list(range(L)), keep, zero_mean=True, dims=dm)
    prev_exec = None
    h = torch.empty((L + 1, dm["d"]), dtype=torch.float16, device="cuda")
    for t in range(3):
        announce("layer_step", tier, path, f"K={K}", f"token {t}")
        h[0].copy_(torch.from_numpy(toks[t]))
        api.layer_step(ctx, model, 0, L, state, t, h)
        assert api.device_status(ctx) == 0
        cur, nxt = t & 1, (t + 1) & 1
        exec_idx = host(state.exec_idx[cur]).copy()
        checker.check(t, host(h).copy(), host(state.x_trace).copy(), exec_idx,
                      host(state.exec_w[cur]).copy(), prev_exec, host(state.route_idx[cur]).copy(),
                      host(state.route_w[cur]).copy(), host(state.route_idx[nxt]).copy(),
                      host(state.route_w[nxt]).copy(), host(state.head_logits).copy())
        prev_exec = exec_idx
    print(f"{tier} K={K} {path}: {checker.steps} layer-steps checked, worst error ratio "
          f"{checker.worst:.3f}")
    model.close()
    ctx.close()
