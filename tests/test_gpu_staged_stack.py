"""GPU parity of the host-staged decode pipeline (pipeline.StagedStack).

Predicted layers read their routed experts through HBM slot pools that
stage_experts fills from a pinned host pool on a side stream while earlier
layers of the same token still run. Per token, after the pipeline (including
the staging of the next token's sets) has drained:
  * every (token, layer) step matches the oracle, re-anchored on the GPU's
    own inputs (stack_check.py), exactly as for resident pools;
  * each predicted layer's slot tables equal the oracle slot policy run on
    (new = next token's prediction, in use = this token's set), bit-exact;
  * every held slot holds its expert's host bundle, byte for byte.
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


# router + head, three predicted layers (the last without a head), router
ROLES = [dict(router=True, head=True), dict(router=False, head=True),
         dict(router=False, head=True), dict(router=False, head=False),
         dict(router=True, head=False)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tier,T,reserve,group,quant", [("35b", 5, 0, 1, 0), ("8b", 4, 0, 1, 0),
                                                        ("35b", 4, 16, 2, 0), ("8b", 4, 8, 3, 0),
                                                        ("35b", 3, 0, 2, 1)])
def test_staged_stack_matches_oracle(api, orc, tier, T, reserve, group, quant):
    """reserve > 0 runs the persistent kernel on fewer workgroups than compute
    units (staging copies then run beside the layers); group = predicted
    layers per launch; quant = 1 stages affine bundles (scales, then biases)
    and runs the layers one kernel per phase."""
    dm = synth.dims(tier, quant=1) if quant else synth.dims(tier)
    _staged_run(api, orc, tier, ROLES, dm, T, reserve, group, quant)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("path", ["chain", "persistent", "flow"])
def test_staged_stack_bench_shape(api, orc, path):
    """The benchmark's staged configuration: the 35B stack's 40 layers (own
    routers on 0-6 and 39, 32 predicted layers staged through slots),
    16 predicted layers per launch and 32 compute units left to the copies,
    with each layer kernel forced; 32 experts per layer instead of 256 keep
    the host pool small, every other shape is the 35B tier's. Every
    layer-step of three tokens against the oracle."""
    dm = synth.dims("35b", E=32)
    _staged_run(api, orc, "35b", synth.stack_roles("35b"), dm, 3, 32, 16, 0, seed=45, path=path)


def _staged_run(api, orc, tier, roles, dm, T, reserve, group, quant, seed=41, path="auto"):
    import torch
    from sparse_moe_decode_amd import pipeline
    from sparse_moe_decode_amd import workloads as wl
    E, K, L = dm["E"], dm["K"], len(roles)
    n_slots = 2 * K
    cons = [l for l in range(L) if not roles[l]["router"]]
    ci = {l: i for i, l in enumerate(cons)}
    ctx = api.Context(dm, max_tokens=1)
    bundle = ctx.bundle_bytes()
    host_pool = torch.empty((len(cons), E, bundle), dtype=torch.uint8, pin_memory=True)
    hbm = torch.zeros((len(cons), n_slots, bundle), dtype=torch.uint8, device="cuda")
    slot_of = torch.empty((len(cons), E), dtype=torch.int32, device="cuda")
    slot_expert = torch.empty((len(cons), n_slots), dtype=torch.int32, device="cuda")
    layers, keep = [], {}
    for l, role in enumerate(roles):
        if l % 8 == 0 or L < 8:
            announce("upload", tier, f"E={E}", f"layer {l}/{L}")
        lw = synth.layer(seed, l, dm, role, zero_mean=True)
        keep[l] = lw
        lay = dict(shared=wl.tree_to_dev(lw["shared"]), attn=dev(lw["attn"]),
                   router=None if lw["router"] is None else dev(lw["router"]),
                   router_bias=None if lw["router_bias"] is None else dev(lw["router_bias"]),
                   head=wl.tree_to_dev(lw["head"]))
        if l in ci:
            host_pool[ci[l]].copy_(torch.from_numpy(api.pack_bundles(lw["routed"], dm)))
            lay.update(routed=api.bundle_view(hbm[ci[l]].data_ptr(), dm), count=n_slots,
                       stride_q=bundle, stride_s=bundle, slot_of=slot_of[ci[l]])
        else:
            lay["routed"] = wl.tree_to_dev(lw["routed"])
        layers.append(lay)
    host_dev = host_pool.to("cuda")
    stager = api.Stager(ctx, host_pool, len(cons), n_slots, hbm, slot_of, slot_expert)
    model = api.Model(ctx, layers)
    model.set_path({"auto": api.PATH_AUTO, "chain": api.PATH_CHAIN,
                    "persistent": api.PATH_PERSISTENT, "flow": api.PATH_FLOW}[path])
    state = api.State(dm, L)
    rng = synth.rng_for(seed, 10_000)
    idx0 = np.stack([synth.random_set(rng, E, K) for _ in range(L)])
    w0 = np.stack([synth.random_weights(rng, K) for _ in range(L)])
    state.route_idx[0].copy_(torch.from_numpy(idx0))
    state.route_w[0].copy_(torch.from_numpy(w0))
    toks = wl.token_inputs(tier, seed, T, rho=0.5)  # sets change between tokens: copies happen
    checker = StackChecker(orc, tier, seed, roles, list(range(L)), keep, zero_mean=True,
                           quant=quant, dims=dm)
    pipe = pipeline.StagedStack(ctx, model, state, stager, cons, L, reserve_cus=reserve,
                                group=group)

    o_slot_of = np.full((len(cons), E), -1, np.int32)
    o_slot_exp = np.full((len(cons), n_slots), -1, np.int32)
    copies = 0
    for i, l in enumerate(cons):
        copies += len(orc.slot_policy(E, n_slots, K, o_slot_of[i], o_slot_exp[i], None, idx0[l]))
    pipe.stage(0, after_token=False)
    prev_exec = None
    h = torch.zeros((L + 1, dm["d"]), dtype=torch.float16, device="cuda")
    for t in range(T):
        announce("staged layer_step", tier, path,
                 f"L={L} E={E} reserve={reserve} group={group} quant={quant}", f"token {t}")
        h[0].copy_(torch.from_numpy(toks[t]))
        pipe.run_token(t, h)
        torch.cuda.synchronize()
        assert api.device_status(ctx) == 0
        cur, nxt = t & 1, (t + 1) & 1
        exec_idx = host(state.exec_idx[cur]).copy()
        route_cur = host(state.route_idx[cur]).copy()
        route_nxt = host(state.route_idx[nxt]).copy()
        checker.check(t, host(h).copy(), host(state.x_trace).copy(), exec_idx,
                      host(state.exec_w[cur]).copy(), prev_exec, route_cur,
                      host(state.route_w[cur]).copy(), route_nxt,
                      host(state.route_w[nxt]).copy(), host(state.head_logits).copy())
        prev_exec = exec_idx
        # the staging of token t+1 has run: compare with the oracle slot policy
        for i, l in enumerate(cons):
            copies += len(orc.slot_policy(E, n_slots, K, o_slot_of[i], o_slot_exp[i],
                                          route_cur[l], route_nxt[l]))
        g_slot_of, g_slot_exp = host(slot_of), host(slot_expert)
        assert np.array_equal(g_slot_of, o_slot_of), f"slot_of differs after token {t}"
        assert np.array_equal(g_slot_exp, o_slot_exp), f"slot_expert differs after token {t}"
        for i, l in enumerate(cons):
            assert np.all(g_slot_of[i][route_nxt[l]] >= 0)
            for s, e in enumerate(g_slot_exp[i]):
                if e >= 0:
                    assert torch.equal(hbm[i, s], host_dev[i, e]), f"t={t} l={l} slot {s}"
    assert stager.copies() == copies, "bundle copies counted by the stager"
    print(f"{tier} staged {path} L={L} E={E}: {checker.steps} layer-steps checked, worst error "
          f"ratio {checker.worst:.3f}, {copies} bundle copies, re-anchored {checker.reanchored}")
    stager.close()
    model.close()
    ctx.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tier,T,C,group", [("35b", 5, 24, 1), ("8b", 4, 64, 2)])
def test_staged_stack_through_hot_cache(api, orc, tier, T, C, group):
    """The predicted layers read their experts from one cross-layer hot cache
    of C entries (C = 2K x 3 layers is the smallest that always fits at
    35B). Per token: every layer-step matches the oracle; the cache's tables
    equal the oracle's cache policy run on the same sets, groups and ticks;
    every owned entry holds its bundle; the copy count matches."""
    import torch
    from sparse_moe_decode_amd import pipeline
    from sparse_moe_decode_amd import workloads as wl
    dm = synth.dims(tier)
    E, K, L = dm["E"], dm["K"], len(ROLES)
    seed = 43
    cons = [l for l in range(L) if not ROLES[l]["router"]]
    ci = {l: i for i, l in enumerate(cons)}
    ctx = api.Context(dm, max_tokens=1)
    bundle = ctx.bundle_bytes()
    host_pool = torch.empty((len(cons), E, bundle), dtype=torch.uint8, pin_memory=True)
    cache = torch.zeros((C, bundle), dtype=torch.uint8, device="cuda")
    slot_of = torch.empty((len(cons), E), dtype=torch.int32, device="cuda")
    owner = torch.empty(C, dtype=torch.int32, device="cuda")
    stamp = torch.empty(C, dtype=torch.int32, device="cuda")
    view = api.bundle_view(cache.data_ptr(), dm)
    layers, keep = [], {}
    for l, role in enumerate(ROLES):
        announce("upload", tier, f"layer {l}/{L}")
        lw = synth.layer(seed, l, dm, role, zero_mean=True)
        keep[l] = lw
        lay = dict(shared=wl.tree_to_dev(lw["shared"]), attn=dev(lw["attn"]),
                   router=None if lw["router"] is None else dev(lw["router"]),
                   router_bias=None if lw["router_bias"] is None else dev(lw["router_bias"]),
                   head=wl.tree_to_dev(lw["head"]))
        if l in ci:
            host_pool[ci[l]].copy_(torch.from_numpy(api.pack_bundles(lw["routed"], dm)))
            lay.update(routed=view, count=C, stride_q=bundle, stride_s=bundle,
                       slot_of=slot_of[ci[l]])
        else:
            lay["routed"] = wl.tree_to_dev(lw["routed"])
        layers.append(lay)
    host_dev = host_pool.to("cuda")
    hc = api.HotCache(ctx, host_pool, len(cons), C, cache, slot_of, owner, stamp)
    model = api.Model(ctx, layers)
    state = api.State(dm, L)
    idx0, w0 = wl.initial_routing(tier, seed, L)
    state.route_idx[0].copy_(torch.from_numpy(idx0))
    state.route_w[0].copy_(torch.from_numpy(w0))
    toks = wl.token_inputs(tier, seed, T, rho=0.5)
    checker = StackChecker(orc, tier, seed, ROLES, list(range(L)), keep, zero_mean=True)
    pipe = pipeline.StagedStack(ctx, model, state, hc, cons, L, group=group)
    so = np.full((len(cons), E), -1, np.int32)
    ow = np.full(C, -1, np.int32)
    st = np.full(C, -1, np.int32)
    copies = 0

    def oracle_stage(routes, tick):
        nonlocal copies
        for g0, g1 in pipe.groups:
            copies += len(orc.cache_policy(E, C, so, ow, st, g0 - cons[0],
                                           [routes[l] for l in range(g0, g1)], tick))

    oracle_stage(idx0, 0)
    pipe.stage(0, after_token=False)
    prev_exec = None
    h = torch.zeros((L + 1, dm["d"]), dtype=torch.float16, device="cuda")
    for t in range(T):
        announce("cached layer_step", tier, f"C={C} group={group}", f"token {t}")
        h[0].copy_(torch.from_numpy(toks[t]))
        pipe.run_token(t, h)
        torch.cuda.synchronize()
        assert api.device_status(ctx) == 0
        cur, nxt = t & 1, (t + 1) & 1
        exec_idx = host(state.exec_idx[cur]).copy()
        route_nxt = host(state.route_idx[nxt]).copy()
        checker.check(t, host(h).copy(), host(state.x_trace).copy(), exec_idx,
                      host(state.exec_w[cur]).copy(), prev_exec, host(state.route_idx[cur]).copy(),
                      host(state.route_w[cur]).copy(), route_nxt,
                      host(state.route_w[nxt]).copy(), host(state.head_logits).copy())
        prev_exec = exec_idx
        oracle_stage(route_nxt, t + 1)
        assert np.array_equal(host(slot_of), so), f"slot_of after token {t}"
        assert np.array_equal(host(owner), ow), f"owner after token {t}"
        assert np.array_equal(host(stamp), st), f"stamp after token {t}"
        for c in np.nonzero(ow >= 0)[0]:
            i, e = divmod(int(ow[c]), E)
            assert torch.equal(cache[c], host_dev[i, e]), f"t={t} entry {c}"
    assert hc.copies() == copies
    print(f"{tier} cached L={L} C={C}: {checker.steps} layer-steps checked, worst error ratio "
          f"{checker.worst:.3f}, {copies} bundle copies")
    hc.close()
    model.close()
    ctx.close()
