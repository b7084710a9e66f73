"""GPU parity of the decode stack over the storage tier
(pipeline.StorageStagedStack): the predicted layers' experts are read from
per-layer stacked files (O_DIRECT) into an initially empty pinned pool, then
staged into HBM slots. Both arms (reads one token ahead, and reads just
before each group runs) must give every (token, layer) step the oracle's
result, and every held slot must hold its bundle from the file.
"""

import os

import numpy as np
import pytest

from gpu_util import announce, dev, host
from stack_check import StackChecker
from sparse_moe_decode_amd import synth

pytestmark = pytest.mark.gpu

ROLES = [dict(router=True, head=True), dict(router=False, head=True),
         dict(router=False, head=True), dict(router=False, head=False),
         dict(router=True, head=False)]


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_moe_decode_amd import api as _api
    return _api


@pytest.mark.timeout(600)
@pytest.mark.parametrize("arm,group,ram", [("prefetch", 1, 0), ("prefetch", 2, 8),
                                           ("ondemand", 1, 0)])
def test_storage_stack_matches_oracle(api, orc, tmp_path, arm, group, ram):
    import torch
    from sparse_moe_decode_amd import pipeline
    from sparse_moe_decode_amd import workloads as wl
    tier, T, seed = "35b", 4, 47
    dm = synth.dims(tier)
    E, K, L = dm["E"], dm["K"], len(ROLES)
    n_slots = 2 * K
    cons = [l for l in range(L) if not ROLES[l]["router"]]
    ci = {l: i for i, l in enumerate(cons)}
    ctx = api.Context(dm, max_tokens=1)
    bundle = ctx.bundle_bytes()
    host_pool = torch.zeros((len(cons), E, bundle), dtype=torch.uint8, pin_memory=True)
    hbm = torch.zeros((len(cons), n_slots, bundle), dtype=torch.uint8, device="cuda")
    slot_of = torch.empty((len(cons), E), dtype=torch.int32, device="cuda")
    slot_expert = torch.empty((len(cons), n_slots), dtype=torch.int32, device="cuda")
    paths = [str(tmp_path / f"layer{i}.bin") for i in range(len(cons))]
    files = {}
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
            packed = api.pack_bundles(lw["routed"], dm)
            packed.tofile(paths[ci[l]])
            files[ci[l]] = torch.from_numpy(packed).cuda()
            lay.update(routed=api.bundle_view(hbm[ci[l]].data_ptr(), dm), count=n_slots,
                       stride_q=bundle, stride_s=bundle, slot_of=slot_of[ci[l]])
        else:
            lay["routed"] = wl.tree_to_dev(lw["routed"])
        layers.append(lay)
    store = api.Store(paths, E, bundle, io_threads=8, direct=True)
    stager = api.Stager(ctx, host_pool, len(cons), n_slots, hbm, slot_of, slot_expert)
    model = api.Model(ctx, layers)
    state = api.State(dm, L)
    idx0, w0 = wl.initial_routing(tier, seed, L)
    state.route_idx[0].copy_(torch.from_numpy(idx0))
    state.route_w[0].copy_(torch.from_numpy(w0))
    toks = wl.token_inputs(tier, seed, T, rho=0.5)
    checker = StackChecker(orc, tier, seed, ROLES, list(range(L)), keep, zero_mean=True)
    pipe = pipeline.StorageStagedStack(ctx, model, state, stager, cons, L, store, host_pool,
                                       ram_bundles=ram, arm=arm, group=group)
    pipe.stage(0, after_token=False)
    prev_exec = None
    h = torch.zeros((L + 1, dm["d"]), dtype=torch.float16, device="cuda")
    for t in range(T):
        announce("storage layer_step", arm, f"group={group} ram={ram}", f"token {t}")
        h[0].copy_(torch.from_numpy(toks[t]))
        pipe.run_token(t, h)
        torch.cuda.synchronize()
        assert api.device_status(ctx) == 0
        cur, nxt = t & 1, (t + 1) & 1
        exec_idx = host(state.exec_idx[cur]).copy()
        checker.check(t, host(h).copy(), host(state.x_trace).copy(), exec_idx,
                      host(state.exec_w[cur]).copy(), prev_exec, host(state.route_idx[cur]).copy(),
                      host(state.route_w[cur]).copy(), host(state.route_idx[nxt]).copy(),
                      host(state.route_w[nxt]).copy(), host(state.head_logits).copy())
        prev_exec = exec_idx
        g_slot_exp = host(slot_expert)
        for i in range(len(cons)):
            for s, e in enumerate(g_slot_exp[i]):
                if e >= 0:
                    assert torch.equal(hbm[i, s], files[i][e]), f"t={t} layer {cons[i]} slot {s}"
    assert store.bytes_read() > 0 and pipe.loads
    print(f"{arm} group={group} ram={ram}: {checker.steps} layer-steps checked, worst error "
          f"ratio {checker.worst:.3f}, {store.bytes_read() // bundle} bundles read, "
          f"blocked {pipe.blocked_s * 1e3:.1f} ms")
    store.close()
    stager.close()
    model.close()
    ctx.close()
