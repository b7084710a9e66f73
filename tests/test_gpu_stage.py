"""GPU parity of expert staging (pinned-host pool -> HBM slot pool).

stage_experts runs the slot policy on the device and copies the missing
expert bundles from pinned host memory into HBM slots on a side stream. Over
a Markov-correlated sequence of predicted sets it is checked against the
oracle's slot policy: slot tables bit-exact, every slot's bytes equal to its
expert's host bundle, the staged set equal to the routed set. A decode through
the staged slots, launched on the main stream after waiting for the staging
event, matches the oracle on the id-indexed pool.
"""

import numpy as np
import pytest

from gpu_util import announce, dev, dev_tree, f16_to_f64, host
from helpers import assert_out_close
from sparse_moe_decode_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_moe_decode_amd import api as _api
    return _api


@pytest.mark.timeout(300)
@pytest.mark.parametrize("tier,T", [("8b", 10), ("35b", 10)])
def test_stage_experts_matches_slot_policy(api, orc, tier, T):
    import torch
    dm = synth.dims(tier)
    E, K, L = dm["E"], dm["K"], 2
    n_slots = 2 * K
    announce("stage_experts", tier, f"L={L} slots={n_slots} T={T}")
    ctx = api.Context(dm, max_tokens=1)
    bundle = ctx.bundle_bytes()
    pools = [synth.routed_pool(synth.rng_for(50, l), dm) for l in range(L)]
    host_pool = torch.empty((L, E, bundle), dtype=torch.uint8, pin_memory=True)
    for l in range(L):
        packed = api.pack_bundles(pools[l], dm)
        assert packed.shape == (E, bundle)
        host_pool[l].copy_(torch.from_numpy(packed))
    host_dev = host_pool.to("cuda")  # reference copy for byte checks
    hbm = torch.zeros((L, n_slots, bundle), dtype=torch.uint8, device="cuda")
    slot_of = torch.empty((L, E), dtype=torch.int32, device="cuda")
    slot_expert = torch.empty((L, n_slots), dtype=torch.int32, device="cuda")
    st = api.Stager(ctx, host_pool, L, n_slots, hbm, slot_of, slot_expert)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    ev = torch.cuda.Event()
    sh = synth.shared_expert(synth.rng_for(51), dm)
    dsh = dev_tree(sh)

    o_slot_of = np.full((L, E), -1, np.int32)
    o_slot_exp = np.full((L, n_slots), -1, np.int32)
    rng = np.random.default_rng(52)
    sets = [synth.markov_sets(synth.rng_for(53, l), E, K, T, keep=0.7) for l in range(L)]
    copies = 0
    for t in range(T):
        for l in range(L):
            new = sets[l][t].astype(np.int32)
            in_use = sets[l][t - 1].astype(np.int32) if t > 0 else None
            dnew = dev(new)
            diu = dev(in_use) if in_use is not None else None
            side.wait_stream(main)  # the id buffers were written on the main stream
            api.stage_experts(st, l, dnew, diu, side_stream=side, done_event=ev)
            copies += len(orc.slot_policy(E, n_slots, K, o_slot_of[l], o_slot_exp[l], in_use,
                                          new))
            # decode through the staged slots once the copies are done
            main.wait_event(ev)
            x = rng.normal(size=(1, dm["d"])).astype(np.float16)
            w = synth.random_weights(rng, K)[None]
            view = api.bundle_view(hbm[l].data_ptr(), dm)
            y = api.moe_int4_decode(ctx, view, dev(x), dev(new[None]), dev(w), shared=dsh,
                                    slot_of=slot_of[l], count=n_slots, stride=bundle)
            ref = orc.moe_decode(dm, pools[l], sh, x[0], new, w[0].astype(np.float64))
            assert_out_close(f16_to_f64(y)[0], ref, f"{tier} t={t} l={l}")
        torch.cuda.synchronize()
        assert api.device_status(ctx) == 0
        g_slot_of, g_slot_exp = host(slot_of), host(slot_expert)
        assert np.array_equal(g_slot_of, o_slot_of), f"slot_of differs at t={t}"
        assert np.array_equal(g_slot_exp, o_slot_exp), f"slot_expert differs at t={t}"
        for l in range(L):
            # staged set == routed set, and every held slot holds its bundle
            assert np.all(g_slot_of[l][sets[l][t]] >= 0)
            for s, e in enumerate(g_slot_exp[l]):
                if e >= 0:
                    assert torch.equal(hbm[l, s], host_dev[l, e]), f"t={t} l={l} slot {s}"
    assert st.copies() == copies, "bundle copies counted by the stager"
    print(f"{tier}: {T} tokens x {L} layers staged, {copies} bundle copies")
    st.close()


@pytest.mark.timeout(120)
def test_stage_event_orders_the_decode(api, orc):
    """The done event really orders work: the side stream is held back by a
    bounded sleep kernel before staging, the main stream only waits on the
    event, and the decode through the slots still sees the staged bundles."""
    import torch
    if not hasattr(torch.cuda, "_sleep"):
        pytest.skip("torch.cuda._sleep unavailable")
    dm = synth.dims("35b")
    E, K = dm["E"], dm["K"]
    n_slots = 2 * K
    announce("stage_experts", "35b", "event ordering")
    ctx = api.Context(dm, max_tokens=1)
    bundle = ctx.bundle_bytes()
    pool = synth.routed_pool(synth.rng_for(60), dm)
    host_pool = torch.empty((1, E, bundle), dtype=torch.uint8, pin_memory=True)
    host_pool[0].copy_(torch.from_numpy(api.pack_bundles(pool, dm)))
    hbm = torch.zeros((1, n_slots, bundle), dtype=torch.uint8, device="cuda")
    slot_of = torch.empty((1, E), dtype=torch.int32, device="cuda")
    slot_expert = torch.empty((1, n_slots), dtype=torch.int32, device="cuda")
    st = api.Stager(ctx, host_pool, 1, n_slots, hbm, slot_of, slot_expert)
    side, main = torch.cuda.Stream(), torch.cuda.current_stream()
    rng = np.random.default_rng(61)
    new = synth.random_set(rng, E, K)
    x = rng.normal(size=(1, dm["d"])).astype(np.float16)
    w = synth.random_weights(rng, K)[None]
    dnew, dx, dw, didx = dev(new), dev(x), dev(w), dev(new[None])
    torch.cuda.synchronize()
    ev = torch.cuda.Event()
    with torch.cuda.stream(side):
        torch.cuda._sleep(40_000_000)  # ~20 ms of spinning, then it exits
    api.stage_experts(st, 0, dnew, None, side_stream=side, done_event=ev)
    main.wait_event(ev)
    view = api.bundle_view(hbm[0].data_ptr(), dm)
    y = api.moe_int4_decode(ctx, view, dx, didx, dw, slot_of=slot_of[0], count=n_slots,
                            stride=bundle)
    torch.cuda.synchronize()
    assert api.device_status(ctx) == 0
    ref = orc.moe_decode(dm, pool, None, x[0], new, w[0].astype(np.float64))
    assert_out_close(f16_to_f64(y)[0], ref, "decode after the staging event")
    st.close()
