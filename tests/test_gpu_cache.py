"""GPU parity of the cross-layer hot-expert cache (stage_experts_cached)
against the oracle's cache policy.

After every staging call the device's slot tables, entry owners and stamps
equal the oracle's (the replacement is integer bookkeeping: bit-exact), and
every owned entry holds its bundle from the host pool byte for byte. Sizes
span a single sort stage, a ragged power of two and the largest cache (4096
entries); tokens are staged in groups of layers, as the decode pipeline does.
Ids out of range and a cache too small for the staged sets raise the range
flag and leave the tables as the oracle leaves them.
"""

import numpy as np
import pytest

from gpu_util import announce, dev, host
from sparse_moe_decode_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_moe_decode_amd import api as _api
    return _api


def _setup(api, tier, L, C, seed):
    import torch
    dm = synth.dims(tier)
    E = dm["E"]
    ctx = api.Context(dm, max_tokens=1)
    bundle = ctx.bundle_bytes()
    rng = np.random.default_rng(seed)
    host_pool = torch.empty((L, E, bundle), dtype=torch.uint8, pin_memory=True)
    host_pool.copy_(torch.from_numpy(rng.integers(0, 256, size=(L, E, bundle), dtype=np.uint8)))
    cache = torch.zeros((C, bundle), dtype=torch.uint8, device="cuda")
    slot_of = torch.empty((L, E), dtype=torch.int32, device="cuda")
    owner = torch.empty(C, dtype=torch.int32, device="cuda")
    stamp = torch.empty(C, dtype=torch.int32, device="cuda")
    hc = api.HotCache(ctx, host_pool, L, C, cache, slot_of, owner, stamp)
    return dm, ctx, host_pool, cache, slot_of, owner, stamp, hc


def _check_state(orc_state, slot_of, owner, stamp, cache, host_dev, E, what):
    so, ow, st = orc_state
    assert np.array_equal(host(slot_of), so), f"{what}: slot_of"
    assert np.array_equal(host(owner), ow), f"{what}: owner"
    assert np.array_equal(host(stamp), st), f"{what}: stamp"
    import torch
    for c in np.nonzero(ow >= 0)[0]:
        l, e = divmod(int(ow[c]), E)
        assert torch.equal(cache[c], host_dev[l, e]), f"{what}: entry {c} bytes"


@pytest.mark.timeout(300)
@pytest.mark.parametrize("tier,L,C,groups,T", [("tiny", 4, 17, ((0, 1), (1, 4)), 30),
                                               ("tiny", 3, 4096, ((0, 3),), 12),
                                               ("8b", 3, 64, ((0, 2), (2, 3)), 10)])
def test_cache_policy_matches_oracle(api, orc, tier, L, C, groups, T):
    import torch
    announce("hot cache", tier, f"L={L} C={C}")
    dm, ctx, host_pool, cache, slot_of, owner, stamp, hc = _setup(api, tier, L, C, 90 + C)
    E, K = dm["E"], dm["K"]
    host_dev = host_pool.to("cuda")
    rng = np.random.default_rng(91 + C)
    seqs = [synth.markov_sets(rng, E, K, T, keep=0.5) for _ in range(L)]
    so = np.full((L, E), -1, np.int32)
    ow = np.full(C, -1, np.int32)
    st = np.full(C, -1, np.int32)
    copies = 0
    side = torch.cuda.Stream()
    for t in range(T):
        for g0, g1 in groups:
            sets = np.stack([seqs[l][t] for l in range(g0, g1)]).astype(np.int32)
            copies += len(orc.cache_policy(E, C, so, ow, st, g0, list(sets), t))
            api.stage_experts_cached(hc, g0, g1 - g0, dev(sets), t, side_stream=side)
        torch.cuda.synchronize()
        assert api.device_status(ctx) == 0
        _check_state((so, ow, st), slot_of, owner, stamp, cache, host_dev, E, f"tick {t}")
    assert hc.copies() == copies
    print(f"{tier} L={L} C={C}: {copies} bundle copies over {T} tokens")
    hc.close()
    ctx.close()


@pytest.mark.timeout(120)
def test_cache_bad_id_and_overflow(api, orc):
    announce("hot cache", "tiny", "errors")
    L, C = 2, 6  # fewer than 2 K L = 8 entries: two disjoint tokens cannot both fit
    dm, ctx, host_pool, cache, slot_of, owner, stamp, hc = _setup(api, "tiny", L, C, 92)
    E = dm["E"]
    host_dev = host_pool.to("cuda")
    so = np.full((L, E), -1, np.int32)
    ow = np.full(C, -1, np.int32)
    st = np.full(C, -1, np.int32)

    def stage(sets, tick, overflow=False):
        sets = np.array(sets, np.int32)
        if overflow:
            with pytest.raises(ValueError):
                orc.cache_policy(E, C, so, ow, st, 0, list(sets), tick)
        else:
            orc.cache_policy(E, C, so, ow, st, 0, list(sets), tick)
        api.stage_experts_cached(hc, 0, len(sets), dev(sets), tick)
        return api.device_status(ctx)

    assert stage([[0, 1], [2, 3]], 0) == 0
    api.stage_experts_cached(hc, 0, 1, dev(np.array([[0, E]], np.int32)), 1)
    assert api.device_status(ctx) == api.E0_ERR_RANGE
    _check_state((so, ow, st), slot_of, owner, stamp, cache, host_dev, E, "after a bad id")
    assert stage([[4, 5], [6, 7]], 1, overflow=True) == api.E0_ERR_RANGE
    _check_state((so, ow, st), slot_of, owner, stamp, cache, host_dev, E, "after an overflow")
    assert stage([[0, 4], [2, 5]], 1) == 0
    assert stage([[0, 6], [2, 3]], 2) == 0
    _check_state((so, ow, st), slot_of, owner, stamp, cache, host_dev, E, "after recovery")
    hc.close()
    ctx.close()
