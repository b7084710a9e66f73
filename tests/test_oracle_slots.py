"""Pins of the staged slot policy (CPU only): invariants over random and
Markov routing sequences. The staged set must equal the routed set ("The Other
Half of the Memory Wall", §3.2 Prediction-as-routing), only changed experts are
copied (§3.1 Executor paths, staged / incremental stack) and 2K slots suffice.
"""

import numpy as np
import pytest

from sparse_moe_decode_amd import synth


def _run(orc, E, K, seq, router_layer=False):
    n_slots = 2 * K
    slot_of = np.full(E, -1, np.int32)
    slot_expert = np.full(n_slots, -1, np.int32)
    prev = None
    total = 0
    for s in seq:
        in_use = None if router_layer else prev
        before_of = slot_of.copy()
        copies = orc.slot_policy(E, n_slots, K, slot_of, slot_expert, in_use, s)
        total += len(copies)
        # Staged set equals the routed set.
        assert all(slot_of[e] >= 0 and slot_expert[slot_of[e]] == e for e in s)
        # Exactly the misses are copied, in ascending id.
        misses = sorted(int(e) for e in s if before_of[e] < 0)
        assert [c[0] for c in copies] == misses
        # Hits keep their slot; the set in use is never evicted.
        for e in s:
            if before_of[e] >= 0:
                assert slot_of[e] == before_of[e]
        if in_use is not None:
            for e in in_use:
                assert slot_of[e] == before_of[e]
        # Tables stay consistent.
        held = slot_expert[slot_expert >= 0]
        assert np.unique(held).size == held.size
        for sl, e in enumerate(slot_expert):
            if e >= 0:
                assert slot_of[e] == sl
        assert (slot_of >= 0).sum() == held.size <= n_slots
        prev = s
    return total


@pytest.mark.parametrize("E,K", [(8, 2), (256, 4), (128, 8)])
def test_slot_policy_markov(orc, E, K):
    rng = np.random.default_rng(20 + K)
    seq = synth.markov_sets(rng, E, K, 300, keep=0.7)
    total = _run(orc, E, K, seq)
    # At most the set changes are copied (K at t=0 plus the new ids of each
    # step); fewer when an id from an older token is still resident.
    new = K + sum(len(set(seq[t]) - set(seq[t - 1])) for t in range(1, len(seq)))
    assert K <= total <= new


@pytest.mark.parametrize("E,K", [(8, 2), (16, 4)])
def test_slot_policy_random_and_router_layers(orc, E, K):
    rng = np.random.default_rng(30 + K)
    seq = [synth.random_set(rng, E, K) for _ in range(200)]
    _run(orc, E, K, seq)
    _run(orc, E, K, seq, router_layer=True)


def test_slot_policy_ascending_free_slots(orc):
    slot_of = np.full(8, -1, np.int32)
    slot_expert = np.full(4, -1, np.int32)
    assert orc.slot_policy(8, 4, 2, slot_of, slot_expert, None, [5, 2]) == [(2, 0), (5, 1)]
    # Token t uses {2, 5}; stage {5, 7}: 5 hits, 7 takes the first free slot (2).
    assert orc.slot_policy(8, 4, 2, slot_of, slot_expert, [5, 2], [5, 7]) == [(7, 2)]
    # Token uses {5, 7}; stage {1, 3}: free slots are 0 (held 2) and 3 (empty).
    assert orc.slot_policy(8, 4, 2, slot_of, slot_expert, [5, 7], [1, 3]) == [(1, 0), (3, 3)]
    assert slot_expert.tolist() == [1, 5, 7, 3]
    with pytest.raises(ValueError):
        orc.slot_policy(8, 4, 2, slot_of, slot_expert, [5, 7], [1, 9])
