"""Pins of the cross-layer hot-expert cache policy (oracle.cache_policy), CPU
only: a hand-worked trace from the pages' LRU reading (tests/golden), a
textbook LRU (ordered dict, move to the back on use, evict the front) on
single-layer single-expert sequences, and invariants over multi-layer Markov
routing: staged sets are resident, the running token's entries are never
taken, misses are copied once in (layer, id) order, the entries taken are
the least recently staged free ones, and a cache holding every bundle ever
used copies each exactly once.
"""

import collections
import json
import os

import numpy as np
import pytest

from sparse_moe_decode_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hot_cache_lru.json")


def _fresh(L, E, C):
    return (np.full((L, E), -1, np.int32), np.full(C, -1, np.int32), np.full(C, -1, np.int32))


def test_hand_worked_trace(orc):
    g = json.load(open(GOLDEN))
    so, ow, st = _fresh(g["L"], g["E"], g["C"])
    for t, s in enumerate(g["sets"]):
        cp = orc.cache_policy(g["E"], g["C"], so, ow, st, 0, [s], t)
        assert [list(c) for c in cp] == g["copies"][t], f"tick {t}"
    assert so.tolist() == g["final_slot_of"]
    assert ow.tolist() == g["final_owner"]
    assert st.tolist() == g["final_stamp"]


@pytest.mark.parametrize("E,C", [(8, 3), (16, 5), (64, 12)])
def test_matches_textbook_lru_for_one_expert_per_token(orc, E, C):
    """K = 1, one layer: the running token's expert is the most recently
    used one, which plain LRU never evicts when C >= 2, so the policy is
    plain LRU."""
    rng = np.random.default_rng(E + C)
    seq = rng.integers(0, E, size=400)
    so, ow, st = _fresh(1, E, C)
    lru = collections.OrderedDict()
    for t, e in enumerate(seq):
        e = int(e)
        hit = e in lru
        if hit:
            lru.move_to_end(e)
        else:
            if len(lru) == C:
                lru.popitem(last=False)
            lru[e] = True
        cp = orc.cache_policy(E, C, so, ow, st, 0, [[e]], t)
        assert (len(cp) == 0) == hit, f"tick {t}"
        assert set(int(o) for o in ow if o >= 0) == set(lru), f"tick {t}"


@pytest.mark.parametrize("E,K,L,C", [(16, 2, 3, 12), (256, 4, 4, 64), (128, 8, 3, 100)])
def test_invariants_over_markov_routing(orc, E, K, L, C):
    rng = np.random.default_rng(40 + K)
    seqs = [synth.markov_sets(rng, E, K, 120, keep=0.5) for _ in range(L)]
    so, ow, st = _fresh(L, E, C)
    total = 0
    for t in range(120):
        before = (so.copy(), ow.copy(), st.copy())
        # stage in two groups of layers, as the pipeline does
        cps = []
        for l0, l1 in ((0, 1), (1, L)):
            pre = (so.copy(), ow.copy(), st.copy())
            got = [(l0 + i, e, c) for i, e, c in
                   orc.cache_policy(E, C, so, ow, st, l0, [seqs[l][t] for l in range(l0, l1)], t)]
            # the entries taken are the least recently staged free ones (the
            # group's own hits are no longer free)
            hits = {int(pre[0][l, e]) for l in range(l0, l1) for e in seqs[l][t] if pre[0][l, e] >= 0}
            # misses are copied once each, in (layer, id) order
            want = [(l, int(e)) for l in range(l0, l1) for e in sorted(set(seqs[l][t].tolist()))
                    if pre[0][l, e] < 0]
            assert [(l, e) for l, e, _ in got] == want
            taken = {c for _, _, c in got}
            free = [c for c in range(C) if (pre[1][c] < 0 or pre[2][c] < t - 1) and c not in hits]
            key = lambda c: (int(pre[2][c]), c)
            if taken:
                worst = max(key(c) for c in taken)
                assert all(key(c) > worst for c in free if c not in taken)
            cps += got
        total += len(cps)
        for l in range(L):
            for e in seqs[l][t]:
                c = so[l, e]
                assert c >= 0 and ow[c] == l * E + e and st[c] == t
        # the running token's entries (stamp t-1 before the call) are kept
        for c in np.nonzero((before[2] == t - 1) & (before[1] >= 0))[0]:
            assert ow[c] == before[1][c]
        # owner and slot_of stay a bijection
        held = ow[ow >= 0]
        assert np.unique(held).size == held.size == (so >= 0).sum()
    # every distinct bundle is copied at least once (compulsory misses)
    assert total >= len({(l, int(e)) for l in range(L) for s in seqs[l] for e in s})


def test_large_cache_copies_each_bundle_once(orc):
    E, K, L = 32, 4, 3
    rng = np.random.default_rng(7)
    seqs = [[synth.random_set(rng, E, K) for _ in range(60)] for _ in range(L)]
    C = L * E
    so, ow, st = _fresh(L, E, C)
    total = 0
    for t in range(60):
        total += len(orc.cache_policy(E, C, so, ow, st, 0, [seqs[l][t] for l in range(L)], t))
    assert total == len({(l, int(e)) for l in range(L) for s in seqs[l] for e in s})


def test_overflow_and_bad_ids_raise_without_changes(orc):
    E, K, L, C = 16, 4, 2, 9  # 2 K L = 16 > C: two disjoint tokens cannot both fit
    so, ow, st = _fresh(L, E, C)
    orc.cache_policy(E, C, so, ow, st, 0, [[0, 1, 2, 3], [4, 5, 6, 7]], 0)
    snap = (so.copy(), ow.copy())
    with pytest.raises(ValueError):
        orc.cache_policy(E, C, so, ow, st, 0, [[8, 9, 10, 11], [12, 13, 14, 15]], 1)
    assert np.array_equal(so, snap[0]) and np.array_equal(ow, snap[1])
    with pytest.raises(ValueError):
        orc.cache_policy(E, C, so, ow, st, 0, [[0, 1, 2, 16]], 2)
