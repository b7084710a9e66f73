"""Pins of the oracle's routing functions ("The Other Half of the Memory Wall",
Appendix A) by brute force over all subsets, library softmax/sigmoid and
constructed cases where a plausible mistake changes the answer.
"""

import itertools

import numpy as np
import pytest
import scipy.special as sp


def _brute_topk(score, K, allowed=None):
    """The K-subset with the largest score sum (unique for distinct scores)."""
    ids = [e for e in range(score.size) if allowed is None or allowed[e]]
    best = max(itertools.combinations(ids, K), key=lambda c: sum(score[list(c)]))
    return sorted(best, key=lambda e: -score[e])


@pytest.mark.parametrize("n,k", [(8, 1), (8, 2), (8, 5), (10, 3), (9, 9)])
def test_topk_brute_force(orc, n, k):
    rng = np.random.default_rng(10 + n * k)
    for _ in range(30):
        s = rng.normal(size=n)
        assert orc.topk(s, k).tolist() == _brute_topk(s, k)


def test_topk_ties_lower_id_first(orc):
    s = np.array([1.0, 3.0, 2.0, 3.0, 2.0, 3.0])
    assert orc.topk(s, 4).tolist() == [1, 3, 5, 2]
    allowed = np.array([1, 0, 1, 0, 1, 1], np.uint8)
    assert orc.topk(s, 3, allowed).tolist() == [5, 2, 4]


def test_softmax_topk_against_library_and_brute_force(orc):
    rng = np.random.default_rng(11)
    for E, K in [(8, 2), (8, 4), (12, 3)]:
        for _ in range(25):
            lg = rng.normal(0, 2, E)
            idx, w = orc.route_softmax_topk(lg, K, norm=True)
            g = sp.softmax(lg)
            assert idx.tolist() == _brute_topk(g, K)
            np.testing.assert_allclose(w, g[idx] / g[idx].sum(), rtol=1e-13)
            # Closed form: renormalised softmax over the chosen logits only.
            np.testing.assert_allclose(w, sp.softmax(lg[idx]), rtol=1e-13)
            assert abs(w.sum() - 1.0) < 1e-14
            idx2, w2 = orc.route_softmax_topk(lg, K, norm=False)
            assert idx2.tolist() == idx.tolist()
            np.testing.assert_allclose(w2, g[idx], rtol=1e-13)


def _brute_sigmoid_group(lg, bias, K, n, Gk, s):
    E = lg.size
    per = E // n
    sig = sp.expit(lg)
    sel = sig + bias
    # Group score: the best pair sum inside the group (= sum of the top two).
    gs = np.array([max(sel[g * per + a] + sel[g * per + b]
                       for a, b in itertools.combinations(range(per), 2)) for g in range(n)])
    groups = max(itertools.combinations(range(n), Gk), key=lambda c: sum(gs[list(c)]))
    allowed = np.zeros(E, bool)
    for g in groups:
        allowed[g * per:(g + 1) * per] = True
    idx = _brute_topk(sel, K, allowed)
    w = s * sig[idx] / (sig[idx].sum() + 1e-20)
    return idx, w


@pytest.mark.parametrize("E,K,n,Gk", [(8, 2, 4, 2), (12, 3, 4, 2), (16, 4, 4, 2), (16, 5, 8, 3)])
def test_sigmoid_group_brute_force(orc, E, K, n, Gk):
    rng = np.random.default_rng(12 + E + K)
    for _ in range(25):
        lg = rng.normal(0, 1.5, E)
        bias = rng.normal(0, 0.3, E)
        idx, w = orc.route_sigmoid_group(lg, bias, K, n, Gk, 2.5)
        bidx, bw = _brute_sigmoid_group(lg, bias, K, n, Gk, 2.5)
        assert idx.tolist() == bidx
        np.testing.assert_allclose(w, bw, rtol=1e-13)


def test_sigmoid_group_one_group_reduces_to_sigmoid_topk(orc):
    """n = G = 1 and no bias: top-K of the logits, weights s*sigmoid/sum."""
    rng = np.random.default_rng(13)
    lg = rng.normal(0, 1, 16)
    idx, w = orc.route_sigmoid_group(lg, np.zeros(16), 5, 1, 1, 2.5)
    want = np.argsort(-lg, kind="stable")[:5]
    assert idx.tolist() == want.tolist()
    sig = sp.expit(lg[want])
    np.testing.assert_allclose(w, 2.5 * sig / sig.sum(), rtol=1e-13)
    np.testing.assert_allclose(w.sum(), 2.5, rtol=1e-13)


def test_sigmoid_group_bias_selects_but_does_not_weight(orc):
    """A large bias pulls an expert into the set; its weight uses raw sigmoid."""
    lg = np.array([3.0, 2.0, 1.0, -4.0, 0.0, 0.0, 0.0, 0.0])
    bias = np.zeros(8)
    bias[3] = 5.0
    idx, w = orc.route_sigmoid_group(lg, bias, 2, 1, 1, 1.0)
    assert idx.tolist() == [3, 0]
    sig = sp.expit(lg[[3, 0]])
    np.testing.assert_allclose(w, sig / sig.sum(), rtol=1e-13)


def test_sigmoid_group_score_is_top2_sum(orc):
    """Group A has one huge score; group B has two medium ones and wins on the top-2 sum."""
    lg = np.array([6.0, -6.0, -6.0, -6.0, 1.0, 1.0, -6.0, -6.0])
    idx, _w, _sel, gs = orc.route_sigmoid_group(lg, np.zeros(8), 2, 2, 1, 1.0, return_scores=True)
    assert sorted(idx.tolist()) == [4, 5]
    np.testing.assert_allclose(gs, [sp.expit(6) + sp.expit(-6), 2 * sp.expit(1)], rtol=1e-13)


def test_routing_dispatch_by_tier(orc):
    from sparse_moe_decode_amd import synth
    rng = np.random.default_rng(14)
    for tier in ("tiny", "8b", "35b"):
        dm = synth.dims(tier)
        lg = rng.normal(size=dm["E"])
        bias = rng.normal(0, 0.02, dm["E"]).astype(np.float32)
        idx, w = orc.route(dm, lg, bias if dm["router_kind"] else None)
        if dm["router_kind"] == 0:
            i2, w2 = orc.route_softmax_topk(lg, dm["K"], True)
        else:
            i2, w2 = orc.route_sigmoid_group(lg, bias.astype(np.float64), dm["K"], dm["n_groups"],
                                             dm["topk_groups"], dm["route_scale"])
        assert idx.tolist() == i2.tolist()
        np.testing.assert_allclose(w, w2, rtol=1e-15)


def test_set_weights_match_the_routing_function_on_its_own_set(orc):
    """route_set_weights (numpy) on the set route() picks reproduces route()'s
    weights (the C++ routine) on every tier and both normalisations."""
    from sparse_moe_decode_amd import synth
    rng = np.random.default_rng(15)
    for tier in ("tiny", "8b", "35b"):
        for norm in (1, 0):
            dm = dict(synth.dims(tier), norm_topk=norm)
            for _ in range(10):
                lg = rng.normal(0, 1.5, dm["E"])
                bias = rng.normal(0, 0.02, dm["E"]).astype(np.float32)
                b = bias if dm["router_kind"] else None
                idx, w = orc.route(dm, lg, b)
                np.testing.assert_allclose(orc.route_set_weights(dm, lg, idx, b), w, rtol=1e-13)


def test_set_weights_closed_forms(orc):
    """Any set, not only the top-K: library softmax and sigmoid."""
    lg = np.array([0.3, -1.2, 2.0, 0.7, -0.1, 1.1])
    soft = dict(router_kind=0, norm_topk=1)
    w = orc.route_set_weights(soft, lg, [4, 1])
    np.testing.assert_allclose(w, [sp.expit(lg[4] - lg[1]), sp.expit(lg[1] - lg[4])], rtol=1e-13)
    w = orc.route_set_weights(dict(soft, norm_topk=0), lg, [4, 1])
    np.testing.assert_allclose(w, sp.softmax(lg)[[4, 1]], rtol=1e-13)
    grp = dict(router_kind=1, route_scale=2.5)
    w = orc.route_set_weights(grp, lg, [5, 0, 3], bias=np.full(6, 7.0))
    s = sp.expit(lg[[5, 0, 3]])
    np.testing.assert_allclose(w, 2.5 * s / s.sum(), rtol=1e-13)
    np.testing.assert_allclose(orc.route_scores(soft, lg), lg, rtol=0)
    bias = np.linspace(-0.1, 0.1, 6)
    np.testing.assert_allclose(orc.route_scores(grp, lg, bias), sp.expit(lg) + bias, rtol=1e-15)
