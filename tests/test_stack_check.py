"""The stack checker's routing rule (check_routing) on constructed logits:
it accepts a GPU set that differs from the oracle's only under a near tie,
re-anchors then, and rejects order or weight mistakes that are not ties."""

import numpy as np
import pytest

from helpers import TIE_GAP
from stack_check import check_routing

SOFT = dict(router_kind=0, norm_topk=1, E=8, K=3)


def _oracle(orc, dm, lg, bias=None):
    return orc.route(dm, lg, bias)


def test_equal_lists_check_weights(orc):
    lg = np.array([0.1, 2.0, -0.5, 1.5, 0.9, -2.0, 0.0, 1.0])
    idx, w = _oracle(orc, SOFT, lg)
    assert not check_routing(orc, SOFT, lg, None, idx, w.astype(np.float32), idx, w, "eq")
    with pytest.raises(AssertionError):
        check_routing(orc, SOFT, lg, None, idx, w + 3e-4, idx, w, "eq")


def test_boundary_near_tie_reanchors(orc):
    lg = np.array([0.1, 2.0, -0.5, 1.5, 0.9, -2.0, 0.9 - 0.2 * TIE_GAP, 1.0])
    idx, w = _oracle(orc, SOFT, lg)
    assert idx.tolist() == [1, 3, 7]
    # a K-th place that is not a near tie: rejected
    bad = [1, 3, 4]
    with pytest.raises(AssertionError):
        check_routing(orc, SOFT, lg, None, bad, orc.route_set_weights(SOFT, lg, bad), idx, w, "x")
    lg2 = lg.copy()
    lg2[7] = 0.9 + 0.3 * TIE_GAP  # ids 7, 4, 6 within the gap at the K-th place
    idx2, w2 = _oracle(orc, SOFT, lg2)
    assert idx2.tolist() == [1, 3, 7]
    got = [1, 3, 4]
    gw = orc.route_set_weights(SOFT, lg2, got)
    assert check_routing(orc, SOFT, lg2, None, got, gw, idx2, w2, "near tie")
    # right set, weights in the wrong order: rejected
    with pytest.raises(AssertionError):
        check_routing(orc, SOFT, lg2, None, got, gw[::-1].copy(), idx2, w2, "near tie")


def test_order_swap_needs_a_near_tie(orc):
    lg = np.array([0.1, 2.0, -0.5, 2.0 - 0.5 * TIE_GAP, 0.9, -2.0, 0.0, 1.0])
    idx, w = _oracle(orc, SOFT, lg)
    assert idx.tolist() == [1, 3, 7]
    got = [3, 1, 7]
    assert check_routing(orc, SOFT, lg, None, got, orc.route_set_weights(SOFT, lg, got), idx, w,
                         "swap")
    got = [1, 7, 3]  # same set, 7 ranked above 3 against a gap of ~1
    with pytest.raises(AssertionError):
        check_routing(orc, SOFT, lg, None, got, orc.route_set_weights(SOFT, lg, got), idx, w,
                      "swap")


def test_sigmoid_group_near_tie_between_groups(orc):
    dm = dict(router_kind=1, norm_topk=1, E=8, K=2, n_groups=4, topk_groups=1, route_scale=1.0)
    lg = np.array([1.0, 0.5, 1.0, 0.5 - 1e-5, -3.0, -3.0, -3.0, -3.0])
    idx, w = _oracle(orc, dm, lg)
    assert idx.tolist() == [0, 1]
    got = [2, 3]  # the other group, whose score trails by 1e-5 (sigmoid-scale)
    gw = orc.route_set_weights(dm, lg, got)
    assert check_routing(orc, dm, lg, None, got, gw, idx, w, "groups")
    got = [0, 2]  # two groups touched with topk_groups = 1: rejected
    with pytest.raises(AssertionError):
        check_routing(orc, dm, lg, None, got, orc.route_set_weights(dm, lg, got), idx, w, "g")
