"""Re-anchored per-layer-step comparison of a GPU decode run with the oracle.

For token t and layer l the oracle starts from the GPU's fp16 input h[l],
the GPU's consumed routing (predicted layers) and the GPU's previous-token
set, computes that one layer-step in fp64 and compares:
  * router layers: the executed ordered set must equal the oracle's, or
    differ from it only under the near-tie rule (check_routing), in which
    case the oracle is re-anchored to the GPU's set; weights within 1e-4 of
    what the routing function gives the GPU's set;
  * predicted layers: the executed set equals the prediction consumed;
  * h_out within 2e-3 + 1e-2 |ref|;
  * head logits (2e-4 absolute) and the prediction for layer l+1 (the same
    rule as router layers).
quant=1 checks layers with affine int4 experts against the affine layer oracle.
"""

from __future__ import annotations

import numpy as np

from helpers import TIE_GAP, W_TOL, assert_out_close, out_err, routing_set_ok
from sparse_moe_decode_amd import synth


def check_routing(orc, dm, logits, bias, got_idx, got_w, ora_idx, ora_w, what) -> bool:
    """The GPU's ordered routing (got) against the oracle's on the oracle's
    fp64 logits ("The Other Half of the Memory Wall", App. A: descending
    score, ties to the lower id). Equal lists: weights within W_TOL. A
    different list passes only if every difference is a near tie:
      * the set is a top-K of the scores up to TIE_GAP (routing_set_ok,
        which also checks the sigmoid-group group stage);
      * no pair is out of order by more than TIE_GAP: for i < j the score of
        got[i] is at least that of got[j] minus TIE_GAP (so a reordering of
        an equal set, too, needs a near tie);
      * the weights equal what the routing function gives the GPU's set in
        the GPU's order (route_set_weights), within W_TOL.
    Returns True when the lists differ (the caller re-anchors)."""
    got = [int(e) for e in got_idx]
    ora = [int(e) for e in ora_idx]
    if got == ora:
        np.testing.assert_allclose(got_w, ora_w, rtol=0, atol=W_TOL, err_msg=what + " weights")
        return False
    assert routing_set_ok(dm, logits, got, bias), f"{what}: set {got} vs oracle {ora}"
    sc = orc.route_scores(dm, logits, bias)
    for i in range(len(got)):
        for j in range(i + 1, len(got)):
            assert sc[got[i]] >= sc[got[j]] - TIE_GAP, \
                f"{what}: {got} ranks id {got[i]} above {got[j]} against a score gap of " \
                f"{sc[got[j]] - sc[got[i]]:.3g} (oracle {ora})"
    np.testing.assert_allclose(got_w, orc.route_set_weights(dm, logits, got, bias), rtol=0,
                               atol=W_TOL, err_msg=what + " weights of the GPU's set")
    return True


class StackChecker:
    def __init__(self, orc, tier: str, seed: int, roles: list[dict], layers: list[int],
                 host_layers: dict | None = None, zero_mean: bool = False, quant: int = 0,
                 dims: dict | None = None):
        self.orc = orc
        if dims is not None:  # the tier's shapes with overrides (e.g. fewer experts)
            self.dm = dims
        else:
            self.dm = synth.dims(tier, quant=1) if quant == 1 else synth.dims(tier)
        oracle_cls = orc.LayerOracleAffine if quant == 1 else orc.LayerOracle
        self.roles = roles
        self.L = len(roles)
        self.layers = layers
        self.lo, self.lo_cons, self.w = {}, {}, {}
        for l in layers:
            lw = (host_layers or {}).get(l)
            if lw is None:
                lw = synth.layer(seed, l, self.dm, roles[l], zero_mean=zero_mean)
            self.w[l] = lw
            self.lo[l] = oracle_cls(self.dm, lw)
            if lw["router"] is not None:
                cons = dict(lw)
                cons["router"] = None
                self.lo_cons[l] = oracle_cls(self.dm, cons)
        self.worst = 0.0
        self.x_ulp_diffs = 0
        self.reanchored = 0       # router layers whose GPU set differed under a near tie
        self.pred_reanchored = 0  # predictions that did
        self.steps = 0

    def check(self, t, h_trace, x_trace, exec_idx, exec_w, prev_idx, route_idx, route_w,
              pred_idx, pred_w, head_logits):
        dm = self.dm
        for l in self.layers:
            what = f"token {t} layer {l}"
            h_in = h_trace[l]
            prev = prev_idx[l] if t > 0 else None
            lw = self.w[l]
            # The normed activation is an fp16 rounding point: the GPU's fp32 norm
            # may round an element to the neighbouring fp16 value. Check that it
            # is within one ulp of the oracle's rounding, then continue from it.
            x_gpu = np.asarray(x_trace[l]).view(np.uint16)
            if lw["router"] is not None:
                out = self.lo[l].step(h_in, prev_idx=prev, x16=x_gpu)
                if check_routing(self.orc, dm, out["router_logits"], lw["router_bias"],
                                 exec_idx[l], exec_w[l], out["exec_idx"], out["exec_w"],
                                 what + " router"):
                    self.reanchored += 1
                    out = self.lo_cons[l].step(h_in, exec_idx[l], exec_w[l], prev, x16=x_gpu)
            else:
                assert list(exec_idx[l]) == list(route_idx[l]), \
                    f"{what}: executed set is not the consumed prediction"
                np.testing.assert_array_equal(exec_w[l], route_w[l])
                out = self.lo[l].step(h_in, exec_idx[l], exec_w[l], prev, x16=x_gpu)
            ulps = np.abs(x_gpu.astype(np.int64) - out["x16"].astype(np.int64))
            assert ulps.max() <= 1, f"{what}: normed activation off by {ulps.max()} ulp"
            self.x_ulp_diffs += int((ulps > 0).sum())
            assert_out_close(h_trace[l + 1].astype(np.float64), out["h_out"], what)
            self.worst = max(self.worst, out_err(h_trace[l + 1], out["h_out"]))
            if lw["head"] is not None:
                np.testing.assert_allclose(head_logits[l], out["head_logits"], rtol=0,
                                           atol=2e-4, err_msg=what + " head logits")
                if l + 1 < self.L:
                    if check_routing(self.orc, dm, out["head_logits"], lw["head"].get("bias"),
                                     pred_idx[l + 1], pred_w[l + 1], out["pred_idx"],
                                     out["pred_w"], what + " prediction"):
                        self.pred_reanchored += 1
            self.steps += 1

