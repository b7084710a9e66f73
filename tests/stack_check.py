"""Re-anchored per-layer-step comparison of a GPU decode run with the oracle.

For token t and layer l the oracle starts from the GPU's fp16 input h[l],
the GPU's consumed routing (predicted layers) and the GPU's previous-token
set, computes that one layer-step in fp64 and compares:
  * router layers: the executed set (bit-exact up to 1e-3 near ties, then the
    oracle is re-anchored to the GPU's set) and its weights (1e-4);
  * predicted layers: the executed set equals the prediction consumed;
  * h_out within 2e-3 + 1e-2 |ref|;
  * head logits (2e-4 absolute) and the prediction for layer l+1 (near-tie
    rule, weights 1e-4).
quant=1 checks layers with affine int4 experts against the affine layer oracle.
"""

from __future__ import annotations

import numpy as np

from helpers import W_TOL, assert_out_close, out_err, routing_set_ok
from sparse_moe_decode_amd import synth


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
        self.reanchored = 0
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
                assert routing_set_ok(dm, out["router_logits"], exec_idx[l], lw["router_bias"]), \
                    f"{what}: router set {exec_idx[l]} vs oracle {out['exec_idx']}"
                if list(out["exec_idx"]) != list(exec_idx[l]):
                    self.reanchored += 1
                    out = self.lo_cons[l].step(h_in, exec_idx[l], exec_w[l], prev, x16=x_gpu)
                else:
                    np.testing.assert_allclose(exec_w[l], out["exec_w"], rtol=0, atol=W_TOL,
                                               err_msg=what)
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
                    bias = lw["head"].get("bias")
                    assert routing_set_ok(dm, out["head_logits"], pred_idx[l + 1], bias), \
                        f"{what}: predicted set {pred_idx[l + 1]} vs oracle {out['pred_idx']}"
                    if list(out["pred_idx"]) == list(pred_idx[l + 1]):
                        np.testing.assert_allclose(pred_w[l + 1], out["pred_w"], rtol=0,
                                                   atol=W_TOL, err_msg=what + " pred w")
            self.steps += 1

