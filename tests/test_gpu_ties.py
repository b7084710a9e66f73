"""Routing ties on the GPU ("The Other Half of the Memory Wall", App. A:
descending score, ties to the lower id; the parity tests pin the routing
functions bit-identical).

* Exact ties: a head whose logits are small integers (fc1 = 0, so the MLP
  adds GELU(0) = 0; lin = [0 | I | I], so a logit counts how many of the
  current and previous sets hold the expert) and routers whose rows come in
  identical pairs. The GPU's sets must equal the oracle's bit for bit, lower
  id first, through prerouter_forward and through router layers and heads in
  layer_step, on softmax-top-K (35B) and sigmoid-group (8B).
* Near ties: router rows in pairs that differ in one column by the smallest
  fp16 subnormal, on rows scaled so that fp32 sums cannot resolve the
  difference while fp64 can. The oracle ranks the odd id of a pair first,
  the GPU sees a tie and ranks the even id first, and the checker must take
  its re-anchor branch and accept."""

import numpy as np
import pytest

from gpu_util import announce, dev, host
from helpers import W_TOL
from test_gpu_layer import _run_and_check
from sparse_moe_decode_amd import synth

pytestmark = pytest.mark.gpu

TWO = [dict(router=True, head=True), dict(router=False, head=True)]


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_moe_decode_amd import api as _api
    return _api


def _integer_head(head: dict, d: int, E: int) -> dict:
    """fc1 = 0 and lin = [0 | I | I]: logits = [e in cur] + [e in prev]."""
    h = dict(head)
    h["fc1"] = np.zeros_like(head["fc1"])
    lin = np.zeros_like(head["lin"])
    lin[np.arange(E), d + np.arange(E)] = 1.0
    lin[np.arange(E), d + E + np.arange(E)] = 1.0
    h["lin"] = lin
    if "bias" in h:
        h["bias"] = np.zeros_like(head["bias"])
    return h


def _paired_router(lw: dict) -> dict:
    lw = dict(lw)
    R = lw["router"].copy()
    R[1::2] = R[0::2]
    lw["router"] = R
    if lw["router_bias"] is not None:
        b = lw["router_bias"].copy()
        b[1::2] = b[0::2]
        lw["router_bias"] = b
    return lw


@pytest.mark.parametrize("tier", ["35b", "8b"])
def test_prerouter_exact_ties(api, orc, tier):
    import torch
    dm = synth.dims(tier)
    d, E, K = dm["d"], dm["E"], dm["K"]
    lw = synth.layer(41, 0, dm, dict(router=True, head=True))
    head = _integer_head(lw["head"], d, E)
    rng = np.random.default_rng(42)
    B = 6
    x = rng.normal(size=(B, d)).astype(np.float16)
    cur = np.stack([synth.random_set(rng, E, K) for _ in range(B)]).astype(np.int32)
    prev = np.stack([synth.random_set(rng, E, K) for _ in range(B)]).astype(np.int32)
    prev[1] = cur[1]                       # every logit 0 or 2
    prev[2, : K // 2] = cur[2, : K // 2]   # a mix of 2, 1 and 0
    ctx = api.Context(dm, max_tokens=B)
    dhead = {k: dev(v) for k, v in head.items()}
    logits = torch.empty((B, E), dtype=torch.float32, device="cuda")
    announce("prerouter exact ties", tier)
    idx, w = api.prerouter_forward(ctx, dhead, dev(x), dev(cur), dev(prev), logits=logits)
    assert api.device_status(ctx) == 0
    lg, gi, gw = host(logits), host(idx), host(w)
    for b in range(B):
        ref = orc.head_logits(head["fc1"], head["fc2"], head["lin"], d, E, dm["P"], K,
                              x[b], cur[b], prev[b])
        assert set(np.unique(ref)) <= {0.0, 1.0, 2.0}
        np.testing.assert_array_equal(lg[b], ref.astype(np.float32), err_msg=f"token {b} logits")
        oi, ow = orc.route(dm, ref, head.get("bias"))
        assert gi[b].tolist() == oi.tolist(), f"{tier} token {b}: {gi[b]} vs oracle {oi}"
        np.testing.assert_allclose(gw[b], ow, rtol=0, atol=W_TOL)
    ctx.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tier", ["35b", "8b"])
@pytest.mark.parametrize("path", ["chain", "flow", "persistent", "phases"])
def test_layer_step_exact_ties(api, orc, tier, path):
    """A router layer with paired rows and heads with integer logits: every
    router set and prediction must equal the oracle's, no re-anchoring."""
    dm = synth.dims(tier)

    def mutate(l, lw):
        if lw["router"] is not None:
            lw = _paired_router(lw)
        if lw["head"] is not None:
            lw = dict(lw, head=_integer_head(lw["head"], dm["d"], dm["E"]))
        return lw

    ck = _run_and_check(api, orc, tier, TWO, seed=43, T=4, check_layers=[0, 1], path=path,
                        mutate=mutate)
    assert ck.reanchored == 0 and ck.pred_reanchored == 0, \
        f"exact ties resolved differently from the oracle ({ck.reanchored} router sets, " \
        f"{ck.pred_reanchored} predictions)"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("path", ["chain", "flow", "persistent", "phases"])
def test_layer_step_near_tie_reanchors(api, orc, path):
    from sparse_moe_decode_amd import workloads as wl
    tier, seed = "35b", 44
    dm = synth.dims(tier)
    # the column: the largest positive normed activation of token 0, layer 0
    lw0 = synth.layer(seed, 0, dm, TWO[0])
    h0 = wl.token_inputs(tier, seed, 1, 0.5)[0].astype(np.float64)
    x0 = orc.rmsnorm(h0 + lw0["attn"].astype(np.float64), dm.get("eps", 1e-6))
    j = int(np.argmax(x0))
    assert x0[j] > 0.5

    def mutate(l, lw):
        if lw["router"] is None:
            return lw
        lw = dict(lw)
        R = (lw["router"].astype(np.float32) * 400.0).astype(np.float16)
        R[1::2] = R[0::2]
        R[0::2, j] = 0.0
        R[1::2, j] = np.array([1], np.uint16).view(np.float16)[0]  # smallest subnormal
        lw["router"] = R
        return lw

    ck = _run_and_check(api, orc, tier, TWO, seed=seed, T=3, check_layers=[0, 1], path=path,
                        mutate=mutate)
    assert ck.reanchored >= 1, "the near tie did not reach the re-anchor branch"
