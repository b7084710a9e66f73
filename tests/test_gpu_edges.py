"""Edge cases of the single-call entry points, through the C ABI.

* empty batches (n_tokens = 0) return success and leave every output
  untouched; negative counts and counts above the context's max_tokens are
  rejected before any launch;
* top-1 routing (K = 1, the degenerate case of the method: the one expert
  gets weight 1) against the oracle, on the per-token GEMV path (B = 1, 3)
  and on the grouped MFMA path (B = 16, 64) at the 35B shapes, and at the
  tiny shapes;
* a batch of exactly max_tokens, and one above it;
* every expert selected (K = E): the head routes all of them in descending
  score with the full softmax as weights, and the decode sums them all.
"""

import ctypes as C

import numpy as np
import pytest

from gpu_util import announce, dev, dev_tree, f16_to_f64
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


@pytest.fixture(scope="module")
def tiny(api):
    dm = synth.dims("tiny")
    rng = synth.rng_for(77)
    pool, sh = synth.routed_pool(rng, dm), synth.shared_expert(rng, dm)
    hd = synth.head(synth.rng_for(78), dm)
    ctx = api.Context(dm, max_tokens=4)
    yield dict(dm=dm, pool=pool, sh=sh, hd=hd, ctx=ctx, rng=rng)
    ctx.close()


def _tokens(rng, dm, B):
    x = rng.normal(size=(B, dm["d"])).astype(np.float16)
    idx = np.stack([synth.random_set(rng, dm["E"], dm["K"]) for _ in range(B)]).astype(np.int32)
    w = np.stack([synth.random_weights(rng, dm["K"]) for _ in range(B)]).astype(np.float32)
    return x, idx, w


def test_empty_batches_leave_outputs_untouched(api, tiny):
    import torch
    dm, ctx = tiny["dm"], tiny["ctx"]
    announce("edges", "tiny", "empty batches")
    x, idx, w = _tokens(tiny["rng"], dm, 1)
    dx, didx, dw = dev(x), dev(idx), dev(w)
    ex = api.experts_struct(dev_tree(tiny["pool"]), dm["E"])
    dsh = dev_tree(tiny["sh"])
    sh = api.shared_struct(dsh)
    y = torch.full((1, dm["d"]), 7.0, dtype=torch.float16, device="cuda")
    rc = api._lib.moe_int4_decode(ctx.handle, C.byref(ex), None, C.byref(sh), api._ptr(dx),
                                  api._ptr(didx), api._ptr(dw), 0, api._ptr(y), None)
    assert rc == 0
    acc = torch.full((1, dm["Is"]), 3.0, dtype=torch.float32, device="cuda")
    rc = api._lib.lora_delta(ctx.handle, api._ptr(dsh["a_gate"]), api._ptr(dsh["b_gate"]), dm["d"],
                             dm["Is"], dm["r"], 1.0, api._ptr(dx), api._ptr(acc), 0, None)
    assert rc == 0
    hs = api.head_struct(dev_tree(tiny["hd"]))
    lg = torch.full((1, dm["E"]), 5.0, dtype=torch.float32, device="cuda")
    oi = torch.full((1, dm["K"]), -9, dtype=torch.int32, device="cuda")
    ow = torch.full((1, dm["K"]), 9.0, dtype=torch.float32, device="cuda")
    rc = api._lib.prerouter_forward(ctx.handle, C.byref(hs), api._ptr(dx), api._ptr(didx), None,
                                    0, api._ptr(lg), api._ptr(oi), api._ptr(ow), None)
    assert rc == 0
    torch.cuda.synchronize()
    assert api.device_status(ctx) == 0
    assert bool((y == 7.0).all()) and bool((acc == 3.0).all())
    assert bool((lg == 5.0).all()) and bool((oi == -9).all()) and bool((ow == 9.0).all())
    for n in (-1, 5):  # max_tokens = 4
        rc = api._lib.moe_int4_decode(ctx.handle, C.byref(ex), None, C.byref(sh), api._ptr(dx),
                                      api._ptr(didx), api._ptr(dw), n, api._ptr(y), None)
        assert rc == api.E0_ERR_ARG
        rc = api._lib.prerouter_forward(ctx.handle, C.byref(hs), api._ptr(dx), api._ptr(didx),
                                        None, n, None, api._ptr(oi), api._ptr(ow), None)
        assert rc == api.E0_ERR_ARG
    assert bool((y == 7.0).all())


def test_max_tokens_batch(api, orc, tiny):
    dm, ctx = tiny["dm"], tiny["ctx"]
    announce("edges", "tiny", "B = max_tokens")
    x, idx, w = _tokens(tiny["rng"], dm, 4)
    y = api.moe_int4_decode(ctx, dev_tree(tiny["pool"]), dev(x), dev(idx), dev(w),
                            shared=dev_tree(tiny["sh"]))
    assert api.device_status(ctx) == 0
    yg = f16_to_f64(y)
    for b in range(4):
        assert_out_close(yg[b], orc.moe_decode(dm, tiny["pool"], tiny["sh"], x[b], idx[b],
                                               w[b].astype(np.float64)), f"token {b}")
    x5, idx5, w5 = _tokens(tiny["rng"], dm, 5)
    with pytest.raises(api.E0Error):
        api.moe_int4_decode(ctx, dev_tree(tiny["pool"]), dev(x5), dev(idx5), dev(w5))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("tier,B", [("tiny", 3), ("35b", 1), ("35b", 3), ("35b", 16),
                                    ("35b", 64)])
def test_top1_routing(api, orc, tier, B):
    dm = synth.dims(tier, K=1)
    announce("edges", tier, f"K=1 B={B}")
    rng = synth.rng_for(79, B)
    n = dm["E"] if B >= 16 else min(dm["E"], 32)  # the grouped path on the full pool
    dmn = dict(dm, E=n)
    pool, sh = synth.routed_pool(rng, dmn), synth.shared_expert(rng, dmn)
    ctx = api.Context(dmn, max_tokens=B)
    x = rng.normal(size=(B, dm["d"])).astype(np.float16)
    idx = rng.integers(0, n, size=(B, 1)).astype(np.int32)
    w = np.ones((B, 1), np.float32)
    y = api.moe_int4_decode(ctx, dev_tree(pool), dev(x), dev(idx), dev(w), shared=dev_tree(sh))
    assert api.device_status(ctx) == 0
    yg = f16_to_f64(y)
    for b in range(B):
        assert_out_close(yg[b], orc.moe_decode(dmn, pool, sh, x[b], idx[b], np.ones(1)),
                         f"{tier} K=1 token {b}")
    ctx.close()


def test_every_expert_selected(api, orc):
    """K = E (the tiny tier's 8 experts, softmax routing): the head's routing
    returns every expert in descending score with the full softmax as
    weights, and the decode sums every expert."""
    import torch
    from gpu_util import host
    from helpers import W_TOL
    dm = synth.dims("tiny", K=8)
    assert dm["K"] == dm["E"]
    announce("edges", "tiny", "K = E")
    rng = synth.rng_for(80)
    pool, sh = synth.routed_pool(rng, dm), synth.shared_expert(rng, dm)
    hd = synth.head(synth.rng_for(81), dm)
    ctx = api.Context(dm, max_tokens=2)
    x = rng.normal(size=(2, dm["d"])).astype(np.float16)
    cur = np.stack([rng.permutation(8) for _ in range(2)]).astype(np.int32)
    prev = np.stack([rng.permutation(8) for _ in range(2)]).astype(np.int32)
    lg = torch.empty((2, dm["E"]), dtype=torch.float32, device="cuda")
    oi, ow = api.prerouter_forward(ctx, dev_tree(hd), dev(x), dev(cur), dev(prev), logits=lg)
    y = api.moe_int4_decode(ctx, dev_tree(pool), dev(x), oi, ow, shared=dev_tree(sh))
    assert api.device_status(ctx) == 0
    oi, ow, lg, yg = host(oi), host(ow), host(lg), f16_to_f64(y)
    for b in range(2):
        ref = orc.head_logits(hd["fc1"], hd["fc2"], hd["lin"], dm["d"], dm["E"], dm["P"], dm["K"],
                              x[b], cur[b], prev[b], 1)
        np.testing.assert_allclose(lg[b], ref, rtol=0, atol=2e-4)
        assert sorted(oi[b].tolist()) == list(range(8))
        assert np.all(np.diff(ref[oi[b]]) <= 2e-4), "selection not in descending score"
        p = np.exp(ref - ref.max())
        np.testing.assert_allclose(ow[b], p[oi[b]] / p.sum(), rtol=0, atol=W_TOL)
        assert_out_close(yg[b], orc.moe_decode(dm, pool, sh, x[b], oi[b], ow[b].astype(np.float64)),
                         f"K = E token {b}")
    ctx.close()
