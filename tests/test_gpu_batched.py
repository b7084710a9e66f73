"""GPU parity of the batched chunk (16..32 tokens per chunk, grouped int4
GEMMs on MFMA) against the fp64 oracle.

moe_int4_decode with B >= 16 groups the tokens by expert and reads each
expert's weights once per chunk of up to 32 tokens. Every token's output is
compared with the oracle's moe_decode for its own routing: 35B shapes with
top-K in {2, 4, 8} and 8B shapes, full chunks of 32, a partial chunk and two
chunks; two runs are bitwise equal; an out-of-range id is flagged.
"""

import numpy as np
import pytest

from gpu_util import announce, dev, dev_tree, f16_to_f64, host
from helpers import assert_out_close, out_err
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
def pools():
    out = {}
    for tier in ("35b", "8b"):
        dm = synth.dims(tier)
        pool = synth.routed_pool(synth.rng_for(60, len(tier)), dm)
        sh = synth.shared_expert(synth.rng_for(61, len(tier)), dm)
        out[tier] = (pool, sh)
    return out


def _tokens(rng, dm, B):
    x = rng.normal(size=(B, dm["d"]))
    x = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + 1e-6)
    idx = np.stack([synth.random_set(rng, dm["E"], dm["K"]) for _ in range(B)]).astype(np.int32)
    w = np.stack([synth.random_weights(rng, dm["K"]) for _ in range(B)]).astype(np.float32)
    return x.astype(np.float16), idx, w


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tier,K,B", [("35b", 2, 32), ("35b", 4, 32), ("35b", 8, 32),
                                      ("8b", 8, 32), ("35b", 4, 20), ("35b", 4, 40)])
def test_batched_chunk_parity(api, orc, pools, tier, K, B):
    import torch
    dm = synth.dims(tier, K=K)
    pool, sh = pools[tier]
    announce("batched chunk", tier, f"K={K} B={B}")
    ctx = api.Context(dm, max_tokens=64)
    dpool, dsh = dev_tree(pool), dev_tree(sh)
    rng = np.random.default_rng(62 + K + B)
    x, idx, w = _tokens(rng, dm, B)
    dx, didx, dw = dev(x), dev(idx), dev(w)
    y = api.moe_int4_decode(ctx, dpool, dx, didx, dw, shared=dsh)
    assert api.device_status(ctx) == 0
    y2 = api.moe_int4_decode(ctx, dpool, dx, didx, dw, shared=dsh)
    assert np.array_equal(host(y).view(np.uint16), host(y2).view(np.uint16)), "not deterministic"
    yg = f16_to_f64(y)
    worst = 0.0
    for b in range(B):
        ref = orc.moe_decode(dm, pool, sh, x[b], idx[b], w[b].astype(np.float64))
        assert_out_close(yg[b], ref, f"{tier} K={K} token {b}")
        worst = max(worst, out_err(yg[b], ref))
    # warm timing of the chunk (context only; the bench is the measurement)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(10):
        api.moe_int4_decode(ctx, dpool, dx, didx, dw, y=y, shared=dsh)
    ev1.record()
    torch.cuda.synchronize()
    union = len(np.unique(idx))
    print(f"{tier} K={K} B={B}: worst error ratio {worst:.3f}, union {union} experts, "
          f"{ev0.elapsed_time(ev1) / 10 * 1e3:.1f} us per call")


def test_batched_bad_id_is_flagged(api, pools):
    dm = synth.dims("35b")
    pool, sh = pools["35b"]
    announce("batched chunk bad id")
    ctx = api.Context(dm, max_tokens=32)
    rng = np.random.default_rng(63)
    x, idx, w = _tokens(rng, dm, 32)
    idx[5, 1] = dm["E"] + 3
    api.moe_int4_decode(ctx, dev_tree(pool), dev(x), dev(idx), dev(w), shared=dev_tree(sh))
    assert api.device_status(ctx) == api.E0_ERR_RANGE
