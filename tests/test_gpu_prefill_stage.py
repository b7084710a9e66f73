"""GPU parity of layer-ahead whole-layer staging for prefill-sized batches
(pipeline.PrefillStack over stage_layer).

The layers' routed experts live in a pinned host pool. Each layer's bundles
are copied as one DMA transfer into one of two HBM layer buffers on a side
stream while the previous layer runs on the main stream. For every layer,
every token's output equals the same layer run with its pool resident in HBM,
bit for bit (the same kernels read the same bytes), and sampled tokens match
the oracle. The side stream is held back by a bounded sleep kernel before the
first copy, so a missing wait would show as a layer computed from a buffer
that has not been filled yet.
"""

import numpy as np
import pytest

from gpu_util import announce, dev, dev_tree, f16_to_f64, host
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


def _tokens(rng, dm, B):
    x = rng.normal(size=(B, dm["d"]))
    x = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + 1e-6)
    idx = np.stack([synth.random_set(rng, dm["E"], dm["K"]) for _ in range(B)]).astype(np.int32)
    w = np.stack([synth.random_weights(rng, dm["K"]) for _ in range(B)]).astype(np.float32)
    return x.astype(np.float16), idx, w


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tier,K,B,L", [("35b", 4, 1024, 3), ("8b", 8, 256, 2)])
def test_prefill_stack_matches_resident(api, orc, tier, K, B, L):
    import torch
    from sparse_moe_decode_amd import pipeline
    dm = synth.dims(tier, K=K)
    E, d = dm["E"], dm["d"]
    announce("prefill staging", tier, f"K={K} B={B} L={L}")
    ctx = api.Context(dm, max_tokens=B)
    bundle = ctx.bundle_bytes()
    pools = [synth.routed_pool(synth.rng_for(70, l, len(tier)), dm) for l in range(L)]
    shs = [synth.shared_expert(synth.rng_for(71, l, len(tier)), dm) for l in range(L)]
    host_pool = torch.empty((L, E * bundle), dtype=torch.uint8, pin_memory=True)
    for l in range(L):
        host_pool[l].copy_(torch.from_numpy(api.pack_bundles(pools[l], dm).reshape(-1)))
    dsh = [dev_tree(s) for s in shs]
    rng = np.random.default_rng(72 + B)
    toks = [_tokens(rng, dm, B) for _ in range(L)]
    dx = torch.stack([dev(t[0]) for t in toks]).contiguous()
    didx = torch.stack([dev(t[1]) for t in toks]).contiguous()
    dw = torch.stack([dev(t[2]) for t in toks]).contiguous()
    y = torch.empty((L, B, d), dtype=torch.float16, device="cuda")
    pipe = pipeline.PrefillStack(ctx, host_pool, dsh)
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        with torch.cuda.stream(pipe.side):
            torch.cuda._sleep(40_000_000)  # ~20 ms of spinning, then it exits
    pipe.run(dx, didx, dw, y)
    torch.cuda.synchronize()
    assert api.device_status(ctx) == 0
    yb = host(y).view(np.uint16)
    for l in range(L):
        yr = api.moe_int4_decode(ctx, dev_tree(pools[l]), dx[l], didx[l], dw[l], shared=dsh[l])
        assert np.array_equal(host(yr).view(np.uint16), yb[l]), f"layer {l}: staged != resident"
        yg = f16_to_f64(y[l])
        x, idx, w = toks[l]
        for b in (0, B // 2, B - 1):
            ref = orc.moe_decode(dm, pools[l], shs[l], x[b], idx[b], w[b].astype(np.float64))
            assert_out_close(yg[b], ref, f"{tier} layer {l} token {b}")
    assert api.device_status(ctx) == 0
    print(f"{tier} K={K} B={B}: {L} staged layers equal the resident ones")
