"""moe_int4_decode_static (the entry point that allocates nothing) against
moe_int4_decode on the same inputs: several calls in a row on the one static
workspace, each smaller than the one before, across both execution paths
(grouped MFMA for 16 tokens and more, per-token GEMV below) and both tiers.
The outputs must be identical bit for bit (the same kernels run on a
different workspace); sampled tokens are also held to the oracle."""

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
def test_static_workspace_matches_context_path(api, orc):
    import torch
    flags = torch.zeros(4, dtype=torch.int32, device="cuda")
    for tier, sizes in (("35b", (40, 17, 3)), ("8b", (24, 2))):
        dm = synth.dims(tier)
        pool = synth.routed_pool(synth.rng_for(70, len(tier)), dm)
        sh = synth.shared_expert(synth.rng_for(71, len(tier)), dm)
        dpool, dsh = dev_tree(pool), dev_tree(sh)
        ctx = api.Context(dm, max_tokens=64)
        rng = np.random.default_rng(72 + len(tier))
        for B in sizes:
            announce("moe_int4_decode_static", tier, f"B={B}")
            x, idx, w = _tokens(rng, dm, B)
            dx, didx, dw = dev(x), dev(idx), dev(w)
            y_ctx = api.moe_int4_decode(ctx, dpool, dx, didx, dw, shared=dsh)
            # the output buffer starts as garbage so a skipped write shows
            y_st = torch.full_like(dx, float("nan"))
            api.moe_int4_decode_static(dm, dpool, dx, didx, dw, y=y_st, shared=dsh, flags=flags)
            torch.cuda.synchronize()
            assert api.device_status(ctx) == 0
            assert int(flags.abs().sum()) == 0, "error bits raised on valid ids"
            a, b = host(y_ctx).view(np.uint16), host(y_st).view(np.uint16)
            assert np.array_equal(a, b), f"{tier} B={B}: {np.count_nonzero(a != b)} outputs differ"
            yg = f16_to_f64(y_st)
            for t in sorted({0, B // 2, B - 1}):
                ref = orc.moe_decode(dm, pool, sh, x[t], idx[t], w[t].astype(np.float64))
                assert_out_close(yg[t], ref, f"{tier} B={B} token {t}")


def test_static_workspace_flags_bad_id(api):
    import torch
    dm = synth.dims("35b")
    pool = synth.routed_pool(synth.rng_for(70, 3), dm)
    dpool = dev_tree(pool)
    rng = np.random.default_rng(73)
    x, idx, w = _tokens(rng, dm, 2)
    idx[1, 0] = dm["E"] + 5
    flags = torch.zeros(4, dtype=torch.int32, device="cuda")
    announce("moe_int4_decode_static", "35b", "bad id")
    api.moe_int4_decode_static(dm, dpool, dev(x), dev(idx), dev(w), flags=flags)
    torch.cuda.synchronize()
    assert int(flags[0]) != 0, "an out-of-range id did not raise the range bit"
