"""GPU parity of the batched path (B >= 16 tokens, grouped int4 GEMMs on
MFMA) against the fp64 oracle.

moe_int4_decode with B >= 16 groups the batch's B*K entries by expert in one
launch and runs tiles of up to 32 of an expert's tokens, each reading the
expert's weights once. Decode chunks: every token's output is compared with
the oracle's moe_decode for its own routing, 35B shapes with top-K in
{2, 4, 8} and 8B shapes, B = 32, a partial tile (20) and two tiles (40);
routed tiles of exactly 1, 8, 9 and 32 tokens (either side of the gate/up
kernel's LDS staging bound); two runs are bitwise equal; an out-of-range id
is flagged.

Prefill-sized batches (the whole-layer path; from 16 entries per expert on
average, B*K >= 16 E, they take the prefill kernels with 64-token tiles):
B = 16 (the smallest batched call) and B = 64 checked token by token; B = 1023
and 1024 either side of the switch at K = 4; B = 256 (8B tier, the union
covers almost every expert), skewed batches of 200 and 1024 tokens whose sets
share 6 hot experts (members of several ragged tiles each; the second on
the prefill kernels) and
B = 3072 (the pages' ~3.1k-token prompt) and B = 8192 (the largest context)
checked against the oracle on sampled tokens, and on every token by a property that holds at any size: a token's
output does not depend on the other tokens of its batch (tile rows are
independent and every sum runs in a fixed order), so the batch equals the same
tokens run in smaller batches that take the same kernels, bit for bit.
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


@pytest.mark.parametrize("n_a,n_b", [(8, 9), (1, 32)])
def test_batched_chunk_tile_sizes(api, orc, pools, n_a, n_b):
    """Routed tiles of exactly n_a and n_b tokens (K = 2, B = 32): 8 and 9
    straddle the gate/up kernel's switch from activations staged in LDS (up
    to 8 tokens) to activations loaded per lane; 1 and 32 are a one-token
    tile and a full routed tile. Every token against the oracle, and two runs
    bitwise equal."""
    dm = synth.dims("35b", K=2)
    pool, sh = pools["35b"]
    announce("batched chunk tile sizes", f"{n_a}/{n_b}")
    ctx = api.Context(dm, max_tokens=32)
    B, E = 32, dm["E"]
    rng = np.random.default_rng(64 + n_a)
    a_id, b_id = 17, 200
    others = np.array([e for e in range(E) if e not in (a_id, b_id)])
    idx = np.zeros((B, 2), np.int32)
    for b in range(B):
        if n_b == B:  # expert b_id in every token, a_id in the first n_a
            idx[b] = [b_id, a_id if b < n_a else rng.choice(others)]
        else:  # a_id in tokens [0, n_a), b_id in [n_a, n_a + n_b)
            first = a_id if b < n_a else (b_id if b < n_a + n_b else rng.choice(others))
            second = rng.choice(others)
            idx[b] = [first, second]
    assert (idx == a_id).sum() == n_a and (idx == b_id).sum() == n_b
    x = rng.normal(size=(B, dm["d"]))
    x = (x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + 1e-6)).astype(np.float16)
    w = np.stack([synth.random_weights(rng, 2) for _ in range(B)]).astype(np.float32)
    dpool, dsh, dx, didx, dw = dev_tree(pool), dev_tree(sh), dev(x), dev(idx), dev(w)
    y = api.moe_int4_decode(ctx, dpool, dx, didx, dw, shared=dsh)
    y2 = api.moe_int4_decode(ctx, dpool, dx, didx, dw, shared=dsh)
    assert api.device_status(ctx) == 0
    assert np.array_equal(host(y).view(np.uint16), host(y2).view(np.uint16)), "not deterministic"
    yg = f16_to_f64(y)
    for b in range(B):
        ref = orc.moe_decode(dm, pool, sh, x[b], idx[b], w[b].astype(np.float64))
        assert_out_close(yg[b], ref, f"tiles {n_a}/{n_b} token {b}")


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


def _prefill_min(dm):
    """Smallest batch that takes the prefill kernels (64-token tiles): at least
    16 entries per expert on average, B*K >= 16 E; smaller batches take the
    chunk kernels (32-token tiles)."""
    return -(-16 * dm["E"] // dm["K"])


def _windows(B, dm):
    """Token windows that take the same kernels as the whole batch: chunks of
    ~32 (none below 16) for the chunk kernels; windows of the prefill minimum,
    the last one ending at B (windows may overlap), for the prefill kernels."""
    PREFILL_MIN = _prefill_min(dm)
    if B < PREFILL_MIN:
        bounds = list(range(0, B, 32)) + [B]
        if len(bounds) > 2 and bounds[-1] - bounds[-2] < 16:
            del bounds[-2]
        return list(zip(bounds[:-1], bounds[1:]))
    starts = sorted(set(list(range(0, B - PREFILL_MIN + 1, PREFILL_MIN)) + [B - PREFILL_MIN]))
    return [(c0, c0 + PREFILL_MIN) for c0 in starts]


def _hot_tokens(rng, dm, B, n_hot):
    """Tokens whose sets are drawn from n_hot hot experts only."""
    x, _, w = _tokens(rng, dm, B)
    hot = rng.choice(dm["E"], size=n_hot, replace=False)
    idx = np.stack([rng.choice(hot, size=dm["K"], replace=False) for _ in range(B)])
    return x, idx.astype(np.int32), w


@pytest.mark.timeout(900)
@pytest.mark.parametrize("tier,K,B,hot,n_check", [("35b", 4, 16, 0, 16), ("35b", 4, 64, 0, 64),
                                                  ("35b", 4, 1023, 0, 16),
                                                  ("35b", 4, 1024, 0, 16),
                                                  ("8b", 8, 256, 0, 24),
                                                  ("35b", 4, 200, 6, 24),
                                                  ("35b", 4, 1024, 6, 16),
                                                  ("35b", 8, 3072, 0, 16),
                                                  ("35b", 8, 8192, 0, 8)])
def test_batched_prefill_parity(api, orc, pools, tier, K, B, hot, n_check):
    import torch
    dm = synth.dims(tier, K=K)
    pool, sh = pools[tier]
    announce("batched prefill", tier, f"K={K} B={B} hot={hot}")
    ctx = api.Context(dm, max_tokens=B)
    dpool, dsh = dev_tree(pool), dev_tree(sh)
    rng = np.random.default_rng(64 + K + B)
    x, idx, w = _hot_tokens(rng, dm, B, hot) if hot else _tokens(rng, dm, B)
    dx, didx, dw = dev(x), dev(idx), dev(w)
    y = api.moe_int4_decode(ctx, dpool, dx, didx, dw, shared=dsh)
    torch.cuda.synchronize()
    assert api.device_status(ctx) == 0
    # sampled tokens (always the first and the last) against the oracle
    check = (np.arange(B) if n_check >= B else
             np.unique(np.concatenate([[0, B - 1], rng.choice(B, size=n_check, replace=False)])))
    yg = f16_to_f64(y)
    worst = 0.0
    for b in check:
        ref = orc.moe_decode(dm, pool, sh, x[b], idx[b], w[b].astype(np.float64))
        assert_out_close(yg[b], ref, f"{tier} K={K} B={B} token {b}")
        worst = max(worst, out_err(yg[b], ref))
    # every token: the batch equals the same tokens run in smaller batches
    # that take the same kernels
    yb = host(y).view(np.uint16)
    for c0, c1 in _windows(B, dm):
        yc = api.moe_int4_decode(ctx, dpool, dx[c0:c1].contiguous(), didx[c0:c1].contiguous(),
                                 dw[c0:c1].contiguous(), shared=dsh)
        assert np.array_equal(host(yc).view(np.uint16), yb[c0:c1]), \
            f"tokens {c0}..{c1} differ between the batch and a smaller batch"
    assert api.device_status(ctx) == 0
    counts = np.bincount(idx.ravel(), minlength=dm["E"])
    print(f"{tier} K={K} B={B}: worst error ratio {worst:.3f} over {len(check)} tokens, "
          f"union {np.count_nonzero(counts)} experts, largest member {counts.max()} tokens")
