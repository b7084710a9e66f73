"""GPU parity of the single-call entry points against the fp64 oracle.

moe_int4_decode, lora_delta and prerouter_forward are called through the C
ABI on synthetic inputs shaped like the tiers (tiny, 8B, 35B), element by
element against the oracle: fp16 outputs within |d| <= 2e-3 + 1e-2 |ref|,
routing sets bit-exact up to 1e-3-wide near ties, routing weights within 1e-4.
"""

import numpy as np
import pytest

from gpu_util import announce, dev, dev_tree, f16_to_f64, host
from helpers import W_TOL, assert_out_close, routing_set_ok
from sparse_moe_decode_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_moe_decode_amd import api as _api
    return _api


TIER_CASES = {"tiny": 64, "8b": 6, "35b": 6}


@pytest.fixture(scope="module", params=["tiny", "8b", "35b"])
def tier(request, api):
    name = request.param
    dm = synth.dims(name)
    rng = synth.rng_for(1000 + len(name))
    pool = synth.routed_pool(rng, dm)
    sh = synth.shared_expert(rng, dm)
    hd = synth.head(synth.rng_for(2000 + len(name)), dm)
    ctx = api.Context(dm, max_tokens=8)
    return dict(name=name, dm=dm, pool=pool, sh=sh, head=hd, ctx=ctx, dpool=dev_tree(pool),
                dsh=dev_tree(sh), dhead=dev_tree(hd))


def test_moe_decode_parity(api, tier, orc):
    dm, ctx = tier["dm"], tier["ctx"]
    rng = np.random.default_rng(7)
    n = TIER_CASES[tier["name"]]
    announce("moe_int4_decode", tier["name"], n)
    worst = 0.0
    for case in range(n):
        B = 1 if case % 2 == 0 else 3
        x = rng.normal(size=(B, dm["d"])).astype(np.float16)
        idx = np.stack([synth.random_set(rng, dm["E"], dm["K"]) for _ in range(B)])
        w = np.stack([synth.random_weights(rng, dm["K"]) for _ in range(B)])
        y = api.moe_int4_decode(ctx, tier["dpool"], dev(x), dev(idx), dev(w),
                                shared=tier["dsh"])
        assert api.device_status(ctx) == 0
        yg = f16_to_f64(y)
        for b in range(B):
            ref = orc.moe_decode(dm, tier["pool"], tier["sh"], x[b], idx[b],
                                 w[b].astype(np.float64))
            assert_out_close(yg[b], ref, f"{tier['name']} case {case} token {b}")
            worst = max(worst, float(np.max(np.abs(yg[b] - ref))))
    print(f"{tier['name']}: worst |dy| = {worst:.3g}")


def test_moe_decode_without_shared_or_lora(api, tier, orc):
    dm, ctx = tier["dm"], tier["ctx"]
    rng = np.random.default_rng(8)
    announce("moe_int4_decode no-shared/no-lora", tier["name"])
    x = rng.normal(size=(1, dm["d"])).astype(np.float16)
    idx = synth.random_set(rng, dm["E"], dm["K"])[None]
    w = synth.random_weights(rng, dm["K"])[None]
    y = api.moe_int4_decode(ctx, tier["dpool"], dev(x), dev(idx), dev(w), shared=None)
    ref = orc.moe_decode(dm, tier["pool"], None, x[0], idx[0], w[0].astype(np.float64))
    assert_out_close(f16_to_f64(y)[0], ref, "no shared")
    base = {k: v for k, v in tier["sh"].items() if not k.startswith(("a_", "b_"))}
    y = api.moe_int4_decode(ctx, tier["dpool"], dev(x), dev(idx), dev(w), shared=dev_tree(base))
    ref = orc.moe_decode(dm, tier["pool"], base, x[0], idx[0], w[0].astype(np.float64))
    assert_out_close(f16_to_f64(y)[0], ref, "no lora")


def test_moe_decode_through_slot_table(api, tier, orc):
    """Experts read through slot_of from a permuted slot pool match the id-indexed result."""
    dm, ctx = tier["dm"], tier["ctx"]
    rng = np.random.default_rng(9)
    announce("moe_int4_decode slot table", tier["name"])
    idx = synth.random_set(rng, dm["E"], dm["K"])
    n_slots = 2 * dm["K"]
    slots = rng.permutation(n_slots)[: dm["K"]]
    slot_of = np.full(dm["E"], -1, np.int32)
    slot_of[idx] = slots
    slot_pool = {}
    for k, v in tier["pool"].items():
        sp = np.zeros((n_slots,) + v.shape[1:], v.dtype)
        sp[slots] = v[idx]
        slot_pool[k] = sp
    x = rng.normal(size=(1, dm["d"])).astype(np.float16)
    w = synth.random_weights(rng, dm["K"])[None]
    y = api.moe_int4_decode(ctx, dev_tree(slot_pool), dev(x), dev(idx[None]), dev(w),
                            shared=tier["dsh"], slot_of=dev(slot_of), count=n_slots)
    y2 = api.moe_int4_decode(ctx, tier["dpool"], dev(x), dev(idx[None]), dev(w),
                             shared=tier["dsh"])
    assert np.array_equal(host(y), host(y2))
    ref = orc.moe_decode(dm, tier["pool"], tier["sh"], x[0], idx, w[0].astype(np.float64))
    assert_out_close(f16_to_f64(y)[0], ref, "slot table")


def test_moe_decode_bad_id_is_flagged(api, tier):
    dm, ctx = tier["dm"], tier["ctx"]
    announce("moe_int4_decode bad id", tier["name"])
    x = np.zeros((1, dm["d"]), np.float16)
    idx = np.array([[dm["E"] + 5] + list(range(dm["K"] - 1))], np.int32)
    w = np.full((1, dm["K"]), 1.0 / dm["K"], np.float32)
    api.moe_int4_decode(ctx, tier["dpool"], dev(x), dev(idx), dev(w), shared=tier["dsh"])
    assert api.device_status(ctx) == api.E0_ERR_RANGE
    assert api.device_status(ctx) == 0  # flags are cleared by the status call


def test_moe_decode_deterministic(api, tier):
    dm, ctx = tier["dm"], tier["ctx"]
    rng = np.random.default_rng(10)
    announce("moe_int4_decode determinism", tier["name"])
    x = dev(rng.normal(size=(2, dm["d"])).astype(np.float16))
    idx = dev(np.stack([synth.random_set(rng, dm["E"], dm["K"]) for _ in range(2)]))
    w = dev(np.stack([synth.random_weights(rng, dm["K"]) for _ in range(2)]))
    a = host(api.moe_int4_decode(ctx, tier["dpool"], x, idx, w, shared=tier["dsh"]))
    b = host(api.moe_int4_decode(ctx, tier["dpool"], x, idx, w, shared=tier["dsh"]))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_lora_delta_parity(api, tier, orc):
    import torch
    dm, ctx = tier["dm"], tier["ctx"]
    rng = np.random.default_rng(11)
    announce("lora_delta", tier["name"])
    sh = tier["sh"]
    c = dm["alpha"] / dm["r"]
    x = rng.normal(size=(2, dm["d"])).astype(np.float16)
    y0 = rng.normal(size=(2, dm["Is"])).astype(np.float32)
    yg = torch.from_numpy(y0.copy()).cuda()
    api.lora_delta(ctx, dev(sh["a_gate"]), dev(sh["b_gate"]), c, dev(x), yg)
    yg = host(yg).astype(np.float64)
    for b in range(2):
        ref = orc.lora_delta(sh["a_gate"], sh["b_gate"], dm["d"], dm["Is"], dm["r"], c,
                             x[b].astype(np.float64), y0[b].astype(np.float64))
        np.testing.assert_allclose(yg[b], ref, rtol=1e-5, atol=1e-6)


def _head_check(dm, orc, hd, x16, cur, prev, lg_gpu, idx_gpu, w_gpu, what):
    ref = orc.head_logits(hd["fc1"], hd["fc2"], hd["lin"], dm["d"], dm["E"], dm["P"], dm["K"],
                          x16, cur, prev, 1)
    np.testing.assert_allclose(lg_gpu, ref, rtol=0, atol=2e-4, err_msg=what)
    bias = hd.get("bias")
    assert routing_set_ok(dm, ref, idx_gpu, bias), f"{what}: routed set {idx_gpu}"
    oidx, ow = orc.route(dm, ref, bias)
    if list(oidx) == list(idx_gpu):
        np.testing.assert_allclose(w_gpu, ow, rtol=0, atol=W_TOL, err_msg=what)
    return ref


def test_prerouter_parity(api, tier, orc):
    import torch
    dm, ctx = tier["dm"], tier["ctx"]
    rng = np.random.default_rng(12)
    n = TIER_CASES[tier["name"]]
    announce("prerouter_forward", tier["name"], n)
    for case in range(n):
        B = 1 if case % 2 == 0 else 2
        x = rng.normal(size=(B, dm["d"])).astype(np.float16)
        cur = np.stack([synth.random_set(rng, dm["E"], dm["K"]) for _ in range(B)])
        prev = np.stack([synth.random_set(rng, dm["E"], dm["K"]) for _ in range(B)])
        first = case % 3 == 2
        logits = torch.empty((B, dm["E"]), dtype=torch.float32, device="cuda")
        oi, ow = api.prerouter_forward(ctx, tier["dhead"], dev(x), dev(cur),
                                       None if first else dev(prev), logits=logits)
        assert api.device_status(ctx) == 0
        lg, oi, ow = host(logits), host(oi), host(ow)
        for b in range(B):
            _head_check(dm, orc, tier["head"], x[b], cur[b], None if first else prev[b],
                        lg[b], oi[b], ow[b], f"{tier['name']} case {case} token {b}")
