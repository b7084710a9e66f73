"""GPU parity of the affine int4 codec (unsigned nibbles, bf16 group scale
and bias) against the fp64 oracle (oracle.moe_decode_affine).

moe_int4_decode on affine experts: the per-token GEMV kernels (B < 16) and
the grouped MFMA kernels (B >= 16: the 32-token chunk kernels, and the
64-token prefill kernels from 16 entries per expert on average) at 35B
shapes, 8B and tiny shapes, the shared expert with its LoRA, an expert pool
read through the bundle layout (scales then biases), and a bad id flagged.
Large batches are checked on evenly spaced sample tokens.
layer_step on affine layers runs on the persistent kernel (its affine
variant) and on the per-phase kernels; every layer-step is checked against
the affine layer oracle, re-anchored on the GPU's own inputs, on two-layer
stacks and on the full 35B stack.
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


def _tokens(rng, dm, B):
    x = rng.normal(size=(B, dm["d"]))
    x = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + 1e-6)
    idx = np.stack([synth.random_set(rng, dm["E"], dm["K"]) for _ in range(B)]).astype(np.int32)
    w = np.stack([synth.random_weights(rng, dm["K"]) for _ in range(B)]).astype(np.float32)
    return x.astype(np.float16), idx, w


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tier,B,bundles,n_check", [
    ("35b", 1, False, 1), ("35b", 4, False, 4), ("35b", 20, False, 20), ("8b", 2, False, 2),
    ("tiny", 3, False, 3), ("35b", 2, True, 2), ("35b", 64, False, 24), ("8b", 40, False, 16),
    ("35b", 1024, False, 16), ("8b", 256, False, 12), ("35b", 48, True, 12)])
def test_affine_moe_decode_matches_oracle(api, orc, tier, B, bundles, n_check):
    dm = synth.dims(tier, quant=1)
    announce("affine moe_int4_decode", tier, f"B={B} bundles={bundles}")
    rng = synth.rng_for(95, len(tier), B)
    n = min(dm["E"], 64)
    pool = synth.routed_pool(rng, dm, n=n)
    sh = synth.shared_expert(rng, dm)
    dmn = dict(dm, E=n)
    ctx = api.Context(dmn, max_tokens=max(B, 1))
    x, idx, w = _tokens(rng, dmn, B)
    if bundles:
        import torch
        bundle = ctx.bundle_bytes()
        packed = torch.from_numpy(api.pack_bundles(pool, dmn)).cuda()
        assert packed.shape[1] == bundle
        view = api.bundle_view(packed.data_ptr(), dmn)
        y = api.moe_int4_decode(ctx, view, dev(x), dev(idx), dev(w), shared=dev_tree(sh),
                                stride=bundle)
    else:
        y = api.moe_int4_decode(ctx, dev_tree(pool), dev(x), dev(idx), dev(w),
                                shared=dev_tree(sh))
    assert api.device_status(ctx) == 0
    yg = f16_to_f64(y)
    worst = 0.0
    for b in sorted(set(np.linspace(0, B - 1, n_check).round().astype(int).tolist())):
        ref = orc.moe_decode_affine(dmn, pool, sh, x[b], idx[b], w[b].astype(np.float64))
        assert_out_close(yg[b], ref, f"{tier} token {b}")
        worst = max(worst, out_err(yg[b], ref))
    print(f"affine {tier} B={B} bundles={bundles}: worst error ratio {worst:.3f}")
    ctx.close()


def test_affine_bad_id_is_flagged(api):
    dm = synth.dims("tiny", quant=1)
    announce("affine moe_int4_decode", "tiny", "bad id")
    rng = synth.rng_for(96)
    pool = synth.routed_pool(rng, dm)
    ctx = api.Context(dm, max_tokens=2)
    x, idx, w = _tokens(rng, dm, 2)
    idx[1, 0] = dm["E"] + 1
    api.moe_int4_decode(ctx, dev_tree(pool), dev(x), dev(idx), dev(w))
    assert api.device_status(ctx) == api.E0_ERR_RANGE
    ctx.close()


def _affine_stack(api, orc, tier, roles, T, path, seed, zero_mean=False):
    import torch
    from stack_check import StackChecker
    from sparse_moe_decode_amd import workloads as wl
    dm = synth.dims(tier, quant=1)
    L = len(roles)
    layers, keep = [], {}
    for l, role in enumerate(roles):
        lw = synth.layer(seed, l, dm, role, zero_mean=zero_mean)
        keep[l] = lw
        if L > 2:
            announce("upload", tier, f"layer {l}/{L}")
        layers.append(dict(routed=wl.tree_to_dev(lw["routed"]), shared=wl.tree_to_dev(lw["shared"]),
                           attn=dev(lw["attn"]),
                           router=None if lw["router"] is None else dev(lw["router"]),
                           router_bias=(None if lw["router_bias"] is None
                                        else dev(lw["router_bias"])),
                           head=wl.tree_to_dev(lw["head"])))
    ctx = api.Context(dm, max_tokens=1)
    model = api.Model(ctx, layers)
    model.set_path(api.PATH_PERSISTENT if path == "persistent" else api.PATH_PHASES)
    state = api.State(dm, L)
    idx0, w0 = wl.initial_routing(tier, seed, L)
    state.route_idx[0].copy_(torch.from_numpy(idx0))
    state.route_w[0].copy_(torch.from_numpy(w0))
    toks = wl.token_inputs(tier, seed, T, 0.5)
    checker = StackChecker(orc, tier, seed, roles, list(range(L)), keep, zero_mean, quant=1)
    prev_exec = None
    h = torch.empty((L + 1, dm["d"]), dtype=torch.float16, device="cuda")
    for t in range(T):
        announce("affine layer_step", tier, path, f"L={L}", f"token {t}")
        h[0].copy_(torch.from_numpy(toks[t]))
        api.layer_step(ctx, model, 0, L, state, t, h)
        assert api.device_status(ctx) == 0
        cur, nxt = t & 1, (t + 1) & 1
        exec_idx = host(state.exec_idx[cur]).copy()
        checker.check(t, host(h).copy(), host(state.x_trace).copy(), exec_idx,
                      host(state.exec_w[cur]).copy(), prev_exec,
                      host(state.route_idx[cur]).copy(), host(state.route_w[cur]).copy(),
                      host(state.route_idx[nxt]).copy(), host(state.route_w[nxt]).copy(),
                      host(state.head_logits).copy())
        prev_exec = exec_idx
    print(f"affine {tier} {path} L={L}: {checker.steps} layer-steps checked, worst error ratio "
          f"{checker.worst:.3f}, re-anchored router sets {checker.reanchored}")
    model.close()
    ctx.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tier,T,path", [("tiny", 8, "phases"), ("8b", 3, "phases"),
                                         ("35b", 3, "phases"), ("8b", 3, "persistent"),
                                         ("35b", 3, "persistent")])
def test_affine_layer_step_matches_oracle(api, orc, tier, T, path):
    """Layer 0 runs its router and owns a head predicting layer 1; layer 1
    consumes that prediction and owns a head with no consumer."""
    roles = [dict(router=True, head=True), dict(router=False, head=True)]
    _affine_stack(api, orc, tier, roles, T, path, seed=33)


@pytest.mark.timeout(900)
def test_affine_stack_35b_persistent(api, orc):
    """The full 35B stack (40 layers, heads on 6-38) with affine experts on
    the persistent kernel, the benchmark's launch configuration."""
    _affine_stack(api, orc, "35b", synth.stack_roles("35b"), 2, "persistent", seed=3,
                  zero_mean=True)
