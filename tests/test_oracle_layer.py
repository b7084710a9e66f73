"""Pins of the oracle's expert, LoRA, head and layer-step functions (CPU only).

References used: the dequantised dense reference the method's math contract
names ("The Other Half of the Memory Wall", §3.1 Math contract) built from an
independent numpy unpacker with torch's fp64 SiLU/GELU; the LoRA merge
identity (§3.3); the head's warm-start special case (§3.2 Head); one-hot block
probes; and the shapes and counts the pages print (tests/golden).
"""

import json
import os

import numpy as np
import pytest
import torch

from helpers import dequant_ref
from sparse_moe_decode_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def _silu(z):
    return torch.nn.functional.silu(torch.from_numpy(z)).numpy()


def _gelu(z):
    return torch.nn.functional.gelu(torch.from_numpy(z), approximate="none").numpy()


def _f(a):
    return np.asarray(a).astype(np.float64)


def _dense_expert(p, e, G, x):
    Wg = dequant_ref(p["gate_q"][e], p["gate_s"][e], G)
    Wu = dequant_ref(p["up_q"][e], p["up_s"][e], G)
    Wd = dequant_ref(p["down_q"][e], p["down_s"][e], G)
    return Wd @ (_silu(Wg @ x) * (Wu @ x))


def _merged(W, A, B, c):
    return W + c * (_f(B) @ _f(A))


def _dense_shared(sh, G, c, x, lora=True):
    Wg = dequant_ref(sh["gate_q"], sh["gate_s"], G)
    Wu = dequant_ref(sh["up_q"], sh["up_s"], G)
    Wd = dequant_ref(sh["down_q"], sh["down_s"], G)
    if lora:
        Wg = _merged(Wg, sh["a_gate"], sh["b_gate"], c)
        Wu = _merged(Wu, sh["a_up"], sh["b_up"], c)
        Wd = _merged(Wd, sh["a_down"], sh["b_down"], c)
    return Wd @ (_silu(Wg @ x) * (Wu @ x))


@pytest.fixture(scope="module")
def tiny():
    dm = synth.dims("tiny")
    rng = synth.rng_for(100)
    return dm, synth.routed_pool(rng, dm), synth.shared_expert(rng, dm)


def test_expert_matches_dequantised_reference(orc, tiny):
    dm, pool, _ = tiny
    x = np.random.default_rng(1).normal(size=dm["d"])
    for e in range(dm["E"]):
        y = orc.expert(pool["gate_q"][e], pool["gate_s"][e], pool["up_q"][e], pool["up_s"][e],
                       pool["down_q"][e], pool["down_s"][e], dm["d"], dm["I"], dm["G"], x)
        np.testing.assert_allclose(y, _dense_expert(pool, e, dm["G"], x), rtol=1e-11, atol=1e-12)


def test_gate_up_swap_is_detected(orc, tiny):
    """Negative control: swapping gate and up must break the tolerance badly."""
    dm, pool, _ = tiny
    x = np.random.default_rng(2).normal(size=dm["d"])
    a = [pool[k][0] for k in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")]
    y = orc.expert(*a, dm["d"], dm["I"], dm["G"], x)
    ys = orc.expert(a[2], a[3], a[0], a[1], a[4], a[5], dm["d"], dm["I"], dm["G"], x)
    rel = np.linalg.norm(ys - y) / np.linalg.norm(y)
    assert rel > 0.5


def test_expert_zero_input(orc, tiny):
    dm, pool, _ = tiny
    a = [pool[k][1] for k in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")]
    y = orc.expert(*a, dm["d"], dm["I"], dm["G"], np.zeros(dm["d"]))
    assert np.all(y == 0.0)


def test_lora_merge_identity(orc):
    """Unmerged W x + (a/r) B A x equals (W + (a/r) B A) x merged in fp64."""
    dm = synth.dims("35b")
    rng = synth.rng_for(101)
    d, Is, G, r = dm["d"], dm["Is"], dm["G"], dm["r"]
    c = dm["alpha"] / r
    q, s = synth.q4_matrix(rng, Is, d, G)
    A, B = synth.f16_normal(rng, (r, d), 0.01), synth.f16_normal(rng, (Is, r), 0.01)
    x = rng.normal(size=d)
    base = orc.q4_matvec(q, s, Is, d, G, x)
    y = orc.lora_delta(A, B, d, Is, r, c, x, base)
    want = _merged(dequant_ref(q, s, G), A, B, c) @ x
    np.testing.assert_allclose(y, want, rtol=1e-10, atol=1e-10)
    # B = 0 leaves the base untouched.
    y0 = orc.lora_delta(A, np.zeros_like(B), d, Is, r, c, x, base)
    assert np.array_equal(y0, base)
    # Weight-level delta RMS of the synthetic adapter sits near the pages' 1e-3.
    delta = c * (_f(B) @ _f(A))
    assert 3e-4 < np.sqrt(np.mean(delta ** 2)) < 3e-3


def test_shared_expert_matches_merged_dense(orc):
    dm = synth.dims("tiny")
    sh = synth.shared_expert(synth.rng_for(102), dm)
    c = dm["alpha"] / dm["r"]
    x = np.random.default_rng(3).normal(size=dm["d"])
    y = orc.shared_expert(sh, dm["d"], dm["Is"], dm["G"], dm["r"], dm["alpha"], x)
    np.testing.assert_allclose(y, _dense_shared(sh, dm["G"], c, x), rtol=1e-10, atol=1e-11)
    base = {k: v for k, v in sh.items() if not k.startswith(("a_", "b_"))}
    y0 = orc.shared_expert(base, dm["d"], dm["Is"], dm["G"], dm["r"], dm["alpha"], x)
    np.testing.assert_allclose(y0, _dense_shared(sh, dm["G"], c, x, lora=False),
                               rtol=1e-10, atol=1e-11)


def test_moe_decode_combine(orc, tiny):
    dm, pool, sh = tiny
    rng = np.random.default_rng(4)
    x16 = rng.normal(size=dm["d"]).astype(np.float16)
    x = x16.astype(np.float64)
    c = dm["alpha"] / dm["r"]
    idx = np.array([5, 2], np.int32)
    w = np.array([0.7, 0.3])
    y = orc.moe_decode(dm, pool, sh, x16, idx, w)
    want = 0.7 * _dense_expert(pool, 5, dm["G"], x) + 0.3 * _dense_expert(pool, 2, dm["G"], x)
    want += _dense_shared(sh, dm["G"], c, x)
    np.testing.assert_allclose(y, want, rtol=1e-10, atol=1e-10)
    # One-hot weights reduce to a single expert plus the shared expert.
    y1 = orc.moe_decode(dm, pool, sh, x16, idx, np.array([1.0, 0.0]))
    np.testing.assert_allclose(y1, _dense_expert(pool, 5, dm["G"], x)
                               + _dense_shared(sh, dm["G"], c, x), rtol=1e-10, atol=1e-10)
    # No shared expert: routed part only.
    y2 = orc.moe_decode(dm, pool, None, x16, idx, w)
    np.testing.assert_allclose(y2, want - _dense_shared(sh, dm["G"], c, x), rtol=1e-9, atol=1e-9)
    with pytest.raises(ValueError):
        orc.moe_decode(dm, pool, sh, x16, np.array([0, dm["E"]], np.int32), w)


def _head_dims():
    return dict(d=64, E=8, P=12, K=2)


def test_head_warm_start_equals_next_router(orc):
    """fc1 = fc2 = 0 and lin = [W_router | 0 | 0]: the head is the next layer's router."""
    dm = _head_dims()
    d, E, P, K = dm["d"], dm["E"], dm["P"], dm["K"]
    rng = np.random.default_rng(5)
    Wr = rng.normal(0, 0.05, (E, d)).astype(np.float16)
    lin = np.zeros((E, d + 2 * E), np.float16)
    lin[:, :d] = Wr
    fc1 = np.zeros((P, d + 2 * E), np.float16)
    fc2 = np.zeros((E, P), np.float16)
    x16 = rng.normal(size=d).astype(np.float16)
    for form in (0, 1):
        lg = orc.head_logits(fc1, fc2, lin, d, E, P, K, x16, [1, 6], [0, 3], form)
        np.testing.assert_allclose(lg, _f(Wr) @ _f(x16), rtol=1e-13, atol=1e-15)


def test_head_onehot_blocks(orc):
    """lin = [0 | I | 0] reads back onehot(cur); lin = [0 | 0 | I] reads onehot(prev)."""
    dm = _head_dims()
    d, E, P, K = dm["d"], dm["E"], dm["P"], dm["K"]
    fc1 = np.zeros((P, d + 2 * E), np.float16)
    fc2 = np.zeros((E, P), np.float16)
    x16 = np.random.default_rng(6).normal(size=d).astype(np.float16)
    cur, prev = [6, 1], [2, 7]
    for block, ids in ((1, cur), (2, prev)):
        lin = np.zeros((E, d + 2 * E), np.float16)
        lin[:, d + (block - 1) * E: d + block * E] = np.eye(E)
        want = np.zeros(E)
        want[ids] = 1.0
        for form in (0, 1):
            lg = orc.head_logits(fc1, fc2, lin, d, E, P, K, x16, cur, prev, form)
            assert np.array_equal(lg, want)
            lg0 = orc.head_logits(fc1, fc2, lin, d, E, P, K, x16, cur, None, form)
            assert np.array_equal(lg0, want if block == 1 else np.zeros(E))


def test_head_mlp_branch(orc):
    """lin = 0 and fc2 = [I | 0]: logits are erf-GELU of the first E fc1 outputs."""
    dm = _head_dims()
    d, E, P, K = dm["d"], dm["E"], dm["P"], dm["K"]
    rng = np.random.default_rng(7)
    fc1 = rng.normal(0, 0.1, (P, d + 2 * E)).astype(np.float16)
    fc2 = np.zeros((E, P), np.float16)
    fc2[:, :E] = np.eye(E)
    lin = np.zeros((E, d + 2 * E), np.float16)
    x16 = rng.normal(size=d).astype(np.float16)
    cur, prev = [3, 4], [0, 5]
    f = np.zeros(d + 2 * E)
    f[:d] = _f(x16)
    f[d + np.array(cur)] = 1.0
    f[d + E + np.array(prev)] = 1.0
    want = _gelu(_f(fc1) @ f)[:E]
    for form in (0, 1):
        lg = orc.head_logits(fc1, fc2, lin, d, E, P, K, x16, cur, prev, form)
        np.testing.assert_allclose(lg, want, rtol=1e-13, atol=1e-15)


def test_head_dense_equals_gather_and_library(orc):
    dm = synth.dims("tiny")
    hw = synth.head(synth.rng_for(103), dm)
    d, E, P, K = dm["d"], dm["E"], dm["P"], dm["K"]
    rng = np.random.default_rng(8)
    x16 = rng.normal(size=d).astype(np.float16)
    cur, prev = synth.random_set(rng, E, K), synth.random_set(rng, E, K)
    a = orc.head_logits(hw["fc1"], hw["fc2"], hw["lin"], d, E, P, K, x16, cur, prev, 0)
    b = orc.head_logits(hw["fc1"], hw["fc2"], hw["lin"], d, E, P, K, x16, cur, prev, 1)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    f = np.zeros(d + 2 * E)
    f[:d] = _f(x16)
    f[d + cur] = 1.0
    f[d + E + prev] = 1.0
    want = _f(hw["lin"]) @ f + _f(hw["fc2"]) @ _gelu(_f(hw["fc1"]) @ f)
    np.testing.assert_allclose(a, want, rtol=1e-12, atol=1e-14)
    with pytest.raises(ValueError):
        orc.head_logits(hw["fc1"], hw["fc2"], hw["lin"], d, E, P, K, x16, [1, 1], prev, 1)


def test_page_shapes_and_bytes():
    """Tier shapes reproduce the head and expert sizes the pages print."""
    for tier, key in (("35b", "35b"), ("8b", "8b")):
        dm = synth.dims(tier)
        hw = synth.head(synth.rng_for(0), dm)
        assert hw["fc1"].shape[1] == GOLD[f"feature_dim_{key}"]["value"]
        assert list(hw["fc1"].shape) == GOLD[f"fc1_shape_{key}"]["value"]
        assert dm["P"] == GOLD["head_hidden"]["value"]
    dm = synth.dims("35b")
    hw = synth.head(synth.rng_for(0), dm)
    n = hw["fc1"].size + hw["fc2"].size + hw["lin"].size
    assert n == GOLD["head_params_35b"]["value"]
    n_heads = len(synth.STACKS["35b"]["head_layers"])
    assert n * n_heads == GOLD["head_params_all_35b"]["value"]
    assert 2 * n * n_heads == GOLD["head_bytes_all_35b"]["value"]
    # The pages' affine format carries a bias array the size of the scales.
    for tier in ("35b", "8b"):
        dm = synth.dims(tier)
        p = synth.routed_pool(synth.rng_for(0), dm, n=1)
        qb = sum(p[k].nbytes for k in ("gate_q", "up_q", "down_q"))
        sb = sum(p[k].nbytes for k in ("gate_s", "up_s", "down_s"))
        affine = qb + 2 * sb
        if tier == "35b":
            assert round(affine / 1e6, 2) == GOLD["expert_bytes_affine_35b_MB"]["value"]
            assert round(affine * dm["E"] / 1e6) == GOLD["layer_expert_bytes_affine_35b_MB"]["value"]
            assert round(affine * dm["E"] * 40 / 2 ** 30, 1) == \
                GOLD["routed_expert_GiB_affine_35b"]["value"]
        else:
            assert affine == GOLD["expert_bytes_affine_8b"]["value"]
    spec = GOLD["moespec_35b"]["value"]
    dm = synth.dims("35b")
    assert (dm["E"], dm["K"], dm["I"], dm["G"]) == (spec["num_experts"], spec["top_k"],
                                                    spec["intermediate_size"], spec["group_size"])
    sg = GOLD["sigmoid_group_8b"]["value"]
    dm = synth.dims("8b")
    assert (dm["n_groups"], dm["topk_groups"], dm["route_scale"], dm["K"]) == \
        (sg["n"], sg["G"], sg["s"], sg["K"])
    assert (dm["r"], dm["alpha"]) == (GOLD["lora"]["value"]["r"], GOLD["lora"]["value"]["alpha"])


def test_stack_schedule_counts():
    for tier, hk, ck in (("35b", "heads_35b", "consumers_35b"), ("8b", "heads_8b", "consumers_8b")):
        roles = synth.stack_roles(tier)
        assert len(roles) == GOLD[ck]["layers"]
        heads = [l for l, r in enumerate(roles) if r["head"]]
        cons = [l for l, r in enumerate(roles) if not r["router"]]
        assert len(heads) == GOLD[hk]["value"]
        assert [heads[0], heads[-1]] == GOLD[hk]["owners"]
        assert len(cons) == GOLD[ck]["value"]
        assert (cons[0], cons[-1]) == (GOLD[ck]["first"], GOLD[ck]["last"])
        # Every consumer layer l is predicted by the head owned by layer l-1.
        assert all(roles[l - 1]["head"] for l in cons)
    assert 3 * GOLD["heads_8b"]["value"] == GOLD["head_tensors_8b"]["value"]


def _layer_fixture(tier, role, seed=104):
    dm = synth.dims(tier)
    return dm, synth.layer(seed, 0, dm, role)


@pytest.mark.parametrize("tier", ["tiny", "8b"])
def test_layer_step_router_layer(orc, tier):
    """Router layer with a head: norm, routing, MoE, residual and prediction compose."""
    dm, lw = _layer_fixture(tier, dict(router=True, head=True))
    rng = np.random.default_rng(9)
    h16 = rng.normal(size=dm["d"]).astype(np.float16)
    prev = synth.random_set(rng, dm["E"], dm["K"])
    lo = orc.LayerOracle(dm, lw)
    out = lo.step(h16, prev_idx=prev)
    ha = _f(h16) + _f(lw["attn"])
    xn = torch.nn.functional.rms_norm(torch.from_numpy(ha), (dm["d"],), eps=dm["eps"]).numpy()
    assert np.array_equal(out["x16"], xn.astype(np.float16).view(np.uint16))
    x = _f(out["x16"].view(np.float16))
    lg = _f(lw["router"]) @ x
    np.testing.assert_allclose(out["router_logits"], lg, rtol=1e-12, atol=1e-13)
    idx, w = orc.route(dm, lg, lw["router_bias"])
    assert out["exec_idx"].tolist() == idx.tolist()
    y = orc.moe_decode(dm, lw["routed"], lw["shared"], out["x16"], idx, w)
    np.testing.assert_allclose(out["h_out"], ha + y, rtol=1e-12, atol=1e-12)
    hl = orc.head_logits(lw["head"]["fc1"], lw["head"]["fc2"], lw["head"]["lin"], dm["d"],
                         dm["E"], dm["P"], dm["K"], out["x16"], idx, prev, 0)
    np.testing.assert_allclose(out["head_logits"], hl, rtol=1e-12, atol=1e-13)
    pidx, pw = orc.route(dm, hl, lw["head"].get("bias"))
    assert out["pred_idx"].tolist() == pidx.tolist()
    np.testing.assert_allclose(out["pred_w"], pw, rtol=1e-12)


def test_layer_step_consumer_zero_experts(orc):
    """All expert scales zero and no adapter: h_out = h + attn exactly."""
    dm, lw = _layer_fixture("tiny", dict(router=False, head=False))
    lw["shared"] = {k: v for k, v in lw["shared"].items() if not k.startswith(("a_", "b_"))}
    for part in ("routed", "shared"):
        for k in list(lw[part]):
            if k.endswith("_s"):
                lw[part][k] = np.zeros_like(lw[part][k])
    h16 = np.random.default_rng(10).normal(size=dm["d"]).astype(np.float16)
    idx = np.array([3, 0], np.int32)
    w = np.array([0.25, 0.75], np.float32)
    out = orc.LayerOracle(dm, lw).step(h16, idx, w)
    np.testing.assert_allclose(out["h_out"], _f(h16) + _f(lw["attn"]), rtol=1e-12, atol=1e-12)
    assert out["exec_idx"].tolist() == [3, 0]
    np.testing.assert_allclose(out["exec_w"], w.astype(np.float64))
