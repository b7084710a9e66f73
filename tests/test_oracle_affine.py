"""Pins of the affine int4 codec (the pages' MLX format: unsigned nibbles,
bf16 group scale and bias, w = s q + b), CPU only:

* bfloat16 decoding against values fixed by the format (1, -2, 2^-7, the
  largest finite value, the smallest subnormal);
* a unit-scale, zero-bias probe: every dequantised weight is its nibble, read
  here by plain integer shifts;
* an identity with the symmetric codec, computed by the independent C++
  oracle: a symmetric matrix (two's-complement q, scale s) is the affine one
  with nibble q + 8, scale s and bias -8 s, so the same MoE decode agrees to
  fp64 rounding;
* the pages' byte counts ("1.77 MB" per expert, "453 MB" per layer,
  K-3): the library's affine bundle size.
"""

import numpy as np
import pytest

from sparse_moe_decode_amd import synth


def test_bf16_decode_fixed_values(orc):
    bits = np.array([0x3F80, 0xC000, 0x3C00, 0x7F7F, 0x0001, 0x0000, 0x8000], np.uint16)
    want = [1.0, -2.0, 2.0 ** -7, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133, 0.0, -0.0]
    got = orc.bf16_decode(bits)
    assert got.tolist() == want


def test_unit_scale_probe_reads_nibbles(orc):
    rng = np.random.default_rng(3)
    rows, cols, G = 5, 64, 32
    q = synth.random_words(rng, (rows, cols // 8))
    one = np.full((rows, cols // G), 0x3F80, np.uint16)
    zero = np.zeros((rows, cols // G), np.uint16)
    W = orc.q4_affine_dequant(q, one, zero, rows, cols, G)
    for o in range(rows):
        for i in range(cols):
            assert W[o, i] == (int(q[o, i // 8]) >> (4 * (i % 8))) & 0xF


def _as_affine(pool: dict, keys) -> dict:
    """Symmetric pool with bf16-exact fp16 scales -> the same weights in the
    affine codec."""
    out = dict(pool)
    for k in keys:
        s16 = pool[f"{k}_s"]
        sb = synth.bf16_bits(s16.astype(np.float32))
        out[f"{k}_q"] = pool[f"{k}_q"] ^ np.uint32(0x88888888)  # nibble -> nibble + 8 (mod 16)
        out[f"{k}_s"] = sb
        out[f"{k}_b"] = synth.bf16_bits(-8.0 * s16.astype(np.float32))
    return out


def _bf16_exact_scales(pool: dict, keys):
    for k in keys:
        s = pool[f"{k}_s"].astype(np.float32)
        pool[f"{k}_s"] = (synth.bf16_bits(s).astype(np.uint32) << 16).view(np.float32).astype(np.float16)


@pytest.mark.parametrize("tier", ["tiny", "35b"])
def test_affine_matches_symmetric_identity(orc, tier):
    dm = synth.dims(tier)
    rng = synth.rng_for(21, len(tier))
    keys = ("gate", "up", "down")
    pool = synth.routed_pool(rng, dm, n=6)
    sh = synth.shared_expert(rng, dm)
    _bf16_exact_scales(pool, keys)
    _bf16_exact_scales(sh, keys)
    apool, ash = _as_affine(pool, keys), _as_affine(sh, keys)
    x = rng.normal(size=dm["d"]).astype(np.float16)
    idx = np.arange(dm["K"], dtype=np.int32)
    w = rng.dirichlet(np.ones(dm["K"]))
    ref = orc.moe_decode(dm, pool, sh, x, idx, w)
    got = orc.moe_decode_affine(dict(dm, quant=1), apool, ash, x, idx, w)
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


def test_pages_byte_counts():
    from sparse_moe_decode_amd import api
    e35 = api.bundle_bytes_of(synth.dims("35b", quant=1))
    assert e35 == 3 * 512 * 2048 // 2 + (3 * 512 * 2048 // 64) * 2 * 2 == 1_769_472
    assert e35 * 256 == 452_984_832
    assert api.bundle_bytes_of(synth.dims("8b", quant=1)) == 1_327_104


@pytest.mark.parametrize("tier", ["tiny", "8b"])
def test_affine_layer_step_matches_symmetric_identity(orc, tier):
    """The affine layer-step (routing, head and residual around the affine
    MoE) equals the C++ symmetric layer-step on the same weights, on a router
    layer with a head and on a predicted layer."""
    dm = synth.dims(tier)
    keys = ("gate", "up", "down")
    for l, role in enumerate([dict(router=True, head=True), dict(router=False, head=True)]):
        lw = synth.layer(23, l, dm, role)
        lw["routed"] = {k: v[:dm["E"]] for k, v in lw["routed"].items()}
        _bf16_exact_scales(lw["routed"], keys)
        _bf16_exact_scales(lw["shared"], keys)
        alw = dict(lw, routed=_as_affine(lw["routed"], keys), shared=_as_affine(lw["shared"], keys))
        sym = orc.LayerOracle(dm, lw)
        aff = orc.LayerOracleAffine(dict(dm, quant=1), alw)
        rng = synth.rng_for(24, l)
        h = rng.normal(size=dm["d"]).astype(np.float16)
        ri = synth.random_set(rng, dm["E"], dm["K"])
        rw = synth.random_weights(rng, dm["K"])
        prev = synth.random_set(rng, dm["E"], dm["K"])
        kw = {} if role["router"] else dict(route_idx=ri, route_w=rw)
        a, s = aff.step(h, prev_idx=prev, **kw), sym.step(h, prev_idx=prev, **kw)
        assert np.array_equal(a["x16"], s["x16"])
        assert list(a["exec_idx"]) == list(s["exec_idx"])
        np.testing.assert_allclose(a["exec_w"], s["exec_w"], rtol=1e-12)
        np.testing.assert_allclose(a["h_out"], s["h_out"], rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(a["head_logits"], s["head_logits"], rtol=1e-10, atol=1e-12)
        assert list(a["pred_idx"]) == list(s["pred_idx"])
        if role["router"]:
            np.testing.assert_allclose(a["router_logits"], s["router_logits"], rtol=1e-10,
                                       atol=1e-12)
