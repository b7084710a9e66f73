"""Pins of the oracle's numeric building blocks (CPU only).

Each check compares the oracle with something other than itself: numpy's
binary16 conversion, torch's fp64 SiLU / GELU / RMSNorm, an independent
numpy int4 unpacker, closed forms and exactness arguments.
"""

import numpy as np
import pytest
import torch

from helpers import dequant_ref, pack_q4, unpack_q4

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_f16_round_matches_numpy(orc):
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.normal(0, 1, 20000),
        rng.normal(0, 1e-5, 5000),            # subnormal range
        rng.normal(0, 3e4, 5000),             # near the top of the range
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -24,
                  2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -14, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, 2048.0 + 1.0, 2048.0 + 3.0]),
    ])
    got = orc.f16_round(vals)
    want = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_f16_decode_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint16)
    got = orc.f16_decode(bits)
    want = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(want)
    assert np.array_equal(got[finite], want[finite])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(np.isinf(got), np.isinf(want))


def test_q4_unit_vector_probe(orc):
    """Scale 1 and x = e_i recover column i of the integer matrix exactly."""
    rng = np.random.default_rng(1)
    rows, cols, G = 24, 64, 32
    Q = rng.integers(-8, 8, size=(rows, cols))
    words = pack_q4(Q)
    scales = np.ones((rows, cols // G), np.float16)
    for i in range(cols):
        x = np.zeros(cols)
        x[i] = 1.0
        y = orc.q4_matvec(words, scales, rows, cols, G, x)
        assert np.array_equal(y, Q[:, i].astype(np.float64)), f"column {i}"


def test_q4_nibble_order_and_sign(orc):
    """Word 0x76543210 holds 0..7, word 0xFEDCBA98 holds -8..-1 (low nibble first)."""
    words = np.array([[0x76543210, 0xFEDCBA98]], np.uint32)
    scales = np.ones((1, 1), np.float16)
    w = orc.q4_dequant(words, scales, 1, 16, 16)
    assert w[0].tolist() == [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]


def test_q4_dequant_exact_against_numpy_unpack(orc):
    rng = np.random.default_rng(2)
    rows, cols, G = 16, 256, 64
    words = rng.integers(0, 2 ** 32, size=(rows, cols // 8), dtype=np.uint64).astype(np.uint32)
    scales = (np.abs(rng.normal(0, 0.02, (rows, cols // G))) + 1e-3).astype(np.float16)
    got = orc.q4_dequant(words, scales, rows, cols, G)
    assert np.array_equal(got, dequant_ref(words, scales, G))
    # Every weight is exactly scale * q with q in [-8, 7].
    q = unpack_q4(words)
    assert q.min() >= -8 and q.max() <= 7
    x = rng.normal(size=cols)
    y = orc.q4_matvec(words, scales, rows, cols, G, x)
    np.testing.assert_allclose(y, dequant_ref(words, scales, G) @ x, rtol=1e-12, atol=1e-12)


def test_silu_gelu_match_torch(orc):
    z = np.linspace(-30, 30, 4001)
    z = np.concatenate([z, np.random.default_rng(3).normal(0, 3, 4000)])
    zt = torch.from_numpy(z)
    np.testing.assert_allclose(orc.silu(z), torch.nn.functional.silu(zt).numpy(),
                               rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(orc.gelu_erf(z),
                               torch.nn.functional.gelu(zt, approximate="none").numpy(),
                               rtol=1e-12, atol=1e-15)


def test_gelu_identities(orc):
    z = np.random.default_rng(4).normal(0, 2, 1000)
    g, gm = orc.gelu_erf(z), orc.gelu_erf(-z)
    np.testing.assert_allclose(g - gm, z, rtol=1e-13, atol=1e-15)  # gelu(z) - gelu(-z) = z
    assert orc.gelu_erf(np.zeros(1))[0] == 0.0


def test_rmsnorm_matches_torch(orc):
    rng = np.random.default_rng(5)
    for d in (64, 1536, 2048):
        h = rng.normal(0, 7, d)
        got = orc.rmsnorm(h, 1e-6)
        want = torch.nn.functional.rms_norm(torch.from_numpy(h), (d,), eps=1e-6).numpy()
        np.testing.assert_allclose(got, want, rtol=1e-13)
        assert abs(np.mean(got ** 2) - 1.0) < 1e-6
