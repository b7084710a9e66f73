"""Properties of the seeded input generators (CPU only)."""

import numpy as np

from helpers import unpack_q4
from sparse_moe_decode_amd import synth


def test_random_words_uniform_codes():
    q = unpack_q4(synth.random_words(synth.rng_for(1), (512, 64)))
    counts = np.bincount(q.ravel() + 8, minlength=16)
    assert counts.min() > 0.9 * q.size / 16 and counts.max() < 1.1 * q.size / 16


def test_fold_min_code_is_zero_mean_and_exact():
    w = synth.random_words(synth.rng_for(2), (512, 64))
    q0 = unpack_q4(w)
    q1 = unpack_q4(synth.fold_min_code(w.copy()))
    assert np.array_equal(q1, np.where(q0 == -8, 0, q0))
    assert q1.min() == -7 and q1.max() == 7
    assert abs(q1.mean()) < 0.02


def test_layer_is_reproducible():
    dm = synth.dims("tiny")
    a = synth.layer(9, 3, dm, dict(router=True, head=True))
    b = synth.layer(9, 3, dm, dict(router=True, head=True))
    for k in ("gate_q", "down_s"):
        assert np.array_equal(a["routed"][k], b["routed"][k])
    assert np.array_equal(a["head"]["fc1"], b["head"]["fc1"])
    c = synth.layer(9, 4, dm, dict(router=True, head=True))
    assert not np.array_equal(a["routed"]["gate_q"], c["routed"]["gate_q"])


def test_markov_sets_overlap():
    sets = synth.markov_sets(np.random.default_rng(3), 256, 4, 2000, keep=0.7)
    ov = np.mean([len(set(sets[t]) & set(sets[t - 1])) / 4 for t in range(1, len(sets))])
    assert abs(ov - 0.7) < 0.03
    assert all(len(set(s)) == 4 for s in sets)
