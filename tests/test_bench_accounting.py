"""Algorithmic byte counts used by bench.py's roofline figures.

The weight bytes a decode step must read follow from the tier shapes
("The Other Half of the Memory Wall" §3.1 and §3.2; the byte audit "I counted
the bytes it can't stream", MoESpec listing). These pin bench.py's formulas to
the totals worked out by hand from those shapes: expert bundle 1,671,168 B
(35B) and 1,253,376 B (8B); head 2,097,152 parameters dense, read over the d
dense columns and the 2K gathered one-hot columns; 33 heads, 32 predicted and
8 router layers in the 35B stack.
"""

import bench
from sparse_moe_decode_amd import synth


def test_expert_bundle_bytes_match_the_tier_shapes():
    for tier, want in (("35b", 1_671_168), ("8b", 1_253_376)):
        dm = synth.dims(tier)
        d, I, G = dm["d"], dm["I"], dm["G"]
        assert 3 * (I * d // 2) + 3 * 2 * (I * d // G) == want


def test_layer_step_bytes():
    # K experts + shared expert + LoRA + head read over d + 2K columns
    assert bench.layer_step_bytes(synth.dims("35b")) == 12_021_760
    assert bench.layer_step_bytes(synth.dims("8b")) == 13_594_624


def test_stack_token_bytes():
    parts = bench.algorithmic_bytes(synth.dims("35b"), synth.stack_roles("35b"))
    assert parts["routed"] == 40 * 4 * 1_671_168
    assert parts["shared"] == 40 * 1_671_168
    assert parts["lora"] == 40 * 245_760
    assert parts["heads"] == 33 * 3_420_160
    assert parts["routers"] == 8 * 2 * 256 * 2048
    assert parts["total"] == 465_317_888


def test_stack_token_bytes_affine():
    # the affine codec adds a bf16 bias per scale: 1,769,472 B per expert
    parts = bench.algorithmic_bytes(synth.dims("35b", quant=1), synth.stack_roles("35b"))
    assert parts["routed"] == 40 * 4 * 1_769_472
    assert parts["shared"] == 40 * 1_769_472
    assert parts["total"] == 465_317_888 + 200 * (1_769_472 - 1_671_168)
