"""Host checks of the seeded input generator (CPU only)."""
import numpy as np

import synth


def test_tiny_is_deterministic_float32():
    w = synth.WORKLOADS["tiny"]
    a, b = synth.make_logits(w), synth.make_logits(w)
    assert a.dtype == np.float32 and a.shape == (1, 16, 1024)
    assert np.array_equal(a, b)


def test_spiked_rows_have_three_spikes():
    w = synth.WORKLOADS["c1_qwen3_8b"]
    x = synth.bf16_bits_to_f32(synth.make_logits(w))
    assert x.shape == (1, 16, 151936)
    # a spike is N(0,1) + U[8,12]; plain N(0,1) draws essentially never pass 6
    big = (x > 6.0).sum(-1)
    assert np.all(big <= 3) and big.mean() > 2.9


def test_block_prefix_is_reproducible():
    w = synth.Workload("t", 3, 4, 300, 4, 64, 2, 256, 32, "bf16", "spiked")
    synth.WORKLOADS_ORDER.append("t")
    try:
        full = synth.make_logits(w)
        part = synth.make_logits(w, num_blocks=2)
    finally:
        synth.WORKLOADS_ORDER.remove("t")
    assert np.array_equal(full[:2], part)


def test_bf16_input_rounding():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0], dtype=np.float32)
    assert synth.bf16_bits_to_f32(synth.f32_to_bf16_bits_rne(x)).tolist() == [1.0, 1.0 + 2 ** -6, -0.0]


def test_head_inputs_are_seeded_and_prefix_stable():
    w = synth.WORKLOADS["paper_c32"]
    h, t = synth.make_head_inputs(w)
    assert h.shape == (32, 16, 4096) and t.shape == (32, 4096) and h.dtype == np.uint16
    h2, t2 = synth.make_head_inputs(w, num_blocks=3)
    assert np.array_equal(h[:3], h2) and np.array_equal(t[:3], t2)
    x = synth.bf16_bits_to_f32(t)
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1.0) < 0.01


def test_uniforms_and_temperatures():
    u = synth.make_uniforms(8, 16, seed=3)
    assert u.dtype == np.float32 and np.all((u >= 0) & (u < 1))
    t = synth.make_temperatures(9, seed=4)
    assert np.all(t[::4] == 0) and np.all((t[1:4] >= 0.5) & (t[1:4] < 1.5))
