"""The seeded input generator (no GPU): determinism, distribution and bf16 rounding."""
import numpy as np

import synth


def test_bf16_rounding_ties_to_even():
    assert synth.bf16_from_double(1.0) == 0x3F80
    assert synth.bf16_from_double(-2.0) == 0xC000
    assert synth.bf16_from_double(1.0 + 2.0 ** -8) == 0x3F80          # tie -> even (down)
    assert synth.bf16_from_double(1.0 + 3 * 2.0 ** -8) == 0x3F82      # tie -> even (up)
    assert synth.bf16_from_double(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81  # above the tie
    assert synth.bf16_from_double(0.0) == 0 and synth.bf16_from_double(-0.0) == 0x8000
    assert synth.bf16_from_double(1e-40) == 0


def test_generator_is_deterministic_and_keyed():
    a = synth.normal_bf16(3, 1, (4, 1000))
    b = synth.normal_bf16(3, 1, (4, 1000))
    c = synth.normal_bf16(3, 2, (4, 1000))
    d = synth.normal_bf16(4, 1, (4, 1000))
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)
    # counter based: a prefix of a longer stream is the shorter stream
    e = synth.normal_bf16(3, 1, (4001,)).ravel()
    assert np.array_equal(e[:4000], a.ravel())


def test_generator_distribution():
    x = synth.bf16_bits_to_f32(synth.normal_bf16(9, 0, (1 << 20,))).astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    assert abs(np.mean(np.abs(x) < 1.0) - 0.6827) < 3e-3
    u = synth.uniforms(9, 0, 100000)
    assert u.min() >= 0.0 and u.max() < 1.0 and abs(u.mean() - 0.5) < 5e-3


def test_half_multiplier_is_exact():
    a = synth.bf16_bits_to_f32(synth.normal_bf16(5, 2, (10000,)))
    b = synth.bf16_bits_to_f32(synth.normal_bf16(5, 2, (10000,), mult=0.5))
    assert np.array_equal(a * 0.5, b)


def test_workload_shapes():
    w = synth.WORKLOADS["gqa_decode"]
    assert (w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Sk"], w["d"]) == (8, 32, 8, 1, 32768, 128)
    assert synth.WORKLOADS["causal_prefill"]["scale"] == np.float32(1 / np.sqrt(128))
