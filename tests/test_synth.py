"""The seeded input generator: published SplitMix64 outputs, RNE rounding to
bf16, moments, and that any slice of a stream can be drawn on its own."""
import numpy as np

import synth

GOLD = 0x9E3779B97F4A7C15
M64 = (1 << 64) - 1


def test_splitmix64_reference_outputs():
    # First outputs of SplitMix64 seeded with 1234567 (the generator's
    # reference implementation by S. Vigna): state advances by the golden gamma.
    L = synth.lib()
    assert L.synth_mix64((1234567 + GOLD) & M64) == 6457827717110365317
    assert L.synth_mix64((1234567 + 2 * GOLD) & M64) == 3203168211198807973
    assert L.synth_mix64(GOLD) == 0xE220A8397B1DCDAF


def test_bf16_round_to_nearest_even():
    f = synth.lib().synth_f32_to_bf16
    as_f = lambda u: np.array([u], np.uint32).view(np.float32)[0]
    assert f(as_f(0x3F808000)) == 0x3F80  # tie -> even (down)
    assert f(as_f(0x3F818000)) == 0x3F82  # tie -> even (up)
    assert f(as_f(0x3F808001)) == 0x3F81  # above half -> up
    assert f(as_f(0x3F807FFF)) == 0x3F80  # below half -> down
    assert f(as_f(0x7F7FFFFF)) == 0x7F80  # rounds up to +inf
    assert f(np.float32(-1.5)) == 0xBFC0


def test_streams_are_deterministic_and_sliceable():
    a = synth.normal(7, 3, 1000, 0.5)
    b = synth.normal(7, 3, 1000, 0.5)
    assert np.array_equal(a, b)
    c = synth.normal(7, 3, 300, 0.5, offset=400)
    assert np.array_equal(a[400:700], c)
    assert not np.array_equal(a, synth.normal(7, 4, 1000, 0.5))
    assert not np.array_equal(a, synth.normal(8, 3, 1000, 0.5))
    h = synth.normal(7, 3, 1000, 0.5, dtype="bf16")
    w = synth.bf16_bits_to_f32(h)
    assert np.all(np.abs(w - a) <= np.abs(a) * 2.0 ** -8)


def test_gaussian_moments():
    a = synth.normal(0, 0, 2_000_000, 2.0).astype(np.float64)
    assert abs(a.mean()) < 0.01 and abs(a.std() - 2.0) < 0.01
    assert abs((a ** 3).mean()) < 0.05 and abs((a ** 4).mean() / 16.0 - 3.0) < 0.05


def test_configs_and_input_shapes():
    cfg = synth.CONFIGS["tiny-f32"]
    inp = synth.make_inputs(cfg)
    assert inp["x"].shape == (64, 128) and inp["x"].dtype == np.float32
    assert inp["w_router"].shape == (128, 8)
    assert inp["w_gate"].shape == (8, 256, 128) and inp["w_down"].shape == (8, 128, 256)
    sm = cfg.with_(d=64, f=128, dtype="bf16", name="s")
    inb = synth.make_inputs(sm)
    assert inb["w_up"].dtype == np.uint16
    assert np.array_equal(synth.make_tokens(sm, 10, 5), inb["x"][5:15])
    b = synth.router_bias(synth.CONFIGS["skewed-masked"])
    assert b[0] == 4.0 and b[3] == 4.0 and b[1] == 0 and np.all(b[44:] == -1e4) and b[43] == 0
