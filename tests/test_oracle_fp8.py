"""Pins of the oracle's 8-bit expert-weight quantization (OCP FP8 E4M3 codes,
one power-of-two scale per weight row; the reading is stated in
oracle/moe_oracle.h). Each check uses something other than the encoder's own
formula: values the E4M3 format fixes, a brute-force nearest-code search over
all 256 codes, the minimality of the scale, and exactness of dequantization."""
import math

import numpy as np
import pytest

import oracle
import synth


def finite_codes():
    return [c for c in range(256) if not math.isnan(oracle.fp8_value(c))]


def test_format_anchor_values():
    # OCP E4M3: bias 7, no infinities, S.1111.111 is NaN.
    assert oracle.fp8_value(0x00) == 0.0 and math.copysign(1, oracle.fp8_value(0x80)) < 0
    assert oracle.fp8_value(0x01) == 2.0 ** -9  # smallest subnormal
    assert oracle.fp8_value(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert oracle.fp8_value(0x08) == 2.0 ** -6  # smallest normal
    assert oracle.fp8_value(0x38) == 1.0
    assert oracle.fp8_value(0x7E) == 448.0  # largest finite
    assert math.isnan(oracle.fp8_value(0x7F)) and math.isnan(oracle.fp8_value(0xFF))
    assert len(finite_codes()) == 254
    pos = [oracle.fp8_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:])), "codes 0..0x7e strictly increasing"
    assert all(oracle.fp8_value(c | 0x80) == -oracle.fp8_value(c) for c in range(0x7F))


def brute_force_code(v: float) -> int:
    """Nearest finite E4M3 code to v; equal distance -> the even code (even
    mantissa); zero keeps the sign of v."""
    best = None
    for c in finite_codes():
        d = abs(oracle.fp8_value(c) - v)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    c = best[1]
    if oracle.fp8_value(c) == 0.0:
        c = 0x80 if math.copysign(1.0, v) < 0 else 0x00
    elif (c & 0x80) != (0x80 if v < 0 else 0):
        c ^= 0x80
    return c


def test_codes_are_the_nearest_value_ties_to_even():
    rng = np.random.default_rng(1)
    vals = list(rng.uniform(-448, 448, 300)) + list(rng.normal(0, 1e-2, 200))
    # exact midpoints between neighbouring codes (normal and subnormal range)
    for c in range(0, 0x7E):
        a, b = oracle.fp8_value(c), oracle.fp8_value(c + 1)
        vals += [(a + b) / 2, -(a + b) / 2]
    vals += [0.0, -0.0, 2.0 ** -11, -2.0 ** -11, 2.0 ** -10, 1.5 * 2.0 ** -10, 448.0, -448.0]
    # one row per value, padded with 448 so that the row scale is exactly 1
    w = np.array([[v, 448.0] for v in vals], dtype=np.float32)
    assert np.array_equal(w[:, 0].astype(np.float64), np.array(vals, dtype=np.float32).astype(np.float64))
    codes, scales = oracle.quantize_fp8(w)
    assert np.all(scales == 1.0)
    for v, c in zip(w[:, 0], codes[:, 0]):
        assert c == brute_force_code(float(v)), (float(v), int(c))


def test_row_scale_is_the_smallest_power_of_two():
    rng = np.random.default_rng(2)
    amaxes = [448.0, 448.0000001, 447.9, 224.0, 224.1, 1.0, 0.875, 0.8750001, 3e-3, 7.5e4]
    rows = []
    for a in amaxes:
        r = rng.uniform(-a, a, 64).astype(np.float32)
        r[5] = np.float32(a)
        rows.append(r)
    w = np.stack(rows)
    codes, scales = oracle.quantize_fp8(w)
    for r, s in zip(w, scales):
        a = float(np.max(np.abs(r.astype(np.float64))))
        e = math.log2(float(s))
        assert e == int(e), "power of two"
        assert a <= 448.0 * s and a > 448.0 * s / 2, (a, s)
    zero = np.zeros((2, 8), dtype=np.float32)
    codes, scales = oracle.quantize_fp8(zero)
    assert np.all(scales == 1.0) and np.all(codes == 0)


def test_dequantize_is_exact_and_within_half_a_step():
    cfg = synth.LayerConfig("q", 4, 256, 2, 1, 128, "bf16")
    w = synth.make_inputs(cfg)["w_gate"].reshape(-1, 256)
    codes, scales = oracle.quantize_fp8(w)
    dq = oracle.dequantize_fp8(codes, scales)
    wv = synth.bf16_bits_to_f32(w).astype(np.float64)
    dv = synth.bf16_bits_to_f32(dq).astype(np.float64)
    vals = np.vectorize(oracle.fp8_value)(codes)
    assert np.array_equal(dv, vals * scales[:, None].astype(np.float64))
    # rounding error: at most half a step of the E4M3 grid at that magnitude
    t = np.abs(wv) / scales[:, None]
    step = np.where(t < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(t, 2.0 ** -6))) - 3))
    assert np.all(np.abs(dv - wv) <= 0.5 * step * scales[:, None] * (1 + 1e-12))
    assert np.all(np.sign(dv) * np.sign(wv) >= 0)


def test_quantized_layer_is_the_layer_on_dequantized_weights():
    cfg = synth.LayerConfig("q", 8, 128, 4, 2, 128, "bf16")
    inp = synth.make_inputs(cfg)
    q = oracle.quantized_expert_weights(inp)
    for name in ("w_gate", "w_up", "w_down"):
        E, rows, cols = inp[name].shape
        codes, scales = oracle.quantize_fp8(inp[name].reshape(E * rows, cols))
        assert np.array_equal(q[name], oracle.dequantize_fp8(codes, scales).reshape(E, rows, cols))
        assert not np.array_equal(q[name], inp[name])
    assert np.array_equal(q["w_router"], inp["w_router"]) and np.array_equal(q["x"], inp["x"])
    L = oracle.Layer.from_inputs(q, cfg.k)
    y = L.forward(q["x"])
    y0 = oracle.Layer.from_inputs(inp, cfg.k).forward(inp["x"])
    rel = np.max(np.abs(y - y0)) / np.max(np.abs(y0))
    assert 0 < rel < 0.1, rel


def test_invalid_arguments():
    with pytest.raises(Exception):
        oracle.quantize_fp8(np.zeros((0, 4), dtype=np.float32))
