"""Pins of the oracle's 8-bit expert-weight quantization (OCP FP8 E4M3 codes,
one power-of-two scale per weight row; the reading is stated in
oracle/moe_oracle.h). Each check uses something other than the encoder's own
formula: values the E4M3 format fixes, a brute-force nearest-code search over
all 256 codes, the minimality of the scale, and exactness of dequantization.
The optional 8-bit activation mode (the token row enters the gate and up
products 8-bit quantized; h and the down product keep the layer's precision) is
pinned by recomputing an expert FFN with those brute-force pieces and numpy,
by its routing on full-precision x, and by constructed rows where quantizing h,
or rounding x before quantizing it, would change the result."""
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


# --- 8-bit activations (the oracle's MOE_ORACLE_ACT_FP8 mode) -----------------

def brute_force_row(vals):
    """8-bit row quantization by search: the smallest power of two 2^e
    (e >= -126) with max|v| <= 448 * 2^e, then every value's nearest code by
    brute force. Returns the dequantized values."""
    amax = max(abs(v) for v in vals)
    e = -126
    while amax > 448.0 * 2.0 ** e:
        e += 1
    if amax == 0.0:
        e = 0
    return [oracle.fp8_value(brute_force_code(v / 2.0 ** e)) * 2.0 ** e for v in vals]


def test_act_fp8_expert_ffn_by_brute_force():
    cfg = synth.LayerConfig("q8", 6, 32, 3, 2, 16, "bf16")
    inp = oracle.quantized_expert_weights(synth.make_inputs(cfg))
    L = oracle.Layer.from_inputs(inp, cfg.k)
    wg = synth.bf16_bits_to_f32(inp["w_gate"]).astype(np.float64)
    wu = synth.bf16_bits_to_f32(inp["w_up"]).astype(np.float64)
    wd = synth.bf16_bits_to_f32(inp["w_down"]).astype(np.float64)
    for t in range(cfg.T):
        xrow = inp["x"][t]
        xq = np.array(brute_force_row(list(synth.bf16_bits_to_f32(xrow).astype(np.float64))))
        for e in range(cfg.E):
            g, u = wg[e] @ xq, wu[e] @ xq
            h = g / (1.0 + np.exp(-g)) * u
            want = wd[e] @ h
            out, h_or = L.expert_ffn(e, xrow, want_h=True, act_fp8=True)
            assert np.allclose(h_or, h, rtol=1e-13, atol=1e-15), (t, e)
            assert np.allclose(out, want, rtol=1e-12, atol=1e-14), (t, e)
            # the mode changes the result (else this pin would be vacuous)
            assert not np.allclose(out, L.expert_ffn(e, xrow), rtol=1e-6, atol=0)


def test_act_fp8_routes_on_full_precision_x():
    cfg = synth.LayerConfig("q8r", 40, 64, 8, 2, 32, "bf16")
    inp = oracle.quantized_expert_weights(synth.make_inputs(cfg))
    L = oracle.Layer.from_inputs(inp, cfg.k)
    x = inp["x"]
    y = L.forward(x, act_fp8=True)
    ids, _, w64 = oracle.topk(L.router(x), cfg.k)
    for t in range(cfg.T):
        ref = sum(w64[t, j] * L.expert_ffn(int(ids[t, j]), x[t], act_fp8=True) for j in range(cfg.k))
        assert np.allclose(y[t], ref, rtol=1e-13, atol=1e-15), t
    y0 = L.forward(x)
    rel = np.max(np.abs(y - y0)) / np.max(np.abs(y0))
    assert 1e-3 < rel < 0.2, rel


def test_act_fp8_constructed_rounding_order():
    """x is quantized as given (not rounded to bf16 first); h is not quantized.
    fp32 layer, one expert, d = f = 2, identity down projection. Gate
    pre-activations of 64 make SiLU exact (SiLU(64) = 64 in double), so h is
    64 * up exactly."""
    f32 = np.float32
    small = 1.0625 + 2.0 ** -12  # just above the midpoint of codes 1.0 and 1.125
    wr = np.ones((2, 1), f32)
    wd = np.eye(2, dtype=f32)[None]
    # 1) x = [1, 0] -> xq = x; h = [64*7, 64*small/64] = [448, small]: h keeps
    #    its value (quantized it would be [448, 1.125]; rounded to bf16 first,
    #    [448, 1.0]).
    L = oracle.Layer(wr, None, np.array([[[64.0, 0.0], [64.0, 0.0]]], f32),
                     np.array([[[7.0, 0.0], [small / 64.0, 0.0]]], f32), wd, 1)
    x = np.array([1.0, 0.0], f32)
    out, h = L.expert_ffn(0, x, want_h=True, act_fp8=True)
    assert list(h) == [448.0, small] and list(out) == [448.0, small]
    # 2) x = [small, 256]: row scale 1, quantized directly: xq = [1.125, 256]
    #    (rounded to bf16 first, small would be the tie 1.0625 and go to the
    #    even code 1.0). g = 0.25 * x_1 = 64 for both units; u_0 = x_0 / 64,
    #    u_1 = 7/256 * x_1 = 7, so h = [xq_0, 448] = [1.125, 448].
    L2 = oracle.Layer(wr, None, np.array([[[0.0, 0.25], [0.0, 0.25]]], f32),
                      np.array([[[1.0 / 64.0, 0.0], [0.0, 7.0 / 256.0]]], f32), wd, 1)
    x2 = np.array([small, 256.0], f32)
    assert float(x2[0]) == small
    out2, h2 = L2.expert_ffn(0, x2, want_h=True, act_fp8=True)
    assert list(h2) == [1.125, 448.0] and list(out2) == [1.125, 448.0]
    _, h2raw = L2.expert_ffn(0, x2, want_h=True)
    assert list(h2raw) == [small, 448.0]
    # 3) the row scale comes from the whole row: x = [1.25 * 2^-9, 512] has
    #    scale 2 (512 > 448), so x_0 / 2 = 0.625 subnormal steps of 2^-9
    #    rounds to one step: xq_0 = 2^-9 * 2 = 2^-8 (at scale 1 it would be
    #    1.25 steps -> 2^-9). g = x_1 / 8 = 64, u_0 = x_0 / 64, u_1 = 7/512 *
    #    x_1 = 7, so h = [xq_0, 448].
    x3 = np.array([1.25 * 2.0 ** -9, 512.0], f32)
    L3 = oracle.Layer(wr, None, np.array([[[0.0, 0.125], [0.0, 0.125]]], f32),
                      np.array([[[1.0 / 64.0, 0.0], [0.0, 7.0 / 512.0]]], f32), wd, 1)
    out3, h3 = L3.expert_ffn(0, x3, want_h=True, act_fp8=True)
    assert list(h3) == [2.0 ** -8, 448.0] and list(out3) == [2.0 ** -8, 448.0], list(h3)
