"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes one part of the definition with something independent: exact
bit patterns, closed forms, a hand-computed example (tests/golden), brute force
over all experts or all k-subsets, invariants, and special cases that reduce to
a textbook formula. Together they are chosen so that a dropped term, a swapped
gate/up, a transposed matrix, a wrong sign or a wrong tie rule fails at least
one test. No GPU is used.
"""
import ctypes
import itertools
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def silu(z):
    return z / (1.0 + np.exp(-z))


def f32layer(w_r, w_g, w_u, w_d, k, b=None):
    return oracle.Layer(np.asarray(w_r, np.float32), None if b is None else np.asarray(b, np.float32),
                        np.asarray(w_g, np.float32), np.asarray(w_u, np.float32),
                        np.asarray(w_d, np.float32), k)


def rand_layer(rng, d, f, E, k, bias=False, dtype="f32"):
    """Random layer; bf16 weights are rounded through the generator's RNE."""
    w_r = rng.standard_normal((d, E)) / math.sqrt(d)
    w_g = rng.standard_normal((E, f, d)) / math.sqrt(d)
    w_u = rng.standard_normal((E, f, d)) / math.sqrt(d)
    w_d = rng.standard_normal((E, d, f)) / math.sqrt(f)
    b = rng.standard_normal(E).astype(np.float32) if bias else None
    ws = [w_r, w_g, w_u, w_d]
    if dtype == "bf16":
        ws = [to_bf16(w) for w in ws]
    else:
        ws = [np.asarray(w, np.float32) for w in ws]
    return oracle.Layer(ws[0], b, ws[1], ws[2], ws[3], k)


def to_bf16(a):
    f = synth.lib().synth_f32_to_bf16
    flat = np.asarray(a, np.float32).ravel()
    return np.array([f(float(v)) for v in flat], dtype=np.uint16).reshape(np.shape(a))


def as_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return synth.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


# ---------------------------------------------------------------- widening --

def test_widen_bf16_exact_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x3EAB, 0x0001, 0x7F7F, 0x8000, 0x0000], np.uint16)
    want = np.array([1.0, -2.0, 3.140625, 0.333984375, 2.0 ** -133,
                     (2.0 - 2.0 ** -7) * 2.0 ** 127, -0.0, 0.0])
    got = oracle.widen(bits).astype(np.float64)
    assert np.array_equal(got, want)
    assert math.copysign(1.0, got[6]) == -1.0


# ----------------------------------------------------------------- router --

def test_router_identity_gives_x_exactly():
    rng = np.random.default_rng(1)
    E = 8
    x = rng.standard_normal((5, E)).astype(np.float32)
    L = f32layer(np.eye(E), np.zeros((E, 1, E)), np.zeros((E, 1, E)), np.zeros((E, E, 1)), 2)
    assert np.array_equal(L.router(x), x)


def test_router_non_square_orientation():
    # W_r is [d][E]: logits[e] = sum_i x[i] W_r[i][e]. A transposed read gives
    # different numbers (and a 3x2 matrix cannot be read as 2x3 by accident).
    w_r = np.array([[1, 0], [0, 10], [100, 0]], np.float32)
    x = np.array([[1, 2, 3]], np.float32)
    L = f32layer(w_r, np.zeros((2, 1, 3)), np.zeros((2, 1, 3)), np.zeros((2, 3, 1)), 1)
    assert L.router(x).tolist() == [[301.0, 20.0]]


def test_router_bias_is_added():
    b = np.array([0.5, -2.0, 7.25], np.float32)
    L = f32layer(np.zeros((4, 3)), np.zeros((3, 1, 4)), np.zeros((3, 1, 4)), np.zeros((3, 4, 1)), 1, b)
    x = np.ones((2, 4), np.float32)
    assert np.array_equal(L.router(x), np.tile(b, (2, 1)))


def test_router_double_sum_rounded_once():
    # 1 + 2^-24 + 2^-24: fp32 running sums round to 1 twice; the double sum
    # is 1 + 2^-23, which fp32 holds exactly.
    x = np.array([[1.0, 2.0 ** -24, 2.0 ** -24]], np.float32)
    L = f32layer(np.ones((3, 1)), np.zeros((1, 1, 3)), np.zeros((1, 1, 3)), np.zeros((1, 3, 1)), 1)
    assert L.router(x)[0, 0] == np.float32(1.0 + 2.0 ** -23)


def test_router_bf16_matches_widened_f32():
    rng = np.random.default_rng(2)
    Lb = rand_layer(rng, 16, 4, 6, 2, dtype="bf16", bias=True)
    xb = to_bf16(rng.standard_normal((7, 16)))
    Lf = oracle.Layer(as_f64(Lb.w_router).astype(np.float32), Lb.b_router,
                      as_f64(Lb.w_gate).astype(np.float32), as_f64(Lb.w_up).astype(np.float32),
                      as_f64(Lb.w_down).astype(np.float32), 2)
    assert np.array_equal(Lb.router(xb), Lf.router(as_f64(xb).astype(np.float32)))


# ------------------------------------------------------------------ top-k --

@pytest.mark.parametrize("E", [2, 3, 5, 8])
def test_topk_equals_max_sum_subset(E):
    rng = np.random.default_rng(10 + E)
    lg = rng.standard_normal((40, E)).astype(np.float32)
    for k in range(1, E + 1):
        ids, w, _ = oracle.topk(lg, k)
        for t in range(lg.shape[0]):
            best = max(itertools.combinations(range(E), k),
                       key=lambda s: sum(float(lg[t, e]) for e in s))
            assert set(ids[t].tolist()) == set(best)
            vals = lg[t, ids[t]]
            assert np.all(vals[:-1] > vals[1:])  # slots in descending order


def test_topk_exact_ties_prefer_lower_index():
    lg = np.array([[1, 3, 3, 0, 3],
                   [2, 2, 2, 2, 2],
                   [0, 5, 1, 5, -1]], np.float32)
    ids2, w2, _ = oracle.topk(lg, 2)
    assert ids2.tolist() == [[1, 2], [0, 1], [1, 3]]
    ids3, _, _ = oracle.topk(lg, 3)
    assert ids3.tolist() == [[1, 2, 4], [0, 1, 2], [1, 3, 2]]
    assert np.all(w2[:2] == np.float32(0.5))


def test_topk_single_expert_and_k_equals_E():
    lg = np.array([[0.3], [-7.0]], np.float32)
    ids, w, _ = oracle.topk(lg, 1)
    assert ids.ravel().tolist() == [0, 0] and np.all(w == 1.0)
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((6, 4)).astype(np.float32)
    ids, _, _ = oracle.topk(lg, 4)
    for t in range(6):
        assert sorted(ids[t].tolist()) == [0, 1, 2, 3]


# ---------------------------------------------------------------- weights --

def test_weights_k1_is_one_and_k2_is_sigmoid_of_gap():
    rng = np.random.default_rng(4)
    lg = (3 * rng.standard_normal((50, 8))).astype(np.float32)
    _, w1, _ = oracle.topk(lg, 1)
    assert np.all(w1 == 1.0)
    ids, w2, wd = oracle.topk(lg, 2)
    l0 = lg[np.arange(50), ids[:, 0]].astype(np.float64)
    l1 = lg[np.arange(50), ids[:, 1]].astype(np.float64)
    sig = 1.0 / (1.0 + np.exp(l1 - l0))
    assert np.allclose(wd[:, 0], sig, rtol=0, atol=1e-15)
    assert np.allclose(wd[:, 1], 1 - sig, rtol=0, atol=1e-15)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 8])
def test_weights_equal_full_softmax_then_renormalise(k):
    rng = np.random.default_rng(5 + k)
    E = 8
    lg = (2 * rng.standard_normal((30, E))).astype(np.float32)
    ids, w, wd = oracle.topk(lg, k)
    p = np.exp(lg.astype(np.float64) - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    ref = sel / sel.sum(axis=1, keepdims=True)
    assert np.allclose(wd, ref, rtol=1e-13, atol=0)
    assert np.allclose(wd.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.array_equal(w, wd.astype(np.float32))
    assert np.all(np.diff(wd, axis=1) <= 0)  # weights follow the slot order


# --------------------------------------------------------------- dispatch --

@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 4, 2), (64, 8, 2), (33, 16, 4), (100, 5, 5)])
def test_dispatch_invariants_and_brute_force(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    r = oracle.dispatch(ids, E)
    c, off, perm, ps, inv = r["counts"], r["offsets"], r["perm"], r["perm_slot"], r["inv"]
    assert c.sum() == T * k
    assert off[0] == 0 and np.all(np.diff(off) == c) and off[-1] == T * k
    for e in range(E):
        seg = perm[off[e]:off[e + 1]].tolist()
        brute = [t for t in range(T) if e in ids[t].tolist()]
        assert seg == brute  # stable: ascending token order
        for p in range(off[e], off[e + 1]):
            assert ids[perm[p], ps[p]] == e
    # every token appears exactly k times, once per slot, and inv inverts perm
    assert np.array_equal(np.bincount(perm, minlength=T), np.full(T, k))
    for t in range(T):
        for j in range(k):
            p = inv[t * k + j]
            assert perm[p] == t and ps[p] == j
    assert sorted(inv.tolist()) == list(range(T * k))


def test_dispatch_empty_experts_and_zero_tokens():
    ids = np.array([[2, 0], [2, 0], [0, 2]], np.int32)
    r = oracle.dispatch(ids, 5)
    assert r["counts"].tolist() == [3, 0, 3, 0, 0]
    assert r["offsets"].tolist() == [0, 3, 3, 6, 6, 6]
    assert r["perm"].tolist() == [0, 1, 2, 0, 1, 2]
    assert r["perm_slot"].tolist() == [1, 1, 0, 0, 0, 1]
    r0 = oracle.dispatch(np.zeros((0, 2), np.int32), 3)
    assert r0["counts"].tolist() == [0, 0, 0] and r0["offsets"].tolist() == [0, 0, 0, 0]


def test_dispatch_rejects_out_of_range_id():
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([[0, 3]], np.int32), 3)


# ------------------------------------------------------------ FFN/combine --

def _hand_layer(k):
    return f32layer(np.eye(2),
                    np.array([[[1, 0]], [[1, 0]]]),
                    np.array([[[1, 0]], [[2, 0]]]),
                    np.array([[[1], [0]], [[0], [1]]]), k)


def test_hand_two_expert_example_golden():
    L3 = math.log(3.0)
    S = 1.0 / (1.0 + math.exp(-1.0))
    xs = {"lnx": np.array([[math.log(3.0), 0.0]], np.float32),
          "tie": np.array([[1.0, 1.0]], np.float32)}
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "two_expert_hand_example.txt"))
            if ln.startswith("case ")]
    assert len(rows) == 4
    for _, name, kk, idss, y0, y1 in rows:
        k = int(kk.split("=")[1])
        x = xs[name]
        env = {"L": L3, "S": S}
        # x holds fp32(ln 3), off exact ln 3 by < 3e-8 relative; the closed
        # forms use exact ln 3, so that case is compared to 1e-6.
        tol = 1e-6 if name == "lnx" else 1e-15
        want = np.array([eval(y0.split("=")[1], {}, env), eval(y1.split("=")[1], {}, env)])
        L = _hand_layer(k)
        ids, _, _ = oracle.topk(L.router(x), k)
        assert ids[0].tolist() == [int(v) for v in idss.split("=")[1].split(",")]
        y = L.forward(x)[0]
        assert np.allclose(y, want, rtol=tol, atol=1e-15), (name, k, y, want)


def _dense_swiglu(x, wg, wu, wd):
    """Textbook SwiGLU FFN in float64 with numpy's matmul: Wd (silu(Wg x) * (Wu x))."""
    return wd @ (silu(wg @ x) * (wu @ x))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_masked_brute_force_over_all_experts(dtype):
    rng = np.random.default_rng(21)
    d, f, E, k, T = 12, 10, 6, 2, 9
    L = rand_layer(rng, d, f, E, k, bias=True, dtype=dtype)
    x = rng.standard_normal((T, d)).astype(np.float32)
    x = to_bf16(x) if dtype == "bf16" else x
    y = L.forward(x)
    xs, wr, wg, wu, wdn = (as_f64(a) for a in (x, L.w_router, L.w_gate, L.w_up, L.w_down))
    lg = (xs @ wr + L.b_router.astype(np.float64)).astype(np.float32)
    ids, _, wts = oracle.topk(lg, k)
    for t in range(T):
        acc = np.zeros(d)
        for e in range(E):  # every expert, masked: no dispatch involved
            m = e in ids[t].tolist()
            wt = wts[t, ids[t].tolist().index(e)] if m else 0.0
            acc += (1.0 if m else 0.0) * wt * _dense_swiglu(xs[t], wg[e], wu[e], wdn[e])
        assert np.allclose(y[t], acc, rtol=1e-12, atol=1e-14)


def test_dense_equivalence_when_k_equals_E():
    rng = np.random.default_rng(22)
    d, f, E, T = 8, 6, 5, 7
    L = rand_layer(rng, d, f, E, E, bias=True)
    x = rng.standard_normal((T, d)).astype(np.float32)
    y = L.forward(x)
    xs = x.astype(np.float64)
    lg = L.router(x).astype(np.float64)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    for t in range(T):
        ref = sum(p[t, e] * _dense_swiglu(xs[t], as_f64(L.w_gate[e]), as_f64(L.w_up[e]), as_f64(L.w_down[e]))
                  for e in range(E))
        assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-14)


def test_single_expert_reduces_to_textbook_swiglu():
    rng = np.random.default_rng(23)
    d, f, T = 16, 24, 5
    L = rand_layer(rng, d, f, 1, 1)
    x = rng.standard_normal((T, d)).astype(np.float32)
    y = L.forward(x)
    for t in range(T):
        ref = _dense_swiglu(x[t].astype(np.float64), as_f64(L.w_gate[0]), as_f64(L.w_up[0]), as_f64(L.w_down[0]))
        assert np.allclose(y[t], ref, rtol=1e-13, atol=1e-15)
    out, h = L.expert_ffn(0, x[0], want_h=True)
    g = as_f64(L.w_gate[0]) @ x[0].astype(np.float64)
    u = as_f64(L.w_up[0]) @ x[0].astype(np.float64)
    assert np.allclose(h, silu(g) * u, rtol=1e-13, atol=1e-15)


def test_gate_and_up_are_not_interchangeable():
    # SiLU is applied to the gate projection only: swapping the two matrices
    # changes the result, and the oracle must follow the gate one.
    w_r = np.ones((1, 1), np.float32)
    L = f32layer(w_r, [[[2.0]]], [[[3.0]]], [[[1.0]]], 1)
    y = L.forward(np.array([[1.0]], np.float32))[0, 0]
    assert math.isclose(y, 2.0 / (1 + math.exp(-2.0)) * 3.0, rel_tol=1e-15)
    assert not math.isclose(y, 3.0 / (1 + math.exp(-3.0)) * 2.0, rel_tol=1e-6)


def test_down_projection_orientation():
    # d=2, f=3: W_d is [d][f]; out_o = sum_i h_i W_d[o][i].
    wg = np.array([[[1, 0], [0, 1], [1, 1]]], np.float32)
    wu = np.ones((1, 3, 2), np.float32)
    wd = np.array([[[1, 10, 100], [1000, 0, 0]]], np.float32)
    L = f32layer(np.ones((2, 1)), wg, wu, wd, 1)
    x = np.array([[1.0, 2.0]], np.float32)
    g = np.array([1.0, 2.0, 3.0])
    h = silu(g) * 3.0
    want = np.array([h[0] + 10 * h[1] + 100 * h[2], 1000 * h[0]])
    assert np.allclose(L.forward(x)[0], want, rtol=1e-15)


def test_linearity_in_down_weights_and_expert_relabelling():
    rng = np.random.default_rng(24)
    d, f, E, k, T = 10, 8, 6, 3, 11
    L = rand_layer(rng, d, f, E, k, bias=True)
    x = rng.standard_normal((T, d)).astype(np.float32)
    y = L.forward(x)
    L2 = oracle.Layer(L.w_router, L.b_router, L.w_gate, L.w_up, 2 * L.w_down, k)
    assert np.array_equal(L2.forward(x), 2 * y)  # exact: scaling by 2 is exact
    pi = rng.permutation(E)  # new expert n is old expert pi[n]
    Lp = oracle.Layer(np.ascontiguousarray(L.w_router[:, pi]), L.b_router[pi],
                      L.w_gate[pi], L.w_up[pi], L.w_down[pi], k)
    assert np.array_equal(Lp.forward(x), y)
    ids, _, _ = oracle.topk(L.router(x), k)
    idp, _, _ = oracle.topk(Lp.router(x), k)
    assert np.array_equal(pi[idp], ids)


def test_forced_routing_mode():
    rng = np.random.default_rng(25)
    d, f, E, k, T = 8, 6, 5, 2, 6
    L = rand_layer(rng, d, f, E, k)
    x = rng.standard_normal((T, d)).astype(np.float32)
    lg = L.router(x)
    ids, _, _ = oracle.topk(lg, k)
    assert np.array_equal(L.forward(x, forced_ids=ids), L.forward(x))
    forced = np.array([[(t + 1) % E, (t + 3) % E] for t in range(T)], np.int32)
    y = L.forward(x, forced_ids=forced)
    for t in range(T):
        l = lg[t, forced[t]].astype(np.float64)
        w = np.exp(l - l[0]) / np.exp(l - l[0]).sum()
        ref = sum(w[j] * L.expert_ffn(forced[t, j], x[t]) for j in range(k))
        assert np.allclose(y[t], ref, rtol=1e-14, atol=1e-16)


def test_token_subset_matches_full_run():
    rng = np.random.default_rng(26)
    L = rand_layer(rng, 8, 4, 4, 2)
    x = rng.standard_normal((10, 8)).astype(np.float32)
    y = L.forward(x)
    sub = np.array([9, 0, 4], np.int32)
    assert np.array_equal(L.forward(x, tokens=sub), y[sub])


def test_silu_of_very_negative_gate_is_zero_not_nan():
    L = f32layer(np.ones((1, 1)), [[[-1000.0]]], [[[1.0]]], [[[1.0]]], 1)
    y = L.forward(np.array([[1.0]], np.float32))
    assert y[0, 0] == 0.0 and not np.isnan(y[0, 0])


def test_result_independent_of_thread_count():
    gomp = ctypes.CDLL("libgomp.so.1")
    rng = np.random.default_rng(27)
    L = rand_layer(rng, 32, 16, 8, 2, bias=True)
    x = rng.standard_normal((40, 32)).astype(np.float32)
    outs = []
    for n in (1, 3, 8):
        gomp.omp_set_num_threads(n)
        outs.append((L.forward(x), L.router(x)))
    gomp.omp_set_num_threads(os.cpu_count() or 1)
    for y, lg in outs[1:]:
        assert np.array_equal(y, outs[0][0]) and np.array_equal(lg, outs[0][1])


def test_invalid_arguments_are_rejected():
    rng = np.random.default_rng(28)
    L = rand_layer(rng, 4, 2, 3, 2)
    with pytest.raises(TypeError):
        L.forward(np.zeros((2, 5), np.float32))
    with pytest.raises(ValueError):
        L.forward(np.zeros((2, 4), np.float32), forced_ids=np.array([[0, 3], [0, 1]], np.int32))
    with pytest.raises(ValueError):
        oracle.topk(np.zeros((2, 3), np.float32), 4)
