"""Pins of the oracle helpers that decide how routing is compared: the near-tie
tests (which tokens' expert order or set may legitimately differ between two
correct fp32 computations of the logits) and the routing weights of given
experts (used to check the GPU's weights on every token, whichever experts it
picked).

The comparison rule for expert ids: a token's sorted fp32 logits l_(0) >= l_(1)
>= ... are near-tied at position i when l_(i) - l_(i+1) < 1e-5 * max(|l_(i)|,
|l_(i+1)|). near_tie_tokens flags a near tie anywhere among the first k+1
(slot order inside the top k, or the k-th / (k+1)-th boundary);
boundary_tie_tokens flags only the boundary pair. Each case below is built so
that a plausible slip (an ascending sort, a flipped comparison, a missing abs,
an absolute instead of a relative gap, an off-by-one in the k+1 window) changes
the answer.
"""
import math

import numpy as np
import pytest

import oracle

REL = 1e-5


def f32(rows):
    return np.array(rows, dtype=np.float32)


def flags(rows, k):
    lg = f32(rows)
    return oracle.near_tie_tokens(lg, k).tolist(), oracle.boundary_tie_tokens(lg, k).tolist()


def test_exact_tie_inside_top_k():
    # experts 0 and 1 tie for slot 0/1; the boundary pair (3, 1) is far apart
    assert flags([[3.0, 3.0, 1.0, 0.0]], 2) == ([True], [False])


def test_exact_tie_at_the_boundary():
    assert flags([[3.0, 1.0, 1.0, 0.0]], 2) == ([True], [True])


def test_tie_below_the_window_is_ignored():
    # the tie is between the (k+1)-th and (k+2)-th logits: outside the window
    assert flags([[3.0, 2.0, 1.0, 1.0]], 2) == ([False], [False])


def test_unsorted_input_is_sorted_descending():
    # ascending storage order; the top 2 are the two 3.0s (a tie inside the
    # top k). An ascending sort would look at (0, 1, 3) and see no tie.
    assert flags([[0.0, 1.0, 3.0, 3.0]], 2) == ([True], [False])
    # the boundary pair sits at the front of the storage order
    assert flags([[1.0, 1.0, 0.0, 5.0]], 2) == ([True], [True])


@pytest.mark.parametrize("gap, tied", [(9.0e-6, True), (1.1e-5, False)])
def test_relative_gap_just_inside_and_outside(gap, tied):
    # l_(0) = 1, l_(1) = 1 - gap (fp32 spacing near 1 is 6e-8)
    b = float(np.float32(1.0 - gap))
    assert flags([[1.0, b, -2.0]], 1) == ([tied], [tied])


def test_gap_is_relative_to_the_magnitude():
    # 0.005 apart at magnitude 1000 is inside 1e-5 relative (0.01); 0.02 is not;
    # an absolute 1e-5 test would call both far apart
    assert flags([[1000.0, float(np.float32(999.995)), 0.0]], 1) == ([True], [True])
    assert flags([[1000.0, float(np.float32(999.98)), 0.0]], 1) == ([False], [False])


def test_negative_logits_use_magnitudes():
    # -1 and -1.000005: gap 5e-6 < 1e-5 * 1.000005. Without the abs the bound
    # would be negative and the tie missed.
    b = float(np.float32(-1.000005))
    assert flags([[-3.0, -1.0, b]], 1) == ([True], [True])
    assert flags([[-3.0, -1.0, -1.5]], 1) == ([False], [False])


def test_well_separated_tokens_are_not_flagged():
    # a flipped comparison would flag every one of these
    rows = [[5.0, 3.0, 1.0, -1.0], [0.5, -0.5, 2.5, 1.5], [-1.0, -2.0, -3.0, -4.0]]
    for k in (1, 2, 3):
        n, b = flags(rows, k)
        assert n == [False, False, False] and b == [False, False, False], k


def test_k_equals_E():
    # every expert is selected: the set cannot differ, only the slot order
    assert flags([[2.0, 2.0]], 2) == ([True], [False])
    assert flags([[2.0, 1.0]], 2) == ([False], [False])
    assert flags([[7.0]], 1) == ([False], [False])


def test_window_is_k_plus_one():
    # k = 3: a tie between the 3rd and 4th largest is the boundary; between the
    # 4th and 5th it is outside
    assert flags([[9.0, 8.0, 7.0, 7.0, 1.0]], 3) == ([True], [True])
    assert flags([[9.0, 8.0, 7.0, 1.0, 1.0]], 3) == ([False], [False])
    assert flags([[9.0, 9.0, 7.0, 1.0, 1.0]], 3) == ([True], [False])


def _loop_flags(row, k):
    """Pure-Python restatement by explicit loops over a sorted copy."""
    s = sorted((float(v) for v in row), reverse=True)
    near = False
    for i in range(min(k + 1, len(s)) - 1):
        a, b = s[i], s[i + 1]
        if a - b < REL * max(abs(a), abs(b)):
            near = True
    bnd = False
    if k < len(s):
        a, b = s[k - 1], s[k]
        bnd = a - b < REL * max(abs(a), abs(b))
    return near, bnd


def test_random_rows_with_planted_near_ties():
    rng = np.random.default_rng(5)
    T, E = 400, 12
    lg = rng.standard_normal((T, E)).astype(np.float32) * np.float32(3.0)
    # plant ties and near ties between a random pair of experts of each token
    for t in range(T):
        a, b = rng.choice(E, size=2, replace=False)
        lg[t, b] = np.float32(lg[t, a] * (1.0 - rng.choice([0.0, 3e-6, 2e-5, 1e-3])))
    for k in (1, 2, 4, 11, 12):
        near = oracle.near_tie_tokens(lg, k)
        bnd = oracle.boundary_tie_tokens(lg, k)
        want = [_loop_flags(lg[t], k) for t in range(T)]
        assert near.tolist() == [w[0] for w in want], k
        assert bnd.tolist() == [w[1] for w in want], k
        assert not np.any(bnd & ~near)  # the boundary is part of the window
        assert 0 < near.sum() < T


# --- routing weights of given experts ----------------------------------------

def test_route_weights_equal_topk_weights_on_its_own_ids():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((300, 16)).astype(np.float32)
    for k in (1, 2, 4, 16):
        ids, w, wd = oracle.topk(lg, k)
        w2, wd2 = oracle.route_weights(lg, ids)
        assert np.array_equal(w, w2) and np.array_equal(wd, wd2), k


def test_route_weights_closed_forms():
    lg = f32([[0.5, 2.0, -1.0], [math.log(3.0), 0.0, 9.0]])
    w, wd = oracle.route_weights(lg, np.array([[1, 0], [0, 1]], np.int32))
    # k = 2: w_0 = sigmoid(l_0 - l_1)
    assert abs(wd[0, 0] - 1.0 / (1.0 + math.exp(-(2.0 - 0.5)))) < 1e-15
    assert abs(wd[1, 0] - 0.75) < 1e-7 and abs(wd[1, 1] - 0.25) < 1e-7
    # k = 1: weight 1 whatever the logit
    w1, _ = oracle.route_weights(lg, np.array([[2], [2]], np.int32))
    assert w1.tolist() == [[1.0], [1.0]]
    # sums to 1 and does not depend on which expert takes slot 0 (beyond rounding)
    ids = np.array([[2, 0, 1], [1, 2, 0]], np.int32)
    _, a = oracle.route_weights(lg, ids)
    _, b = oracle.route_weights(lg, ids[:, ::-1].copy())
    assert np.allclose(a.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.allclose(a, b[:, ::-1], rtol=1e-14, atol=0)
    # the full softmax over the three logits of token 0
    e = np.exp(lg[0].astype(np.float64) - lg[0].max())
    assert np.allclose(a[0], (e / e.sum())[[2, 0, 1]], rtol=1e-14, atol=0)


def test_route_weights_reject_ids_out_of_range():
    lg = f32([[0.0, 1.0]])
    with pytest.raises(ValueError):
        oracle.route_weights(lg, np.array([[2]], np.int32))
    with pytest.raises(ValueError):
        oracle.route_weights(lg, np.array([[-1]], np.int32))
