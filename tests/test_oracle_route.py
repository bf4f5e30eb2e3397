"""Pins for the oracle's router: fp32 logits, top-k selection, weights.

The logit is defined as one fp32 fused-multiply-add chain over h ascending;
the tests pin the operand orientation (x [T][H] times Wr [H][E]), the order
of the chain, the fusing, the -0 canonicalisation, the selection order with
ties, and the two scoring rules through closed forms."""
import math

import numpy as np
import pytest
import scipy.special

from oracle import moe


def test_logits_exact_on_integer_inputs_non_square():
    rng = np.random.default_rng(0)
    x = rng.integers(-8, 9, (5, 7)).astype(np.float32)
    wr = rng.integers(-8, 9, (7, 3)).astype(np.float32)
    b = np.array([0.5, -1.0, 2.0], dtype=np.float32)
    l = moe.router_logits(x, wr, b)
    exact = x.astype(np.int64) @ wr.astype(np.int64) + b
    np.testing.assert_array_equal(l, exact.astype(np.float32))


def test_logits_within_fp32_chain_error_bound():
    rng = np.random.default_rng(1)
    T, H, E = 9, 7168, 16
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((H, E)) / math.sqrt(H)).astype(np.float32)
    l = moe.router_logits(x, wr, None).astype(np.float64)
    ref = x.astype(np.float64) @ wr.astype(np.float64)
    bound = H * 2.0 ** -24 * (np.abs(x.astype(np.float64)) @ np.abs(wr.astype(np.float64)))
    assert (np.abs(l - ref) <= bound).all()


def test_logits_chain_is_sequential_ascending():
    # 2^24 + 1 rounds back to 2^24 (tie to even), then -2^24 cancels: a
    # sequential ascending fp32 chain gives exactly 0; any other order gives 1.
    x = np.ones((1, 3), dtype=np.float32)
    wr = np.array([[2.0 ** 24], [1.0], [-(2.0 ** 24)]], dtype=np.float32)
    assert moe.router_logits(x, wr, None)[0, 0] == 0.0
    # reversed rows: -2^24 + 1 is exact, + 2^24 gives 1
    assert moe.router_logits(x, wr[::-1].copy(), None)[0, 0] == 1.0


def test_logits_use_fused_multiply_add():
    # acc = -(1 + 2^-11); fma((1+2^-12), (1+2^-12), acc) = 2^-24 exactly,
    # whereas a rounded product would give 0.
    a = 1.0 + 2.0 ** -12
    x = np.array([[1.0, a]], dtype=np.float32)
    wr = np.array([[-(1.0 + 2.0 ** -11)], [a]], dtype=np.float32)
    assert moe.router_logits(x, wr, None)[0, 0] == np.float32(2.0 ** -24)


def test_logits_negative_zero_canonicalised():
    x = np.array([[1.0]], dtype=np.float32)
    wr = np.array([[-0.0, 0.0]], dtype=np.float32)
    l = moe.router_logits(x, wr, None)
    assert not np.signbit(l).any()


def _brute_topk_valid(l, ids, k):
    T, E = l.shape
    for t in range(T):
        sel = list(ids[t])
        assert len(set(sel)) == k
        key = lambda e: (l[t, e], -e)
        for a, b in zip(sel, sel[1:]):
            assert key(a) > key(b)
        worst = min(key(e) for e in sel)
        for e in range(E):
            if e not in sel:
                assert key(e) < worst


def test_topk_brute_force_with_many_ties():
    rng = np.random.default_rng(2)
    l = rng.integers(-3, 4, (200, 32)).astype(np.float32)   # heavy exact ties
    ids = moe.select_topk(l, 8)
    _brute_topk_valid(l, ids, 8)


def test_topk_all_equal_picks_lowest_indices_in_order():
    l = np.zeros((3, 256), dtype=np.float32)
    np.testing.assert_array_equal(moe.select_topk(l, 8), np.tile(np.arange(8), (3, 1)))


def test_weights_closed_forms():
    # logits (0, ln 3): sigmoid gives 1/2 and 3/4 -> renormalised 0.4, 0.6;
    # softmax gives 1/4 and 3/4.  The selection order is by logit, so the
    # expert with ln 3 comes first.
    x = np.array([[1.0]], dtype=np.float32)
    wr = np.array([[0.0, math.log(3.0)]], dtype=np.float32)
    l3 = float(np.float32(math.log(3.0)))
    ids, w, _ = moe.route(x, wr, None, 2, "sigmoid")
    np.testing.assert_array_equal(ids, [[1, 0]])
    s1, s0 = 1 / (1 + math.exp(-l3)), 0.5
    np.testing.assert_allclose(w[0], [s1 / (s1 + s0), s0 / (s1 + s0)], rtol=1e-7)
    assert abs(w[0, 0] - 0.6) < 1e-6
    ids, w, _ = moe.route(x, wr, None, 2, "softmax")
    assert abs(w[0, 0] - 0.75) < 1e-6 and abs(w[0, 1] - 0.25) < 1e-6


def test_bias_moves_selection_and_weights():
    x = np.array([[1.0]], dtype=np.float32)
    wr = np.array([[0.0, 1.0, 0.5]], dtype=np.float32)
    b = np.array([2.0, 0.0, 0.0], dtype=np.float32)       # expert 0 logit becomes 2
    ids, w, l = moe.route(x, wr, b, 1, "sigmoid")
    assert ids[0, 0] == 0 and w[0, 0] == 1.0
    ids, w, l = moe.route(x, wr, b, 2, "softmax")
    np.testing.assert_array_equal(ids, [[0, 1]])
    np.testing.assert_allclose(w[0], [1 / (1 + math.exp(-1)), math.exp(-1) / (1 + math.exp(-1))], rtol=1e-6)


def test_softmax_with_k_equal_E_is_full_softmax():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((11, 64)).astype(np.float32)
    wr = (rng.standard_normal((64, 8)) / 8).astype(np.float32)
    ids, w, l = moe.route(x, wr, None, 8, "softmax")
    full = scipy.special.softmax(l.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids, axis=1), rtol=1e-6)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_weights_sum_to_one_and_k1_is_one(score):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((300, 128)).astype(np.float32)
    wr = (rng.standard_normal((128, 256)) / math.sqrt(128)).astype(np.float32)
    ids, w, _ = moe.route(x, wr, None, 8, score)
    assert np.abs(w.astype(np.float64).sum(axis=1) - 1).max() <= 1e-6
    assert (w > 0).all()
    ids, w, _ = moe.route(x, wr, None, 1, score)
    assert (w == 1.0).all()
