"""Pins of the oracle's router variants (selection-only bias, hash-routed
rows, sqrt-softplus scores) against closed forms, hand-worked cases and the
plain routing they reduce to."""
import math

import numpy as np
import scipy.special

from oracle import moe


def _logit_layer(Lrow):
    """x, Wr whose logits are exactly Lrow (one token): x = e_0, Wr[:, 0] = L."""
    E = len(Lrow)
    x = np.zeros((1, 8))
    x[0, 0] = 1.0
    wr = np.zeros((E, 8))
    wr[:, 0] = Lrow
    return x, wr


def test_softplus_closed_forms():
    L = np.array([0.0, math.log(math.e - 1.0), -40.0, 40.0, 1000.0, -1000.0, 2.5])
    sp = moe.softplus(L)
    assert abs(sp[0] - math.log(2.0)) < 1e-15
    assert abs(sp[1] - 1.0) < 1e-15
    assert abs(sp[2] / math.exp(-40.0) - 1.0) < 1e-12  # log(1 + e^-40) = e^-40 (1 - e^-40 / 2 ...)
    assert abs(sp[3] - 40.0) < 1e-15 and sp[4] == 1000.0 and sp[5] == 0.0
    assert abs(sp[6] - math.log1p(math.exp(2.5))) < 1e-15


def test_plain_variant_reduces_to_route():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 64))
    wr = rng.standard_normal((40, 64)) * 0.3
    ids, w, _ = moe.route(x, wr, 6)
    ids2, w2, _, _ = moe.route_variant(x, wr, 6)
    assert np.array_equal(ids, ids2)
    assert np.allclose(w, w2, rtol=1e-14, atol=0)


def test_selection_bias_forces_experts_and_keeps_unbiased_weights():
    rng = np.random.default_rng(6)
    E, k = 32, 4
    L = rng.standard_normal(E)
    x, wr = _logit_layer(L)
    forced = np.array([30, 3, 17, 9])
    b = np.zeros(E)
    b[forced] = 2.0  # any probability plus 2 beats every unbiased probability
    ids, w, _, sel = moe.route_variant(x, wr, k, select_bias=b)
    p = scipy.special.softmax(L)
    want = forced[np.argsort(-(p[forced] + 2.0), kind="stable")]
    assert np.array_equal(ids[0], want)
    assert np.allclose(w[0], scipy.special.softmax(L[want]), rtol=1e-13)  # renormalised unbiased softmax
    assert np.allclose(sel[0], p + b, rtol=1e-14)


def test_selection_bias_tie_goes_to_lower_index():
    E, k = 10, 3
    x, wr = _logit_layer(np.zeros(E))  # uniform probabilities 1/E
    b = np.zeros(E)
    b[[7, 2, 5]] = 0.5
    ids, w, _, _ = moe.route_variant(x, wr, k, select_bias=b)
    assert ids[0].tolist() == [2, 5, 7]
    assert np.allclose(w[0], 1.0 / 3.0, rtol=1e-15)


def test_hash_rows_replace_selection():
    rng = np.random.default_rng(7)
    E, k, T = 24, 3, 4
    x = rng.standard_normal((T, 16))
    wr = rng.standard_normal((E, 16))
    table = np.array([[5, 0, 23], [1, 2, 3], [23, 22, 21], [7, 11, 13]])
    for score in (moe.SCORE_SOFTMAX, moe.SCORE_SQRT_SOFTPLUS):
        ids, w, L, _ = moe.route_variant(x, wr, k, score=score, hash_ids=table)
        assert np.array_equal(ids, table)
        for t in range(T):
            if score == moe.SCORE_SOFTMAX:
                want = scipy.special.softmax(L[t, table[t]])
            else:
                s = np.sqrt(np.log1p(np.exp(L[t, table[t]])))
                want = s / s.sum()
            assert np.allclose(w[t], want, rtol=1e-13)


def test_sqrt_softplus_hand_example():
    L = np.array([0.0, math.log(math.e - 1.0), 3.0, -2.0])
    x, wr = _logit_layer(L)
    ids, w, _, _ = moe.route_variant(x, wr, 2, score=moe.SCORE_SQRT_SOFTPLUS)
    s2 = math.sqrt(3.0 + math.log1p(math.exp(-3.0)))
    assert ids[0].tolist() == [2, 1]
    assert np.allclose(w[0], [s2 / (s2 + 1.0), 1.0 / (s2 + 1.0)], rtol=1e-15)


def test_sqrt_softplus_selection_follows_logit_order():
    # without a bias the score is increasing in the logit, so the selection is
    # the plain one (ties included)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((9, 32))
    wr = rng.standard_normal((50, 32))
    ids, _, _ = moe.route(x, wr, 6)
    ids2, _, _, _ = moe.route_variant(x, wr, 6, score=moe.SCORE_SQRT_SOFTPLUS)
    assert np.array_equal(ids, ids2)
