"""Pins for the fp64 likelihood-mode oracle (CPU only).

Checked against closed forms (uniform logits give -log V; logits that are
log-probabilities give those log-probabilities back), the normalisation of a
distribution (exp of the scores of every possible target sums to one), shift
invariance of a row, brute force without the maximum subtraction on small
logits, and rows whose logits would overflow exp() without it.
"""
import math

import numpy as np

import oracle


def test_uniform_logits_score_minus_log_vocab():
    V = 1000
    logits = np.full((3, 4, V), 2.5)
    targets = np.array([[0, 1, 999, 500]] * 3)
    lp = oracle.token_logprobs(logits, targets)
    assert lp.shape == (3, 4)
    np.testing.assert_allclose(lp, -math.log(V), rtol=0, atol=1e-12)


def test_log_probabilities_come_back():
    rng = np.random.default_rng(1)
    p = rng.dirichlet(np.ones(37), size=5)
    t = rng.integers(0, 37, size=5)
    lp = oracle.token_logprobs(np.log(p), t)
    np.testing.assert_allclose(lp, np.log(p[np.arange(5), t]), rtol=0, atol=1e-12)


def test_scores_of_all_targets_normalise_and_shift():
    rng = np.random.default_rng(2)
    row = rng.normal(0, 3, size=50)
    all_t = np.arange(50)
    lp = oracle.token_logprobs(np.broadcast_to(row, (50, 50)), all_t)
    assert abs(np.exp(lp).sum() - 1.0) < 1e-12
    lp2 = oracle.token_logprobs(np.broadcast_to(row + 123.0, (50, 50)), all_t)
    np.testing.assert_allclose(lp, lp2, rtol=0, atol=1e-10)


def test_brute_force_small_logits():
    rng = np.random.default_rng(3)
    logits = rng.normal(0, 1, size=(6, 9))
    targets = rng.integers(0, 9, size=6)
    lp = oracle.token_logprobs(logits, targets)
    for i in range(6):
        den = 0.0
        for v in range(9):
            den += math.exp(float(logits[i, v]))
        assert abs(lp[i] - math.log(math.exp(float(logits[i, targets[i]])) / den)) < 1e-12


def test_large_logits_stay_finite_and_out_of_range_target_is_nan():
    logits = np.array([[1000.0, 999.0, 0.0]])
    lp = oracle.token_logprobs(logits, np.array([1]))
    # p(1) = e^999 / (e^1000 + e^999 + 1) = 1 / (e + 1 + e^-999)
    assert abs(lp[0] + math.log(math.e + 1.0)) < 1e-12
    assert math.isnan(oracle.token_logprobs(logits, np.array([3]))[0])
    assert math.isnan(oracle.token_logprobs(logits, np.array([-1]))[0])


def test_sequence_loglik_is_the_sum():
    rng = np.random.default_rng(4)
    logits = rng.normal(0, 2, size=(2, 7, 11))
    targets = rng.integers(0, 11, size=(2, 7))
    ll = oracle.sequence_loglik(logits, targets)
    lp = oracle.token_logprobs(logits, targets)
    np.testing.assert_allclose(ll, lp.sum(axis=1), rtol=0, atol=1e-12)
