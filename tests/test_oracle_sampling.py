"""Pins of the oracle's temperature / top-k sampler: closed forms of two-candidate
draws, argmax special cases, tie order, exclusion of everything below the top k, and
stratified draws against the softmax."""

import math

import numpy as np

from oracle.sampling import sample_top_k, top_k_order


def test_top_k_one_or_zero_temperature_is_argmax():
    g = np.random.default_rng(0)
    l = g.normal(size=300).astype(np.float32)
    for u in (0.0, 0.3, 0.999):
        assert sample_top_k(l, 0.8, 1, u) == int(np.argmax(l))
        assert sample_top_k(l, 0.0, 250, u) == int(np.argmax(l))
    tie = np.array([0, 4, 1, 4, 4], np.float32)
    assert sample_top_k(tie, 0.7, 1, 0.9) == 1


def test_two_candidates_boundary_closed_form():
    """logits [2, 1, 0], top 2, temperature 1: index 0 has probability 1/(1+e^-1);
    the draw switches from index 0 to index 1 exactly at u = 1/(1+e^-1) = 0.73106."""
    l = np.array([2.0, 1.0, 0.0], np.float32)
    b = 1.0 / (1.0 + math.exp(-1.0))
    assert abs(b - 0.7310585786) < 1e-9
    assert sample_top_k(l, 1.0, 2, b - 1e-9) == 0
    assert sample_top_k(l, 1.0, 2, b + 1e-9) == 1
    assert sample_top_k(l, 1.0, 2, 0.999999) == 1      # index 2 is outside the top 2
    # temperature 0.7 sharpens: boundary 1/(1+exp(-1/0.7)), temperature widened from float32
    t = float(np.float32(0.7))
    b7 = 1.0 / (1.0 + math.exp(-1.0 / t))
    assert sample_top_k(l, 0.7, 2, b7 - 1e-9) == 0
    assert sample_top_k(l, 0.7, 2, b7 + 1e-9) == 1
    # all three: boundaries at 1/Z and (1+e^-1)/Z, Z = 1 + e^-1 + e^-2
    Z = 1 + math.exp(-1) + math.exp(-2)
    assert sample_top_k(l, 1.0, 3, 1 / Z - 1e-9) == 0
    assert sample_top_k(l, 1.0, 3, 1 / Z + 1e-9) == 1
    assert sample_top_k(l, 1.0, 3, (1 + math.exp(-1)) / Z + 1e-9) == 2


def test_draw_exactly_on_a_boundary_takes_the_next_candidate():
    """Two equal top logits have weights 1 and 1 (running sums 1, 2); u = 0.5 puts the
    threshold u * 2 = 1 exactly on the first running sum. The draw is the first candidate
    whose running sum exceeds the threshold strictly: index 1 (u = 0.5 - 2^-40: index 0)."""
    l = np.array([0.0, 0.0, -50.0], np.float32)
    assert sample_top_k(l, 1.0, 2, 0.5) == 1
    assert sample_top_k(l, 1.0, 2, 0.5 - 2.0 ** -40) == 0
    assert sample_top_k(l, 1.0, 3, 0.0) == 0


def test_order_and_ties_at_the_cut():
    """Equal logits are ordered by lower index, also across the top-k cut."""
    l = np.array([0, 5, 3, 5, 3, 3], np.float32)
    assert list(top_k_order(l, 3)) == [1, 3, 2]
    drawn = {sample_top_k(l, 1.0, 3, u) for u in np.linspace(0, 0.999999, 4001)}
    assert drawn == {1, 3, 2}
    # u = 0 always takes the largest logit (lowest index among equals)
    assert sample_top_k(l, 1.0, 3, 0.0) == 1


def test_nothing_below_the_top_k_is_drawn():
    g = np.random.default_rng(1)
    l = g.normal(size=2048).astype(np.float32)
    keep = set(np.argsort(-l.astype(np.float64), kind="stable")[:250].tolist())
    us = g.random(3000)
    got = [sample_top_k(l, 0.8, 250, u) for u in us]
    assert set(got) <= keep
    assert len(set(got)) > 150                          # the draws do spread over the set


def test_stratified_draws_match_softmax():
    """With N stratified draws u = (i + 1/2)/N, the count of each candidate is within one
    of N times its probability (the draw inverts the categorical CDF)."""
    g = np.random.default_rng(2)
    l = (3 * g.normal(size=40)).astype(np.float32)
    k, t, N = 7, 0.8, 20000
    idx = np.argsort(-l.astype(np.float64), kind="stable")[:k]
    z = l[idx].astype(np.float64) / float(np.float32(t))
    p = np.exp(z - z.max())
    p /= p.sum()
    counts = {int(i): 0 for i in idx}
    for i in range(N):
        counts[sample_top_k(l, t, k, (i + 0.5) / N)] += 1
    for j, i in enumerate(idx):
        assert abs(counts[int(i)] - N * p[j]) <= 1.0 + 1e-9, (i, counts[int(i)], N * p[j])
