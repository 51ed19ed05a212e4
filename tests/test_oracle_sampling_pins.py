"""Pins of the oracle's temperature / top-p sampler against facts fixed outside it: a worked
example derived by hand, the greedy and uniform special cases, the softmax from scipy, the
temperature as a logit scale, and a brute-force nucleus over every candidate set of a tiny
vocabulary."""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

from oracle.sampling import nucleus, sample, sample_row


def test_worked_example_by_hand():
    # logits [0, 2, -1, 1], T = 1: probabilities (by hand, e^x over 11.475217)
    # token1 0.643914, token3 0.236883, token0 0.087144, token2 0.032059.
    # top_p 0.9: largest-first running mass 0.6439, 0.8808, 0.9679 -> nucleus {1, 3, 0}, mass 0.967941.
    # Draw in id order over the nucleus: running 0.087144 (t0), 0.731058 (t1), 0.967941 (t3).
    l = [0.0, 2.0, -1.0, 1.0]
    assert list(np.nonzero(nucleus(l, 1.0, 0.9))[0]) == [0, 1, 3]
    cases = {0.05: 0, 0.08: 0, 0.0901: 1, 0.5: 1, 0.9: 3, 0.999: 3}   # u * 0.967941 against the running mass
    for u, tok in cases.items():
        assert sample_row(l, 1.0, 0.9, u) == tok, u
    # top_p 0.85: 0.8808 already reaches it -> nucleus {1, 3}; u = 0.05 lands on token 1
    assert list(np.nonzero(nucleus(l, 1.0, 0.85))[0]) == [1, 3]
    assert sample_row(l, 1.0, 0.85, 0.05) == 1
    assert sample_row(l, 1.0, 0.85, 0.75) == 3   # 0.75 * 0.880797 = 0.6606 > 0.643914


def test_greedy_is_argmax():
    rng = np.random.default_rng(0)
    l = rng.standard_normal((5, 300))
    l[2, [7, 9]] = 10.0                          # tie: the lower id wins
    ids = sample(l, 0.0, 0.95, rng.random(5))
    np.testing.assert_array_equal(ids, np.argmax(l, axis=1))
    assert ids[2] == 7


def test_all_equal_logits_draw_floor_u_times_v():
    v = 1000
    for u in [0.0, 0.3141, 0.5003, 0.99999]:   # away from the k / v boundaries, where rounding decides
        assert sample_row(np.full(v, 1.25), 1.0, 0.95, u) == int(np.floor(u * v))   # all tied: nucleus is every token


def test_tiny_top_p_keeps_only_the_top_logit():
    rng = np.random.default_rng(1)
    l = rng.standard_normal(500)
    for u in np.linspace(0, 0.999, 7):
        assert sample_row(l, 1.0, 1e-9, u) == int(np.argmax(l))


def test_stratified_draws_reproduce_softmax():
    # u_k = (k + 1/2) / n: an inverse-CDF draw hits token i about n * p_i times (within 1)
    rng = np.random.default_rng(2)
    l = rng.standard_normal(40) * 2
    n = 20000
    us = (np.arange(n) + 0.5) / n
    counts = np.bincount([sample_row(l, 1.0, 1.0, u) for u in us], minlength=40)
    np.testing.assert_allclose(counts, n * softmax(l), atol=1.0 + 1e-9)
    # with top_p < 1 the draws follow the renormalised nucleus and nothing outside it
    keep = nucleus(l, 1.0, 0.8)
    counts = np.bincount([sample_row(l, 1.0, 0.8, u) for u in us], minlength=40)
    p = np.where(keep, softmax(l), 0.0)
    np.testing.assert_allclose(counts, n * p / p.sum(), atol=1.0 + 1e-9)
    assert counts[~keep].sum() == 0


def test_temperature_scales_logits():
    rng = np.random.default_rng(3)
    l = rng.standard_normal(200) * 3
    for t in [0.5, 0.7, 2.0]:
        for u in rng.random(10):
            assert sample_row(l, t, 0.95, u) == sample_row(l / t, 1.0, 0.95, u)
        np.testing.assert_array_equal(nucleus(l, t, 0.9), nucleus(l / t, 1.0, 0.9))


@pytest.mark.parametrize("seed", range(6))
def test_nucleus_brute_force(seed):
    # every set closed under "higher logit" (ties move together) with mass >= top_p: the nucleus
    # is the one of least mass
    rng = np.random.default_rng(10 + seed)
    l = np.round(rng.standard_normal(7) * 1.5, 1)        # rounding makes ties likely
    p = softmax(l)
    for top_p in [0.3, 0.6, 0.9, 0.95]:
        best = None
        for bits in itertools.product([0, 1], repeat=len(l)):
            s = np.array(bits, dtype=bool)
            if not s.any():
                continue
            if s.any() and (l[~s].max(initial=-np.inf) >= l[s].min()):
                continue                                   # not upward-closed (a higher or tied logit left out)
            m = p[s].sum()
            if m >= top_p and (best is None or m < best[0]):
                best = (m, s)
        np.testing.assert_array_equal(nucleus(l, 1.0, top_p), best[1])


def test_mass_reaching_top_p_exactly_is_enough():
    # logits [0, ln 3]: the top token holds 3/4 of the mass, so top_p = 0.75 keeps it alone
    l = [0.0, float(np.log(3.0))]
    np.testing.assert_array_equal(nucleus(l, 1.0, 0.75), [False, True])
    assert all(sample_row(l, 1.0, 0.75, u) == 1 for u in [0.0, 0.2, 0.9])
    np.testing.assert_array_equal(nucleus(l, 1.0, 0.76), [True, True])


def test_tiny_temperature_keeps_only_the_maximum_and_its_ties():
    """A positive temperature so small that (l - max) / T overflows: every logit below the maximum
    gets probability 0, and the tied maxima share the mass evenly (the T -> 0+ limit of the
    softmax), so the draw picks among them by u in id order."""
    l = np.array([0.5, 2.0, -1.0, 2.0, 1.999])
    for u, want in ((0.0, 1), (0.49, 1), (0.5, 3), (0.99, 3)):
        assert sample_row(l, 1e-40, 0.95, u) == want
        assert sample_row(l, 1e-40, 1.0, u) == want
    assert sample_row(l, 0.0, 0.95, 0.99) == 1      # T = 0 is greedy: the lowest tied id

