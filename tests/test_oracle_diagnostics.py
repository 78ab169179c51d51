"""Pins of the routing diagnostics (QEvict notes, section 3) -- CPU only.

Each quantity is checked against a case whose answer follows from its
definition by hand: uniform attention (zero query) gives shares equal to
token counts over N, two logits ln 3 apart give 3/4 and 1/4, Jaccard
distances of small sets, and re-entry counts of a hand-made membership
history.
"""
import math

import numpy as np
import pytest

from oracle import diagnostics as dg


def test_full_attention_zero_query_is_uniform_and_fmm_counts_dropped():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((2, 10, 8))
    p = dg.full_attention(np.zeros((4, 8)), k)
    assert p.shape == (4, 10)
    np.testing.assert_allclose(p, 0.1, rtol=0, atol=1e-15)
    held = np.ones(10, bool)
    held[[1, 4, 7]] = False
    assert dg.future_missed_mass(p, held) == pytest.approx(0.3, abs=1e-15)
    assert dg.future_missed_mass(p, np.ones(10, bool)) == 0.0


def test_full_attention_two_logits_ln3_apart():
    # d = 1: logits q*k / sqrt(1) = ln 3 and 0 -> probabilities 3/4, 1/4
    q = np.array([[math.log(3.0)]])
    k = np.array([[[1.0], [0.0]]])
    p = dg.full_attention(q, k)
    np.testing.assert_allclose(p, [[0.75, 0.25]], rtol=0, atol=1e-15)
    assert dg.future_missed_mass(p, np.array([False, True])) == pytest.approx(0.75, abs=1e-15)


def test_full_attention_groups_query_heads_onto_their_kv_head():
    # Hq = 2, Hkv = 2 (G = 1) against Hq = 2, Hkv = 1 (G = 2): with one KV
    # head both query heads read it; with two, head 1 reads KV head 1
    k = np.array([[[0.0], [1.0]], [[1.0], [0.0]]])            # [Hkv=2, N=2, d=1]
    q = np.array([[math.log(3.0)], [math.log(3.0)]])
    p = dg.full_attention(q, k)
    np.testing.assert_allclose(p, [[0.25, 0.75], [0.75, 0.25]], atol=1e-15)
    p1 = dg.full_attention(q, k[:1])
    np.testing.assert_allclose(p1, [[0.25, 0.75], [0.25, 0.75]], atol=1e-15)
    # the share is the mean over query heads
    assert dg.future_missed_mass(p, np.array([True, False])) == pytest.approx(0.5, abs=1e-15)


def test_tier_shares_sum_to_one_and_follow_counts_under_uniform_attention():
    tiers = np.array([1, 2, 2, 3, 4, 4, 4, 5, 5, 5, 5, 2])
    p = dg.full_attention(np.zeros((2, 4)), np.ones((1, len(tiers), 4)))
    sh = dg.tier_shares(p, tiers, (1, 2, 3, 4, 5))
    assert sum(sh.values()) == pytest.approx(1.0, abs=1e-14)
    for t, n in {1: 1, 2: 3, 3: 1, 4: 3, 5: 4}.items():
        assert sh[t] == pytest.approx(n / len(tiers), abs=1e-15)
    assert dg.future_missed_mass(p, tiers != 5) == pytest.approx(sh[5], abs=1e-15)


def test_jaccard_distance_cases():
    assert dg.jaccard_distance({1, 2, 3}, {2, 3, 4}) == pytest.approx(0.5)
    assert dg.jaccard_distance({1, 2}, {1, 2}) == 0.0
    assert dg.jaccard_distance({1}, {2}) == 1.0
    assert dg.jaccard_distance(set(), set()) == 0.0
    assert dg.jaccard_distance({1, 2, 3, 4}, {1}) == pytest.approx(0.75)
    assert dg.churn([{1, 2}, {1, 2}, {2, 3}, {4}]) == pytest.approx([0.0, 2 / 3, 1.0])


def test_recovery_counts_hand_history():
    # window 1 leaves at event 1 and returns at event 2; window 2 leaves at
    # event 2 and returns at event 3; window 3 is new at event 1 (an entry,
    # not a re-entry); window 4 enters at event 3 for the first time
    hist = [{1, 2}, {2, 3}, {1, 3}, {1, 2, 3, 4}]
    assert dg.recovery_counts(hist) == (2, 2)
    assert dg.lir(hist) == 1.0
    # exits that never come back
    assert dg.recovery_counts([{1, 2, 3}, {1}, {1, 4}, {4, 5}]) == (0, 3)
    assert dg.lir([{1, 2, 3}, {1}, {1, 4}, {4, 5}]) == 0.0
    # no exits at all
    assert dg.lir([{1}, {1, 2}, {1, 2, 3}]) == 0.0
    # a window may exit and return twice: two exits, two re-entries
    assert dg.recovery_counts([{7}, set(), {7}, set(), {7}]) == (2, 2)
