"""Pins of the head-less draft step of the oracle (scale, soft cap, argmax).

The pages say only that a draft without a Markov head scales and soft caps
the backbone rows and that a greedy request takes the best token of every
row; the formula is the reading stated in oracle.draft_step.scale_cap.  These
checks tie it to closed forms and to a brute-force scan, so that a dropped
multiplier, a cap applied before the multiplier, a highest-id tie rule or a
wrong d2t direction fails one of them.
"""
import math

import numpy as np
import pytest

import draft_inputs as di
from oracle import draft_step as O


def test_no_cap_is_the_multiplier_alone():
    z = np.array([-3.5, 0.0, 1.25, 7.0])
    assert np.array_equal(O.scale_cap(z, 2.0, 0.0), 2.0 * z)
    assert np.array_equal(O.scale_cap(z, 0.5, -1.0), 0.5 * z)


def test_cap_closed_forms():
    # cap * tanh(scale * z / cap): tanh(atanh(y)) = y, odd, bounded by the cap
    cap, scale = 3.0, 2.0
    z = cap * math.atanh(0.25) / scale            # -> cap * 0.25
    assert O.scale_cap(np.array([z]), scale, cap)[0] == pytest.approx(0.75, rel=1e-15)
    assert O.scale_cap(np.array([0.0]), scale, cap)[0] == 0.0
    x = np.linspace(-40, 40, 81)
    y = O.scale_cap(x, scale, cap)
    assert np.allclose(y, -O.scale_cap(-x, scale, cap), rtol=0, atol=0)
    assert np.all(np.abs(y) <= cap) and y[-1] == pytest.approx(cap, rel=1e-12)
    # the multiplier comes first: cap * tanh(scale z / cap), not scale * cap * tanh(z / cap)
    z1 = np.array([1.7])
    assert O.scale_cap(z1, scale, cap)[0] == pytest.approx(cap * math.tanh(scale * 1.7 / cap), rel=1e-15)
    assert abs(O.scale_cap(z1, scale, cap)[0] - scale * cap * math.tanh(1.7 / cap)) > 1e-3


def test_small_values_follow_the_multiplier():
    # |scale z| << cap: cap tanh(x / cap) = x - x^3 / (3 cap^2) + ...
    z = np.array([1e-3, -2e-3, 5e-4])
    y = O.scale_cap(z, 1.5, 30.0)
    x = 1.5 * z
    assert np.allclose(y, x - x ** 3 / (3 * 30.0 ** 2), rtol=1e-12, atol=0)


def test_positive_multiplier_required():
    with pytest.raises(AssertionError):
        O.scale_cap(np.zeros(3), 0.0, 1.0)
    with pytest.raises(AssertionError):
        O.scale_cap(np.zeros(3), -1.0, 0.0)


def _brute_argmax(row):
    best, arg = -math.inf, 0
    for v, x in enumerate(row):      # ascending ids, strict >: the lowest id wins a tie
        if x > best:
            best, arg = x, v
    return arg


@pytest.mark.parametrize("seed", range(20))
def test_argmax_rows_equals_a_scan(seed):
    rng = np.random.default_rng(seed)
    M, V = 6, 97
    z = rng.normal(size=(M, V)) * rng.uniform(0.1, 20)
    scale, cap = float(rng.uniform(0.3, 3.0)), float(rng.choice([0.0, 1.0, 5.0, 30.0]))
    ids, tok, vals = O.argmax_rows(z, scale, cap, None)
    zs = O.scale_cap(z, scale, cap)
    for m in range(M):
        assert ids[m] == _brute_argmax(zs[m])
        assert vals[m] == zs[m, ids[m]]
    assert np.array_equal(tok, ids)


def test_ties_after_the_cap_take_the_lowest_id():
    # tanh saturates to exactly 1.0 in fp64 past about 19.1: ids 3 and 5 tie at the cap
    z = np.array([[5.0, 1.0, -2.0, 40.0, 0.0, 60.0, 3.0]])
    ids, _, vals = O.argmax_rows(z, 1.0, 1.0, None)
    assert ids[0] == 3 and vals[0] == 1.0
    # without the cap the larger logit wins
    ids2, _, _ = O.argmax_rows(z, 1.0, 0.0, None)
    assert ids2[0] == 5


def test_exact_ties_on_dyadic_rows():
    z = np.array([[0.5, 0.75, 0.75, -1.0], [-0.25, -0.25, -0.25, -0.25]])
    ids, _, _ = O.argmax_rows(z, 2.0, 0.0, None)
    assert list(ids) == [1, 0]


def test_d2t_maps_the_winner():
    z = np.array([[0.0, 3.0, 1.0], [2.0, -1.0, 0.0]])
    d2t = np.array([10, 20, 30], np.int64)        # target = draft id + d2t[id]
    ids, tok, _ = O.argmax_rows(z, 1.0, 0.0, d2t)
    assert list(ids) == [1, 0] and list(tok) == [21, 10]


def test_monotone_transform_keeps_the_argmax_without_saturation():
    inp = di.make_inputs(di.SHAPES["tiny"])
    z = O.logits(inp.hidden, inp.lm_head)
    ids_plain, _, _ = O.argmax_rows(z, 1.0, 0.0, None)
    ids_cap, _, _ = O.argmax_rows(z, 1.3, 50.0, None)   # |z| << 50: no ties created
    assert np.array_equal(ids_plain, ids_cap)
    assert np.array_equal(ids_plain, np.argmax(z, axis=1))


def test_draft_argmax_composes_the_steps():
    inp = di.make_inputs(di.SHAPES["tiny"])
    ids, tok, vals = O.draft_argmax(inp.hidden, inp.lm_head, None, 0.8, 2.0)
    z = O.logits(inp.hidden, inp.lm_head)
    ids2, tok2, vals2 = O.argmax_rows(z, 0.8, 2.0, None)
    assert np.array_equal(ids, ids2) and np.array_equal(tok, tok2) and np.array_equal(vals, vals2)
