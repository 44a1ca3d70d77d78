"""Pins of the dense Markov walk of the oracle (one biased argmax per position).

Checked against a scalar brute force (every dot product written out), closed
forms (zero tables reduce it to the head-less argmax; rank-1 tables give the
bias a_s b_t), the token chain s_0 = last token, s_{p+1} = t(c_p), ragged
blocks and the target-id indexing of the tables under a pruned vocabulary.
"""
import math

import numpy as np
import pytest

import draft_inputs as di
from oracle import draft_step as O


def _brute(z, scale, cap, d2t, tables, last_tok, off):
    M, V = z.shape
    r = tables.shape[2]
    ids = []
    for q in range(len(last_tok)):
        s = int(last_tok[q])
        for m in range(off[q], off[q + 1]):
            best, arg = -math.inf, 0
            for v in range(V):
                t = v + (int(d2t[v]) if d2t is not None else 0)
                bias = sum(float(tables[0][s][i]) * float(tables[1][t][i]) for i in range(r))
                x = float(scale) * float(z[m, v])
                f = cap * math.tanh(x / cap) if cap > 0 else x
                if f + bias > best:
                    best, arg = f + bias, v
            ids.append(arg)
            s = arg + (int(d2t[arg]) if d2t is not None else 0)
    return np.array(ids)


@pytest.mark.parametrize("seed", range(6))
def test_dense_walk_equals_brute_force(seed):
    rng = np.random.default_rng(seed)
    R, L, V, Vt, r = 2, 3, 23, 31, 5
    z = rng.normal(size=(R * L, V))
    d2t = None
    if seed % 2:
        sub = rng.permutation(Vt)[:V]
        d2t = (sub - np.arange(V)).astype(np.int64)
    tables = rng.normal(size=(2, Vt, r)) * 0.7
    last = rng.integers(0, Vt, R)
    off = np.arange(R + 1) * L
    scale, cap = (1.3, 2.0) if seed % 3 else (0.9, 0.0)
    res = O.dense_walk(z, scale, cap, d2t, tables, last)
    assert np.array_equal(res.ids, _brute(z, scale, cap, d2t, tables, last, off))
    assert np.array_equal(res.tokens, O.draft_to_target(res.ids, d2t))


def test_zero_tables_reduce_to_the_headless_argmax():
    inp = di.make_inputs(di.SHAPES["tiny"])
    z = O.logits(inp.hidden, inp.lm_head)
    zero = np.zeros_like(inp.tables)
    res = O.dense_walk(z, 1.1, 3.0, None, zero, inp.last_tok)
    ids, tok, vals = O.argmax_rows(z, 1.1, 3.0, None)
    assert np.array_equal(res.ids, ids) and np.array_equal(res.values, vals)


def test_rank_one_tables_closed_form():
    # A[s] = a_s e, B[t] = b_t e: the bias of v after s is a_s * b_v
    V, r = 9, 3
    a = np.linspace(-1, 1, V)
    b = np.array([0.0, 2.0, -1.0, 0.5, 3.0, -2.0, 1.0, 0.25, -0.5])
    e = np.array([1.0, 0.0, 0.0])
    tables = np.stack([np.outer(a, e), np.outer(b, e)])
    z = np.zeros((2, V))
    res = O.dense_walk(z, 1.0, 0.0, None, tables, np.array([V - 1]))   # a_s = 1: bias = b_v
    assert res.ids[0] == 4                                             # b_4 = 3 is the largest
    # next position: s = 4, a_4 = 0 -> no bias, all tie -> lowest id
    assert res.ids[1] == 0
    assert res.values[0] == 3.0 and res.values[1] == 0.0


def test_chain_of_previous_tokens_and_override():
    rng = np.random.default_rng(5)
    V, r = 17, 4
    z = rng.normal(size=(4, V))
    tables = rng.normal(size=(2, V, r))
    last = np.array([3])
    res = O.dense_walk(z, 1.0, 0.0, None, tables, last)
    # re-checking with the walk's own previous tokens reproduces it
    prev = np.concatenate([[3], res.tokens[:-1]])
    res2 = O.dense_walk(z, 1.0, 0.0, None, tables, last, prev_override=prev)
    assert np.array_equal(res.ids, res2.ids)
    # row 0 depends on last_tok only
    c0, _, _ = O.dense_row(z[0], 1.0, 0.0, None, tables, 3)
    assert c0 == res.ids[0]


def test_ragged_blocks_walk_separately():
    rng = np.random.default_rng(9)
    V, r = 13, 3
    z = rng.normal(size=(5, V))
    tables = rng.normal(size=(2, V, r))
    last = np.array([1, 7, 2])
    off = np.array([0, 2, 2, 5])
    res = O.dense_walk(z, 1.0, 0.0, None, tables, last, row_offsets=off)
    a = O.dense_walk(z[0:2], 1.0, 0.0, None, tables, last[0:1])
    c = O.dense_walk(z[2:5], 1.0, 0.0, None, tables, last[2:3])
    assert np.array_equal(res.ids, np.concatenate([a.ids, c.ids]))


def test_pruned_vocabulary_indexes_the_tables_by_target_id():
    # B is zero outside the subset; the bias of draft v must use row t(v) of B
    V, Vt, r = 4, 10, 1
    d2t = np.array([6, 2, 5, -1], np.int64)          # targets 6, 3, 7, 2
    tables = np.zeros((2, Vt, r))
    tables[0, 0, 0] = 1.0
    tables[1, 7, 0] = 5.0                             # only target 7 (draft id 2) gets a bias
    z = np.array([[1.0, 2.0, 0.0, 1.5]])
    res = O.dense_walk(z, 1.0, 0.0, d2t, tables, np.array([0]))
    assert res.ids[0] == 2 and res.tokens[0] == 7 and res.values[0] == 5.0
