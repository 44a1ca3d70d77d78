"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Every oracle function is checked here against at least one of: values worked
by hand (tests/golden/, with their derivation), closed forms, exact rational
arithmetic, brute-force enumeration on tiny inputs, and invariants of the
mathematics.  A plausible mistake (a dropped term, a swapped table, a
transposed operand, a wrong tie rule) fails at least one of them.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import draft_inputs as di
from oracle import draft_step as O


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _bits(x):
    """float values that are exact in bf16 -> bf16 bit patterns (test helper, exact cases only)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


# ---------------------------------------------------------------- bf16 / logits

def test_bf16_widening_known_patterns():
    # IEEE binary32 upper halves: 1.0, -2.0, 1+2^-7, smallest subnormal 2^-133, +inf, 0.15625
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F80, 0x3E20], dtype=np.uint16)
    got = O.bf16_to_f64(bits)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, math.inf, 0.15625]
    assert list(got) == want


def test_bf16_rounding_of_generator_is_rne():
    # ties to even at the 16-bit boundary: 1 + 2^-8 is halfway between 1 and 1+2^-7 -> 1.0 (even)
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20], np.float32)
    got = O.bf16_to_f64(di.round_to_bf16_bits(x))
    assert list(got) == [1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7]


def test_logits_exact_rational():
    rng = np.random.default_rng(11)
    hb = di.round_to_bf16_bits(rng.standard_normal((3, 40)).astype(np.float32))
    wb = di.round_to_bf16_bits((0.02 * rng.standard_normal((17, 40))).astype(np.float32))
    z = O.logits(hb, wb, vocab_block=5)   # several vocabulary blocks
    h = O.bf16_to_f64(hb)
    w = O.bf16_to_f64(wb)
    for m in range(3):
        for v in range(17):
            exact = sum(Fraction(float(w[v, i])) * Fraction(float(h[m, i])) for i in range(40))
            bound = 40 * 2.0 ** -52 * float(sum(abs(Fraction(float(w[v, i] * h[m, i]))) for i in range(40)))
            assert abs(Fraction(float(z[m, v])) - exact) <= Fraction(bound)


def test_logits_one_hot_hidden_picks_a_column():
    rng = np.random.default_rng(3)
    wb = di.round_to_bf16_bits((0.02 * rng.standard_normal((50, 16))).astype(np.float32))
    h = np.zeros((2, 16), np.float32)
    h[0, 3] = 1.0
    h[1, 7] = -4.0
    z = O.logits(_bits(h), wb)
    w = O.bf16_to_f64(wb)
    assert np.array_equal(z[0], w[:, 3])
    assert np.array_equal(z[1], -4.0 * w[:, 7])


# ---------------------------------------------------------------- LSE

def test_lse_closed_forms():
    # a constant row c over V entries: c + ln V
    for c, V in [(0.0, 1024), (-3.25, 151936), (7.5, 48)]:
        assert abs(O.row_lse(np.full((1, V), c))[0] - (c + math.log(V))) < 1e-12
    # two entries: a + log1p(e^(b-a))
    a, b = 1.5, -0.75
    assert abs(O.row_lse(np.array([[a, b]]))[0] - (a + math.log1p(math.exp(b - a)))) < 1e-15
    # no overflow for large logits, and shift covariance lse(z + c) = lse(z) + c
    z = np.array([[1000.0, 999.0, 998.0]])
    assert abs(O.row_lse(z)[0] - (1000.0 + math.log(1 + math.exp(-1) + math.exp(-2)))) < 1e-12
    rng = np.random.default_rng(0)
    z = rng.standard_normal((4, 300))
    assert np.allclose(O.row_lse(z + 12.5), O.row_lse(z) + 12.5, atol=1e-12)


# ---------------------------------------------------------------- Top-K

def _rank_definition(z_row, K):
    """Slot k is the id whose count of (strictly larger, or equal with smaller id) entries is k."""
    V = len(z_row)
    out = [None] * K
    for v in range(V):
        rank = sum(1 for w in range(V) if z_row[w] > z_row[v] or (z_row[w] == z_row[v] and w < v))
        if rank < K:
            out[rank] = v
    return out


@pytest.mark.parametrize("seed", range(20))
def test_topk_matches_rank_definition_with_many_ties(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(1, 90))
    K = int(rng.integers(1, V + 1))
    z = rng.integers(-3, 4, size=V).astype(np.float64) * 0.5   # heavy exact ties
    assert list(O.topk_slots(z, K)) == _rank_definition(list(z), K)


def test_topk_special_cases():
    # all-equal row -> ids 0..K-1
    assert list(O.topk_slots(np.zeros(1000), 64)) == list(range(64))
    # -0.0 and +0.0 are equal, so the lower id wins
    z = np.array([-0.0, 0.0, -1.0, -0.0])
    assert list(O.topk_slots(z, 4)) == [0, 1, 3, 2]
    # planted maxima
    z = np.linspace(-1, 0, 500)
    z[[17, 400, 3]] = [5.0, 4.0, 3.0]
    assert list(O.topk_slots(z, 4)) == [17, 400, 3, 499]
    # K = V: the full order
    rng = np.random.default_rng(5)
    z = rng.standard_normal(48)
    assert list(O.topk_slots(z, 48)) == list(np.argsort(-z, kind="stable"))


def test_k_is_min_64_and_draft_vocab():
    # optimum-intel page "Support MiniCPM-OCR-1.0-DSpark": top_k = min(64, draft_vocab_size);
    # its tiny draft predicts 48 target tokens
    assert O.top_k_count(48) == 48
    assert O.top_k_count(114688) == 64
    assert O.top_k_count(64) == 64


# ---------------------------------------------------------------- d2t

def test_d2t_maps_i_to_i_plus_offset():
    sub = np.random.default_rng(9).permutation(200)[:48]   # unsorted subset of 48 target tokens
    d2t = sub - np.arange(48)
    assert np.array_equal(O.draft_to_target(np.arange(48), d2t), sub)
    assert np.array_equal(O.draft_to_target(np.array([[5, 0], [47, 5]]), d2t),
                          np.array([[sub[5], sub[0]], [sub[47], sub[5]]]))
    assert np.array_equal(O.draft_to_target(np.array([3, 1]), None), [3, 1])
    assert O.check_d2t(d2t, 48, 200) == (True, True)
    bad = d2t.copy()
    bad[2] = 200 - 2           # target 200 is out of range
    assert O.check_d2t(bad, 48, 200) == (False, False)
    dup = d2t.copy()
    dup[1] = sub[0] - 1        # draft 1 -> the same target as draft 0
    assert O.check_d2t(dup, 48, 200) == (True, False)
    assert O.check_d2t(d2t[:-1], 48, 200) == (False, False)


# ---------------------------------------------------------------- gate / pairwise

def test_gate_closed_forms():
    assert O.gate(np.ones(8), None) == 1.0
    assert O.gate(np.ones(8), np.zeros(8)) == 0.5
    assert O.gate(np.array([1.0, 2.0]), np.array([math.log(3.0), 0.0])) == pytest.approx(0.75, abs=1e-15)
    assert O.gate(np.array([1.0]), np.array([-800.0])) == 0.0


def test_pairwise_rank1_and_zero():
    V, r = 30, 1
    rng = np.random.default_rng(2)
    t = rng.standard_normal((2, V, r))
    prev = np.array([4, 9, 4])
    cand = np.array([1, 2])
    pi = O.pairwise(t, prev, cand, 0.25)
    want = np.array([[0.25 * t[0, s, 0] * t[1, c, 0] for c in cand] for s in prev])
    assert np.allclose(pi, want, rtol=0, atol=1e-15)
    assert np.all(O.pairwise(np.zeros((2, V, 16)), prev, cand, 1.0) == 0.0)


# ---------------------------------------------------------------- walk: hand-worked fixtures

def test_golden_lattice_k2_l3(golden_dir):
    g = _load(golden_dir, "lattice_hand_k2_l3.json")
    u = np.array(g["u"])
    S = [np.array(s) for s in g["S"]]
    path, score, margin = O.viterbi(u, S)
    assert list(path) == g["viterbi_path"] and score == g["viterbi_score"] and margin == g["viterbi_margin"]
    path, score, gap = O.greedy(u, S)
    assert list(path) == g["greedy_path"] and score == g["greedy_score"] and gap == g["greedy_gap"]
    bp, bs, bm = O.bruteforce(u, S)
    assert list(bp) == g["viterbi_path"] and bs == g["viterbi_score"] and bm == g["viterbi_margin"]
    assert O.path_score(u, S, g["viterbi_path"]) == g["viterbi_score"]


def test_golden_lattice_greedy_differs(golden_dir):
    g = _load(golden_dir, "lattice_hand_greedy_differs.json")
    u = np.array(g["u"])
    S = [np.array(s) for s in g["S"]]
    path, score, margin = O.viterbi(u, S)
    assert list(path) == g["viterbi_path"] and score == g["viterbi_score"] and margin == g["viterbi_margin"]
    path, score, gap = O.greedy(u, S)
    assert list(path) == g["greedy_path"] and score == g["greedy_score"] and gap == g["greedy_gap"]


@pytest.mark.parametrize("variant", ["ungated", "gated", "gated_off"])
def test_golden_draft_step(golden_dir, variant):
    g = _load(golden_dir, "draft_step_hand_v4.json")
    hidden = _bits(np.array(g["hidden"]))
    W = _bits(np.array(g["lm_head"]))
    d2t = np.array(g["d2t"], np.int64)
    tables = np.zeros((2, g["target_vocab"], 1))
    tables[0, :, 0] = g["table_A"]
    tables[1, :, 0] = g["table_B"]
    w = None if variant == "ungated" else np.array(g[variant + "_w"] if variant != "gated" else g["gated_w"])
    res = O.draft_block(hidden, W, d2t, tables, w, np.array([g["last_tok"]]), g["K"])
    want = g[variant]
    assert list(res.cand.idx[0]) == [1, 3] and list(res.cand.idx[1]) == [2, 3]
    assert list(res.slots) == want["slots"]
    assert list(res.tokens) == want["tokens"]
    assert res.scores[0] + res.cand.lse.sum() == pytest.approx(want["score_plus_lse"], abs=1e-15)


# ---------------------------------------------------------------- walk: brute force

def _run_walks(inp, walk=O.WALK_VITERBI):
    s = inp.shape
    return O.draft_block(inp.hidden, inp.lm_head, inp.d2t, inp.tables, inp.gate_w, inp.last_tok,
                         s.K, inp.row_offsets, walk)


def _check_against_bruteforce(res, R, L):
    for r in range(R):
        S = res.S[r]
        u = res.cand.unary[r * L:(r + 1) * L]
        bp, bs, bm = O.bruteforce(u, S)
        vp = res.slots[r * L:(r + 1) * L]
        assert abs(res.scores[r] - bs) <= 1e-12 * max(1.0, abs(bs))
        assert abs(res.margins[r] - bm) <= 1e-9 * max(1.0, abs(bs))
        if bm > 1e-9:
            assert list(vp) == list(bp)
        assert abs(O.path_score(u, S, vp) - bs) <= 1e-12 * max(1.0, abs(bs))


def test_tiny_viterbi_equals_bruteforce():
    inp = di.make_inputs(di.SHAPES["tiny"])
    res = _run_walks(inp)
    _check_against_bruteforce(res, 1, 5)


@pytest.mark.parametrize("base", ["tiny", "tiny_stress"])
def test_seed_sweep_viterbi_equals_bruteforce(base):
    s0 = di.SHAPES[base]
    first = 1000 if base == "tiny" else 2000
    changed = 0
    for seed in range(first, first + 200):
        shape = di.custom_shape(base, R=1, L=5, H=64, Vd=1024, K=8, r=16, table_std=s0.table_std,
                                seed=seed, weight_seed=seed)
        res = _run_walks(di.make_inputs(shape))
        _check_against_bruteforce(res, 1, 5)
        changed += int(np.any(res.slots != 0))
    if base == "tiny_stress":
        assert changed > 100   # the pairwise term really changes the choices


@pytest.mark.parametrize("seed", range(30))
def test_random_lattices_all_shapes(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 6))
    K = int(rng.integers(1, 6))
    u = rng.standard_normal((L, K))
    S = [rng.standard_normal((1, K))] + [rng.standard_normal((K, K)) for _ in range(L - 1)]
    vp, vs, vm = O.viterbi(u, S)
    bp, bs, bm = O.bruteforce(u, S)
    assert list(vp) == list(bp) and abs(vs - bs) < 1e-12 and (vm == bm or abs(vm - bm) < 1e-12)
    gp, gs, _ = O.greedy(u, S)
    assert gs <= vs + 1e-12
    # greedy run step by step from its definition
    prev = 0
    for p in range(L):
        vals = [u[p][k] + S[p][prev, k] for k in range(K)]
        best = max(vals)
        assert gp[p] == vals.index(best)
        prev = gp[p]


@pytest.mark.parametrize("seed", range(40))
def test_dyadic_exact_ties_follow_lowest_slot_rule(seed):
    # small integers: many exact ties, every sum exact in binary64
    rng = np.random.default_rng(500 + seed)
    L = int(rng.integers(1, 5))
    K = int(rng.integers(1, 5))
    u = rng.integers(-2, 3, size=(L, K)).astype(np.float64)
    S = [rng.integers(-2, 3, size=(1, K)).astype(np.float64)] + \
        [rng.integers(-2, 3, size=(K, K)).astype(np.float64) for _ in range(L - 1)]
    vp, vs, _ = O.viterbi(u, S)
    bp, bs, _ = O.bruteforce(u, S)
    assert list(vp) == list(bp) and vs == bs
    # the brute-force choice is, by its construction, min over optimal paths of the reversed sequence
    best = max(O.path_score(u, S, p) for p in itertools.product(range(K), repeat=L))
    opt = [p for p in itertools.product(range(K), repeat=L) if O.path_score(u, S, p) == best]
    assert tuple(vp) == min(opt, key=lambda p: tuple(reversed(p)))
    gp, _, _ = O.greedy(u, S)
    prev = 0
    for p in range(L):
        vals = [u[p][k] + S[p][prev, k] for k in range(K)]
        assert gp[p] == vals.index(max(vals))
        prev = gp[p]


def test_special_cases_zero_pairwise_k1_l1():
    rng = np.random.default_rng(7)
    L, K = 4, 6
    u = -np.sort(-rng.standard_normal((L, K)), axis=1)      # slot order: u descending
    Z = [np.zeros((1, K))] + [np.zeros((K, K)) for _ in range(L - 1)]
    vp, vs, _ = O.viterbi(u, Z)
    assert list(vp) == [0] * L and vs == pytest.approx(u[:, 0].sum(), abs=1e-15)
    gp, gs, _ = O.greedy(u, Z)
    assert list(gp) == [0] * L and gs == vs
    # K = 1: slot 0 everywhere
    u1 = rng.standard_normal((5, 1))
    S1 = [rng.standard_normal((1, 1))] + [rng.standard_normal((1, 1)) for _ in range(4)]
    vp, vs, vm = O.viterbi(u1, S1)
    assert list(vp) == [0] * 5 and vm == math.inf
    # L = 1: argmax of u_0 + S_0
    u2 = rng.standard_normal((1, 7))
    S2 = [rng.standard_normal((1, 7))]
    vp, vs, _ = O.viterbi(u2, S2)
    assert vp[0] == int(np.argmax(u2[0] + S2[0][0]))


# ---------------------------------------------------------------- invariants of the whole step

def _small_shape(**kw):
    base = dict(R=3, L=4, H=32, Vd=300, r=8, table_std=0.5, seed=77)
    base.update(kw)
    return di.custom_shape("small", **base)


def test_row_shift_invariance():
    inp = di.make_inputs(_small_shape())
    s = inp.shape
    z = O.logits(inp.hidden, inp.lm_head)
    a = O.draft_from_logits(z, s.K, None, inp.tables, inp.hidden, None, inp.last_tok)
    shift = np.arange(s.M)[:, None] * 0.375 - 1.0
    b = O.draft_from_logits(z + shift, s.K, None, inp.tables, inp.hidden, None, inp.last_tok)
    assert np.array_equal(a.tokens, b.tokens)
    assert np.allclose(a.scores, b.scores, atol=1e-12)


def test_request_isolation():
    inp = di.make_inputs(_small_shape())
    s = inp.shape
    a = _run_walks(inp)
    h2 = inp.hidden.copy()
    h2[s.L:2 * s.L] = di.round_to_bf16_bits(np.random.default_rng(1).standard_normal((s.L, s.H)).astype(np.float32))
    lt2 = inp.last_tok.copy()
    lt2[1] = (lt2[1] + 17) % s.Vt
    b = O.draft_block(h2, inp.lm_head, None, inp.tables, None, lt2, s.K)
    keep = np.r_[0:s.L, 2 * s.L:3 * s.L]
    assert np.array_equal(a.tokens[keep], b.tokens[keep])
    assert a.scores[0] == b.scores[0] and a.scores[2] == b.scores[2]
    assert not np.array_equal(a.tokens[s.L:2 * s.L], b.tokens[s.L:2 * s.L]) or a.scores[1] != b.scores[1]


def test_zero_d2t_equals_no_d2t_and_pruned_permutation_invariance():
    inp = di.make_inputs(_small_shape())
    s = inp.shape
    a = _run_walks(inp)
    b = O.draft_block(inp.hidden, inp.lm_head, np.zeros(s.Vd, np.int64), inp.tables, None, inp.last_tok, s.K)
    assert np.array_equal(a.tokens, b.tokens) and np.array_equal(a.scores, b.scores)
    # pruned: permuting the draft vocabulary (W rows and d2t targets together) leaves the tokens unchanged
    p = di.make_inputs(_small_shape(Vd=120, Vt=300, pruned=True, seed=5))
    ref = _run_walks(p)
    perm = np.random.default_rng(4).permutation(120)
    targets = np.arange(120) + p.d2t
    d2t_perm = targets[perm] - np.arange(120)
    res = O.draft_block(p.hidden, p.lm_head[perm], d2t_perm, p.tables, None, p.last_tok, p.shape.K)
    assert np.array_equal(ref.tokens, res.tokens)
    assert np.allclose(ref.scores, res.scores, atol=1e-12)
    assert set(ref.tokens) <= set(targets)


def test_pruned_tables_are_zero_outside_the_subset():
    p = di.make_inputs(_small_shape(Vd=120, Vt=300, pruned=True, seed=8))
    targets = np.arange(120) + p.d2t
    outside = np.setdiff1d(np.arange(300), targets)
    assert np.all(p.tables[:, outside] == 0) and np.all(np.any(p.tables[:, targets] != 0, axis=-1))


def test_ragged_blocks_equal_separate_runs():
    lengths = [3, 0, 5, 1]
    R = len(lengths)
    M = sum(lengths)
    shape = _small_shape(R=1, L=M)
    inp = di.make_inputs(shape)
    last = np.array([5, 6, 7, 8], np.int64)
    off = di.ragged_offsets(lengths)
    res = O.draft_block(inp.hidden, inp.lm_head, None, inp.tables, None, last, shape.K, off)
    for r in range(R):
        a, b = off[r], off[r + 1]
        if b == a:
            assert res.scores[r] == 0.0
            continue
        one = O.draft_block(inp.hidden[a:b], inp.lm_head, None, inp.tables, None, last[r:r + 1], shape.K)
        assert np.array_equal(one.tokens, res.tokens[a:b]) and one.scores[0] == res.scores[r]


def test_greedy_le_viterbi_and_equal_without_pairwise():
    inp = di.make_inputs(_small_shape(R=4))
    v = _run_walks(inp, O.WALK_VITERBI)
    g = _run_walks(inp, O.WALK_GREEDY)
    assert np.all(g.scores <= v.scores + 1e-12)
    inp.tables[:] = 0
    v = _run_walks(inp, O.WALK_VITERBI)
    g = _run_walks(inp, O.WALK_GREEDY)
    assert np.array_equal(v.tokens, g.tokens) and np.allclose(v.scores, g.scores, atol=1e-13)
    assert np.all(v.slots == 0)
