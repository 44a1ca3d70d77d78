"""Pins of the oracle's sampled walk (CPU).

The sampled walk draws every position from the lattice row after the slot
drawn before, with float weights, double sums and a double uniform
(openvino.genai page "Add DSpark and DFlash v2 drafts and sampled drafting ...",
commit "DFlash-2 Markov head / BlockRowSource" and the sampled-drafting
commits on double sums and double uniforms).  These tests pin it to closed
forms, to the greedy walk in the zero-temperature limit, to the exact
inverse-CDF counts of a uniform grid, and to the double-sum behaviour the
pages describe (weights below half a float ulp of the running sum are drawn).
"""
import numpy as np
import pytest

from oracle import draft_step as O


def lattice(L, K, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((L, K)) * scale
    S = [rng.standard_normal((1, K)) * scale] + [rng.standard_normal((K, K)) * scale for _ in range(L - 1)]
    return u.astype(np.float32).astype(np.float64), [s.astype(np.float32).astype(np.float64) for s in S]


def test_single_candidate_is_always_drawn():
    u, S = lattice(5, 1, 0)
    sw = O.sampled(u, S, np.array([0.0, 0.3, 0.5, 0.9, 0.999999]))
    assert np.all(sw.path == 0)
    assert np.all(sw.q == 1.0)


def test_equal_rows_draw_the_floor_of_k_times_u():
    # all scores equal: q = 1/K and slot = floor(K U) (dyadic boundaries are exact)
    K, L = 4, 7
    u = np.zeros((L, K))
    S = [np.zeros((1, K))] + [np.zeros((K, K)) for _ in range(L - 1)]
    U = np.array([0.0, 0.2499999, 0.25, 0.5, 0.7499, 0.75, 0.9999999])
    sw = O.sampled(u, S, U)
    assert list(sw.path) == [0, 0, 1, 2, 2, 3, 3]
    assert np.all(sw.q == 0.25)


def test_two_slot_closed_form():
    # q_1 = 1 / (1 + e^{-(x_1 - x_0)}): slot 1 iff U >= q_0
    d = 0.7
    u = np.array([[0.0, d]])
    S = [np.zeros((1, 2))]
    w1 = float(np.float32(np.exp(np.float64(np.float32(0.0)))))   # the max row entry has weight 1
    w0 = float(np.float32(np.exp(np.float64(np.float32(-np.float32(d))))))
    q0 = w0 / (w0 + w1)
    assert abs(q0 - 1.0 / (1.0 + np.exp(d))) < 1e-7
    for U, want in [(q0 * 0.999, 0), (q0 * 1.001, 1), (0.0, 0), (0.999999, 1)]:
        sw = O.sampled(u, S, np.array([U]))
        assert sw.path[0] == want, (U, q0)


@pytest.mark.parametrize("seed", range(20))
def test_zero_temperature_limit_is_the_greedy_walk(seed):
    u, S = lattice(6, 8, seed, scale=3.0)
    path_g, score_g, gap = O.greedy(u, S)
    if gap < 1e-2:
        pytest.skip("near tie")
    U = np.random.default_rng(seed + 100).random(6)
    sw = O.sampled(u, S, U, temperature=1e-4)
    assert list(sw.path) == list(path_g)
    assert sw.score == pytest.approx(score_g)


@pytest.mark.parametrize("seed", range(5))
def test_uniform_grid_counts_match_q(seed):
    # one position: over N equally spaced uniforms the count of each slot is N q_k up to
    # one grid step per boundary (the inverse CDF of the recorded proposal)
    K, N = 16, 20000
    u, S = lattice(1, K, seed, scale=2.0)
    counts = np.zeros(K)
    q = None
    for i in range(N):
        sw = O.sampled(u, S, np.array([(i + 0.5) / N]))
        counts[sw.path[0]] += 1
        q = sw.q[0]
    assert abs(q.sum() - 1.0) < 1e-12
    assert np.all(np.abs(counts / N - q) <= 2.0 / N)


def test_chain_follows_the_slot_drawn_before():
    # transitions that strongly favour staying: every later draw repeats the first
    K, L = 8, 6
    u = np.zeros((L, K))
    first = np.zeros((1, K))
    stay = np.full((K, K), -40.0)
    np.fill_diagonal(stay, 0.0)
    S = [first] + [stay.copy() for _ in range(L - 1)]
    for U0 in (0.05, 0.3, 0.55, 0.95):
        U = np.array([U0, 0.5, 0.01, 0.99, 0.7, 0.2])
        sw = O.sampled(u, S, U)
        assert np.all(sw.path == int(U0 * K))
        # later rows are the rows of the drawn slot: q concentrated on it
        assert np.all(sw.q[1:, sw.path[0]] > 1 - 1e-12)


def test_tail_below_half_a_float_ulp_is_drawn():
    # one weight 1 and 63 weights of about 2^-26 each (below half a float ulp of 1):
    # summed in float the tail would vanish; in double it holds 63 * 2^-26 of the mass
    K = 64
    x = np.full(K, np.log(2.0 ** -26))
    x[0] = 0.0
    u = x[None, :]
    S = [np.zeros((1, K))]
    sw = O.sampled(u, S, np.array([1.0 - 1e-7]))
    assert sw.path[0] >= 1
    tail = sw.q[0][1:].sum()
    assert tail == pytest.approx(63 * 2.0 ** -26 / (1 + 63 * 2.0 ** -26), rel=1e-6)
    assert O.sampled(u, S, np.array([0.999])).path[0] == 0
    # the exact slot: running sums 1 + k w in double (w = the fp32 weight of the tail)
    w = float(np.float32(np.exp(np.float64(np.float32(np.log(2.0 ** -26))))))
    total = 1.0
    for _ in range(63):
        total += w
    U = (1.0 + 10.5 * w) / total
    assert O.sampled(u, S, np.array([U])).path[0] == 11


def test_uniform_at_one_draws_the_last_slot():
    # U * total never exceeds the last running sum for U < 1; U = 1 (past the [0, 1)
    # contract) finds no slot and takes the last one
    K = 5
    u = np.array([[0.3, -0.2, 0.9, 0.0, -1.0]])
    S = [np.zeros((1, K))]
    assert O.sampled(u, S, np.array([1.0])).path[0] == K - 1
    assert O.sampled(u, S, np.array([np.nextafter(1.0, 0.0)])).path[0] == K - 1


@pytest.mark.parametrize("seed", range(10))
def test_score_is_the_path_score(seed):
    u, S = lattice(5, 6, seed)
    U = np.random.default_rng(seed).random(5)
    sw = O.sampled(u, S, U, temperature=0.7)
    assert sw.score == pytest.approx(O.path_score(u, S, sw.path))
    # every recorded row is a distribution, and the drawn slot has positive mass
    assert np.allclose(sw.q.sum(axis=1), 1.0)
    assert np.all(sw.q[np.arange(5), sw.path] > 0)


def test_temperature_scales_the_row():
    # T = 2 on the row x is T = 1 on the row x / 2
    u, S = lattice(4, 8, 3)
    U = np.array([0.1, 0.4, 0.6, 0.9])
    a = O.sampled(u, S, U, temperature=2.0)
    half = [s / 2 for s in S]
    b = O.sampled(u / 2, half, U, temperature=1.0)
    assert list(a.path) == list(b.path)
    assert np.allclose(a.q, b.q, rtol=1e-6)


def test_block_level_sampled_walk_uses_each_requests_rows():
    # the whole step with a sampled walk: ragged blocks draw with their own uniforms
    import draft_inputs as di
    sh = di.custom_shape("samp", R=3, L=4, H=64, Vd=300, K=8, r=8, table_std=0.5, seed=4)
    inp = di.make_inputs(sh)
    off = di.ragged_offsets([4, 0, 3])
    hidden = inp.hidden[:7]
    U = np.random.default_rng(9).random(7)
    res = O.draft_block(hidden, inp.lm_head, None, inp.tables, None, inp.last_tok, 8, row_offsets=off,
                        walk=O.WALK_SAMPLED, uniforms=U, temperature=1.0)
    assert res.q.shape == (7, 8)
    for r, (a, b) in enumerate([(0, 4), (4, 4), (4, 7)]):
        if b == a:
            assert res.scores[r] == 0.0
            continue
        sw = O.sampled(res.cand.unary[a:b], res.S[r], U[a:b])
        assert list(res.slots[a:b]) == list(sw.path)
        assert np.array_equal(res.tokens[a:b], res.cand.tok[a:b][np.arange(b - a), sw.path])
