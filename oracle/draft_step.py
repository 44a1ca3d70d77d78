"""CPU oracle of the DFlash/DSpark draft step.

TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
statement of what the draft step computes.  Only ``tests/``, the smoke check
in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may use it;
the product path (``block_draft_markov_amd``) never imports it and shares no
code with it.

Sources (the three pull-request pages the method is described on):
  [G] openvino.genai "Add DSpark and DFlash v2 drafts and sampled drafting to
      DFlash speculative decoding": Description; Change (Markov heads); the
      commit "DFlash-2 Markov head / BlockRowSource" (a Top-K scorer run once
      over the packed block rows, the gated scorer reading the draft hidden
      states, the greedy walk "taking the best candidate after the token
      before"); the TopP commit (ties ordered by index); the d2t commit
      (greedy drafting accepts any d2t mapping).
  [E] optimum-intel "Export DFlash v2 and DSpark drafts for PagedAttention
      and continuous batching": What does this PR do? (packed Top-K lattice,
      transitions gated by the draft hidden states, no dense step).
  [X] optimum-intel "Support MiniCPM-OCR-1.0-DSpark": What does this PR do?
      (draft lm_head over the draft vocabulary; d2t maps draft token i to
      target token i + d2t[i]; the next-token table is zero outside the draft
      vocabulary; K = min(64, draft vocabulary)); Tests (a reference that
      scores over the draft vocabulary).

The pages fix no scoring formula.  The one used here (stated once):

  z_m[v]   = sum_i W[v, i] * h_m[i]                   logits of row m (fp64 from bf16)
  lse_m    = log sum_v exp(z_m[v])                    over the draft vocabulary
  slots    = the K largest z_m, ordered by (z desc, draft id asc)
  t_m[k]   = cand_m[k] + d2t[cand_m[k]]               (cand_m[k] when d2t is absent)
  u_m[k]   = z_m[cand_m[k]] - lse_m                   unary: log-softmax of the candidate
  g_m      = 1 / (1 + exp(-w . h_m))                  gated (DFlash v2) heads; 1 otherwise
  pi_m(s,k)= g_m * sum_i A[s, i] * B[t_m[k], i]       pairwise: previous token s -> candidate k
  Score(c) = sum_p u_{m(p)}[c_p] + pi_{m(p)}(s_p, c_p),  s_0 = last accepted token,
                                                      s_p = t_{m(p-1)}[c_{p-1}]
  Viterbi: the path of maximal Score; at every max the lowest slot wins.
  Greedy:  c_p = lowest argmax_k u_p[k] + pi_p(s_p, k), position by position.
  Sampled: c_p drawn from the row x_p[k] = (u_p[k] + pi_p(s_p, k)) / T with one
           double uniform per position: float weights exp(x - max x), running and
           total sums in double, the smallest k whose running sum exceeds U * total
           (see `sampled`); q_p = weights / total is the recorded proposal.

Readings where the pages are silent (each listed in the design notes):
  * the gate of a transition uses the hidden state of the row that produced
    the destination candidate, position 0 included;
  * the log-softmax runs over the draft vocabulary (V_d entries);
  * -0.0 and +0.0 compare equal (IEEE), so they tie and the lower id wins.

Every function here is pinned by tests/test_oracle_pins.py (brute force over
all K^L paths, closed forms, hand-worked fixtures in tests/golden/).
"""
from __future__ import annotations

import itertools
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------
# step 1: lm_head logits and their log-sum-exp
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64.

    A bf16 number is the upper 16 bits of an IEEE binary32, so widening
    to binary32 (and then binary64) is exact.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def logits(hidden_bits: np.ndarray, lm_head_bits: np.ndarray,
           vocab_block: int = 1 << 15) -> np.ndarray:
    """z[m, v] = sum_i W[v, i] * h[m, i] in float64, W in nn.Linear layout [V, H].

    A product of two bf16 numbers is exact in binary64 and the binary64 sum
    of H such products is far below any tolerance used against it.  Each
    z[m, v] is one dot product; the vocabulary is only split into separate
    matrix products to bound the float64 copy of W held at once.
    """
    h = bf16_to_f64(hidden_bits)
    V = lm_head_bits.shape[0]
    z = np.empty((h.shape[0], V), dtype=np.float64)
    for v0 in range(0, V, vocab_block):
        w = bf16_to_f64(lm_head_bits[v0:v0 + vocab_block])
        z[:, v0:v0 + w.shape[0]] = h @ w.T
    return z


def row_lse(z: np.ndarray) -> np.ndarray:
    """log sum_v exp(z[m, v]) per row, with the row maximum taken out first."""
    z = np.asarray(z, dtype=np.float64)
    mx = z.max(axis=-1)
    return mx + np.log(np.exp(z - mx[..., None]).sum(axis=-1))


# --------------------------------------------------------------------------
# step 2: Top-K slots, d2t, unary
# --------------------------------------------------------------------------

def top_k_count(draft_vocab: int) -> int:
    """K = min(64, draft vocabulary): at most one candidate per draft token ([X])."""
    return min(64, int(draft_vocab))


def topk_slots(z_row: np.ndarray, K: int) -> np.ndarray:
    """The K slots of one row: a full sort of the row by (z desc, draft id asc).

    Ordering equal logits by id follows the index-ordered ties of the TopP
    commit of [G] and the "lowest candidate slot" rule.
    """
    z_row = np.asarray(z_row, dtype=np.float64)
    ids = np.arange(z_row.shape[0])
    order = np.lexsort((ids, -z_row))   # last key is primary: -z ascending = z descending
    return order[:K].astype(np.int64)


def draft_to_target(cand: np.ndarray, d2t: Optional[np.ndarray]) -> np.ndarray:
    """Draft token i -> target token i + d2t[i] ([X]); the identity without d2t."""
    cand = np.asarray(cand, dtype=np.int64)
    if d2t is None:
        return cand.copy()
    return cand + np.asarray(d2t, dtype=np.int64)[cand]


@dataclass
class Candidates:
    idx: np.ndarray     # int64 [M, K] draft ids in slot order
    tok: np.ndarray     # int64 [M, K] target ids
    unary: np.ndarray   # float64 [M, K] log-softmax of the candidates
    z: np.ndarray       # float64 [M, K] their logits
    lse: np.ndarray     # float64 [M]
    zk1: np.ndarray     # float64 [M] the (K+1)-th largest logit (-inf when K = V_d)


def candidates(z: np.ndarray, K: int, d2t: Optional[np.ndarray]) -> Candidates:
    """Top-K slots, target ids and unary scores of every row of z."""
    z = np.asarray(z, dtype=np.float64)
    M, V = z.shape
    lse = row_lse(z) if M else np.zeros(0)
    idx = np.zeros((M, K), np.int64)
    zk1 = np.full(M, -np.inf)
    for m in range(M):
        order = topk_slots(z[m], min(K + 1, V))
        idx[m] = order[:K]
        if V > K:
            zk1[m] = z[m, order[K]]
    zc = np.take_along_axis(z, idx, axis=1)
    return Candidates(idx, draft_to_target(idx, d2t), zc - lse[:, None], zc, lse, zk1)


# --------------------------------------------------------------------------
# step 3: gate and pairwise transition scores
# --------------------------------------------------------------------------

def gate(hidden_row_f64: np.ndarray, w: Optional[np.ndarray]) -> float:
    """g = sigmoid(w . h) for a gated (DFlash v2) head, 1 for an ungated one."""
    if w is None:
        return 1.0
    x = float(np.dot(np.asarray(w, dtype=np.float64), np.asarray(hidden_row_f64, np.float64)))
    return 1.0 / (1.0 + np.exp(-x))


def pairwise(tables: np.ndarray, prev_tok: np.ndarray, cand_tok: np.ndarray, g: float) -> np.ndarray:
    """pi[j, k] = g * sum_i A[prev_tok[j], i] * B[cand_tok[k], i]   (float64).

    tables[0] is A (indexed by the previous token), tables[1] is B (indexed
    by the candidate token).
    """
    A = np.asarray(tables[0][np.asarray(prev_tok, np.int64)], dtype=np.float64)
    B = np.asarray(tables[1][np.asarray(cand_tok, np.int64)], dtype=np.float64)
    return g * (A @ B.T)


def lattice_scores(tok: np.ndarray, tables: np.ndarray, hidden_f64: np.ndarray,
                   gate_w: Optional[np.ndarray], last_tok: int) -> List[np.ndarray]:
    """Transition matrices of one request's block of L rows.

    S[0] has shape [1, K] (from the last accepted token); S[p] for p >= 1 has
    shape [K, K], S[p][j, k] = pi_p(t_{p-1}[j], k).
    """
    L = tok.shape[0]
    S = []
    for p in range(L):
        g = gate(hidden_f64[p], gate_w)
        prev = np.array([last_tok], np.int64) if p == 0 else tok[p - 1]
        S.append(pairwise(tables, prev, tok[p], g))
    return S


# --------------------------------------------------------------------------
# step 4: the walk
# --------------------------------------------------------------------------

def path_score(u: np.ndarray, S: Sequence[np.ndarray], path: Sequence[int]) -> float:
    """Score(c) = sum_p u_p[c_p] + S_p[c_{p-1}, c_p]   (c_{-1} is row 0 of S[0])."""
    total = 0.0
    prev = 0
    for p, c in enumerate(path):
        total += u[p][c] + S[p][prev, c]
        prev = c
    return float(total)


def _lowest_argmax(x: np.ndarray) -> int:
    return int(np.flatnonzero(x == x.max())[0])


def viterbi(u: np.ndarray, S: Sequence[np.ndarray]):
    """Max-score path through the lattice, with its score and runner-up margin.

    delta_0(k) = u_0[k] + S_0[0, k]
    delta_p(k) = u_p[k] + max_j (delta_{p-1}(j) + S_p[j, k]),  back-pointer = lowest such j
    last slot  = lowest k of max delta_{L-1}; then follow the back-pointers.

    The margin is (best path score) - (second best path score) over distinct
    slot paths, from a two-best list Viterbi (textbook list decoding): every
    state keeps its two best incoming path scores.  +inf when only one path
    exists.
    """
    u = np.asarray(u, dtype=np.float64)
    L, K = u.shape
    if L == 0:
        return np.zeros(0, np.int64), 0.0, np.inf
    d1 = u[0] + S[0][0]
    d2 = np.full(K, -np.inf)
    back = np.zeros((L, K), np.int64)
    for p in range(1, L):
        cand1 = d1[:, None] + S[p]          # [j, k]: best path into j, then j -> k
        cand2 = d2[:, None] + S[p]          # second best path into j, then j -> k
        back[p] = np.argmax(cand1, axis=0)  # numpy returns the first (lowest) j at ties
        best = cand1[back[p], np.arange(K)]
        # second best over all 2K incoming paths = max of (cand1 without its argmax entry, cand2)
        c1 = cand1.copy()
        c1[back[p], np.arange(K)] = -np.inf
        second = np.maximum(c1.max(axis=0), cand2.max(axis=0))
        d1, d2 = u[p] + best, u[p] + second
    last = _lowest_argmax(d1)
    path = np.zeros(L, np.int64)
    path[L - 1] = last
    for p in range(L - 1, 0, -1):
        path[p - 1] = back[p][path[p]]
    pool = np.concatenate([d1, d2])
    order = np.sort(pool)[::-1]
    margin = float(order[0] - order[1]) if order.size > 1 and np.isfinite(order[1]) else np.inf
    return path, float(d1[last]), margin


def greedy(u: np.ndarray, S: Sequence[np.ndarray]):
    """Greedy walk: c_p = lowest argmax_k u_p[k] + S_p[c_{p-1}, k].

    Returns the path, its score and the smallest gap, over positions, between
    the best and the second-best choice (+inf when K = 1).
    """
    u = np.asarray(u, dtype=np.float64)
    L, K = u.shape
    path = np.zeros(L, np.int64)
    prev, total, gap = 0, 0.0, np.inf
    for p in range(L):
        v = u[p] + S[p][prev]
        c = _lowest_argmax(v)
        if K > 1:
            srt = np.sort(v)[::-1]
            gap = min(gap, float(srt[0] - srt[1]))
        path[p], total, prev = c, total + v[c], c
    return path, float(total), gap


def bruteforce(u: np.ndarray, S: Sequence[np.ndarray]):
    """Enumerate all K^L slot paths (tiny inputs only).

    Every path's score is summed position by position as in path_score.
    Among the paths of maximal score, return the one whose reversed slot
    sequence (c_{L-1}, ..., c_0) is lexicographically smallest; that is the
    path the Viterbi back-tracking rule selects.  Returns (path, score,
    margin to the best path with a different slot sequence).
    """
    u = np.asarray(u, dtype=np.float64)
    L, K = u.shape
    paths = np.array(list(itertools.product(range(K), repeat=L)), dtype=np.int64).reshape(-1, L)
    scores = u[0][paths[:, 0]] + S[0][0, paths[:, 0]]
    for p in range(1, L):
        scores = scores + (u[p][paths[:, p]] + S[p][paths[:, p - 1], paths[:, p]])
    ties = np.flatnonzero(scores == scores.max())
    # np.lexsort sorts by its last key first: keys (c_0, ..., c_{L-1}) order by c_{L-1}, then c_{L-2}, ...
    pick = ties[np.lexsort(paths[ties].T)[0]]
    srt = np.sort(scores)[::-1]
    margin = float(srt[0] - srt[1]) if srt.size > 1 else np.inf
    return paths[pick].copy(), float(scores[pick]), margin


@dataclass
class SampledWalk:
    path: np.ndarray      # int64 [L] drawn slots
    q: np.ndarray         # float64 [L, K] the distribution each slot was drawn from
    score: float          # Score(c) of the drawn path (no temperature)
    gaps: np.ndarray      # float64 [L] distance of U * total to the nearest slot boundary, / total


def sampled(u: np.ndarray, S: Sequence[np.ndarray], uniforms: np.ndarray, temperature: float = 1.0) -> SampledWalk:
    """Sampled walk of one request through its lattice.

    [G] commit "DFlash-2 Markov head / BlockRowSource": a sampled request walks
    the lattice with the request's draft RNG, drawing every position from the
    lattice row after the token drawn before; the sampled-drafting commits of
    [G] fix the arithmetic of a draw: the weights come from a float exp, their
    running and total sums are doubles, the uniform is a double, and the
    proposal q is recorded normalized in double for the target's rejection
    sampling.  The random numbers are inputs (one double uniform in [0, 1)
    per position), so the walk is a function of them.

    At position p (c_{-1} selects row 0 of S_0):
      x_k   = fp32(fp32(u_p[k] + S_p[c_{p-1}, k]) / T)    the row drawn from, in fp32
      w_k   = fp32(exp(x_k - max_j x_j))                   float exp, correctly rounded
      W_k   = w_0 + ... + w_k in double, in slot order;   total = W_{K-1}
      c_p   = the smallest k with U_p * total < W_k
      q_p   = w / total (double)
    """
    u32 = np.asarray(u, dtype=np.float32)
    L, K = u32.shape
    T = np.float32(temperature)
    path = np.zeros(L, np.int64)
    q = np.zeros((L, K))
    gaps = np.zeros(L)
    prev = 0
    for p in range(L):
        row = np.asarray(S[p], dtype=np.float32)[prev]
        x = (u32[p] + row) / T                                   # float32 arithmetic
        w = np.exp((x - x.max()).astype(np.float64)).astype(np.float32)
        total = 0.0
        for k in range(K):
            total += float(w[k])
        thr = float(uniforms[p]) * total
        c, run = K - 1, 0.0
        bounds = []
        for k in range(K):
            run += float(w[k])
            bounds.append(run)
            if thr < run:
                c = k
                break
        # distance to the nearest running sum the draw compared with, relative to the total.
        # 0 and the last running sum (the total itself) are no boundaries: U * total < total
        # for every U < 1, and U = 0 draws slot 0, however the weights round
        b = np.array(bounds[:K - 1])
        gaps[p] = float(np.min(np.abs(b - thr))) / total if b.size else np.inf
        q[p] = w.astype(np.float64) / total
        path[p] = c
        prev = c
    return SampledWalk(path, q, path_score(u, S, path), gaps)


# --------------------------------------------------------------------------
# the whole draft step
# --------------------------------------------------------------------------

WALK_VITERBI, WALK_GREEDY, WALK_SAMPLED = 0, 1, 2


@dataclass
class DraftResult:
    tokens: np.ndarray        # int64 [M] drafted target ids
    scores: np.ndarray        # float64 [R] path scores
    slots: np.ndarray         # int64 [M] chosen slot per row
    margins: np.ndarray       # float64 [R] runner-up margin (Viterbi), smallest step gap (greedy),
                              # smallest relative draw gap (sampled)
    cand: Candidates
    S: List[List[np.ndarray]]  # per request, per position
    q: Optional[np.ndarray] = None   # float64 [M, K] proposals of a sampled walk


def _offsets(R: int, M: int, row_offsets) -> np.ndarray:
    """Row range of every request: uniform blocks of M / R rows, or row_offsets [R+1]."""
    if row_offsets is not None:
        return np.asarray(row_offsets, dtype=np.int64)
    if R == 0:
        return np.zeros(1, np.int64)
    assert M % R == 0, "uniform blocks need M = R * L"
    return np.arange(R + 1, dtype=np.int64) * (M // R)


def walk_from_candidates(cand: Candidates, tables, hidden_bits, gate_w, last_tok,
                         row_offsets=None, walk=WALK_VITERBI, uniforms=None,
                         temperature: float = 1.0) -> DraftResult:
    """Pairwise scores and the walk for every request, given the slots.

    A sampled walk takes one uniform per row (uniforms [M])."""
    R = len(last_tok)
    M = cand.idx.shape[0]
    off = _offsets(R, M, row_offsets)
    h = bf16_to_f64(hidden_bits) if hidden_bits is not None else None
    tokens = np.zeros(M, np.int64)
    slots = np.zeros(M, np.int64)
    scores = np.zeros(R)
    margins = np.full(R, np.inf)
    qs = np.zeros(cand.idx.shape) if walk == WALK_SAMPLED else None
    S_all = []
    for r in range(R):
        a, b = int(off[r]), int(off[r + 1])
        if b <= a:
            S_all.append([])
            continue
        hr = h[a:b] if h is not None else np.zeros((b - a, 1))
        S = lattice_scores(cand.tok[a:b], tables, hr, gate_w, int(last_tok[r]))
        if walk == WALK_VITERBI:
            path, score, margin = viterbi(cand.unary[a:b], S)
        elif walk == WALK_SAMPLED:
            sw = sampled(cand.unary[a:b], S, np.asarray(uniforms)[a:b], temperature)
            path, score, margin = sw.path, sw.score, float(np.min(sw.gaps))
            qs[a:b] = sw.q
        else:
            path, score, margin = greedy(cand.unary[a:b], S)
        slots[a:b] = path
        tokens[a:b] = cand.tok[a:b][np.arange(b - a), path]
        scores[r], margins[r] = score, margin
        S_all.append(S)
    return DraftResult(tokens, scores, slots, margins, cand, S_all, qs)


def draft_from_logits(z: np.ndarray, K: int, d2t, tables, hidden_bits, gate_w, last_tok,
                      row_offsets=None, walk=WALK_VITERBI, uniforms=None,
                      temperature: float = 1.0) -> DraftResult:
    """Steps 2-4 from given logits (used to feed the GPU and the oracle the same logits)."""
    cand = candidates(z, K, d2t)
    return walk_from_candidates(cand, tables, hidden_bits, gate_w, last_tok, row_offsets,
                                walk=walk, uniforms=uniforms, temperature=temperature)


def draft_block(hidden_bits, lm_head_bits, d2t, tables, gate_w, last_tok, K,
                row_offsets=None, walk=WALK_VITERBI, uniforms=None,
                temperature: float = 1.0) -> DraftResult:
    """The whole draft step: hidden states of the packed block rows -> drafted tokens."""
    z = logits(hidden_bits, lm_head_bits)
    return draft_from_logits(z, K, d2t, tables, hidden_bits, gate_w, last_tok, row_offsets, walk,
                             uniforms, temperature)


# --------------------------------------------------------------------------
# without a Markov head: the scaled, soft-capped rows and their argmax
# --------------------------------------------------------------------------

def scale_cap(z: np.ndarray, scale: float, cap: float) -> np.ndarray:
    """The backbone rows as a draft without a Markov head uses them.

    [G] commit "DFlash-2 Markov head / BlockRowSource": without a head the
    selector scales and soft caps the backbone rows (the Markov head's rows
    differ from them by the output multiplier and the soft cap).  The pages
    give no formula; reading: the multiplier first, then the usual tanh cap,
        z' = cap * tanh(scale * z / cap)   when cap > 0,
        z' = scale * z                     otherwise (no cap),
    with a positive multiplier.
    """
    assert scale > 0, "the output multiplier must be positive"
    x = float(scale) * np.asarray(z, np.float64)
    if cap > 0:
        return float(cap) * np.tanh(x / float(cap))
    return x


def argmax_rows(z: np.ndarray, scale: float, cap: float, d2t: Optional[np.ndarray]):
    """Greedy head-less drafting: per row the best token of the scaled, capped row.

    [G] same commit: a greedy request whose logit processors keep the argmax
    takes the best token of every row.  Ties go to the lowest draft id (the
    index order of the TopP commit).  Returns (draft ids [M], target ids [M],
    the winning z' [M]).
    """
    zs = scale_cap(z, scale, cap)
    ids = np.array([_lowest_argmax(row) for row in zs], dtype=np.int64)
    tok = draft_to_target(ids, d2t)
    vals = zs[np.arange(zs.shape[0]), ids] if zs.shape[0] else np.zeros(0)
    return ids, tok, vals


def draft_argmax(hidden_bits, lm_head_bits, d2t, scale: float, cap: float):
    """The whole head-less draft step: hidden states -> logits -> scaled, capped argmax."""
    return argmax_rows(logits(hidden_bits, lm_head_bits), scale, cap, d2t)


# --------------------------------------------------------------------------
# the dense Markov walk: one biased argmax per position
# --------------------------------------------------------------------------

@dataclass
class DenseResult:
    ids: np.ndarray       # int64 [M] chosen draft ids
    tokens: np.ndarray    # int64 [M] chosen target ids
    values: np.ndarray    # float64 [M] the winning biased value
    margins: np.ndarray   # float64 [M] gap between the best and the second best value of the row


def dense_row(z_row: np.ndarray, scale: float, cap: float, d2t, tables: np.ndarray, prev_tok: int):
    """The biased row of one position and its lowest-id argmax.

    [G] commit "DFlash-2 Markov head / BlockRowSource": a dense Markov step is
    run per position and biases the scaled rows by the token drafted before;
    a greedy request takes the best biased token.  [G] Description: the dense
    walk (markov_head_top_k = 0, DSpark only: no gate) corrects every drafted
    position.  Reading: the bias of draft id v after token s is the pairwise
    term of the Top-K lattice, <A[s], B[t(v)]> with t(v) = v + d2t[v], added to
    the scaled, soft-capped row.
    """
    Vd = z_row.shape[0]
    t_all = draft_to_target(np.arange(Vd), d2t)
    A = np.asarray(tables[0], np.float64)[int(prev_tok)]
    B = np.asarray(tables[1], np.float64)[t_all]           # [V_d, r]
    row = scale_cap(z_row, scale, cap) + B @ A
    c = _lowest_argmax(row)
    second = np.max(np.delete(row, c)) if Vd > 1 else -np.inf
    return c, row[c], row[c] - second


def dense_walk(z: np.ndarray, scale: float, cap: float, d2t, tables, last_tok, row_offsets=None,
               prev_override: Optional[np.ndarray] = None) -> DenseResult:
    """The dense walk of every request: s_0 = last accepted token, s_{p+1} = t(c_p).

    prev_override [M] (optional) gives the previous token of every row instead
    of the walk's own choice (to re-check another walk's decisions one by one).
    """
    R = len(last_tok)
    M = z.shape[0]
    off = _offsets(R, M, row_offsets)
    ids = np.zeros(M, np.int64)
    vals = np.zeros(M)
    margins = np.full(M, np.inf)
    for r in range(R):
        a, b = int(off[r]), int(off[r + 1])
        s = int(last_tok[r])
        for m in range(a, b):
            if prev_override is not None:
                s = int(prev_override[m])
            c, v, g = dense_row(z[m], scale, cap, d2t, tables, s)
            ids[m], vals[m], margins[m] = c, v, g
            s = int(draft_to_target(np.array([c]), d2t)[0])
    return DenseResult(ids, draft_to_target(ids, d2t), vals, margins)


def draft_dense(hidden_bits, lm_head_bits, d2t, tables, last_tok, scale: float, cap: float,
                row_offsets=None) -> DenseResult:
    """The whole dense-walk draft step."""
    return dense_walk(logits(hidden_bits, lm_head_bits), scale, cap, d2t, tables, last_tok, row_offsets)


def check_d2t(d2t: np.ndarray, Vd: int, Vt: int):
    """(valid, injective): every i + d2t[i] lies in [0, V_t), and no two draft ids share a target.

    Greedy drafting accepts any mapping; only sampled drafting needs an
    injective one (d2t commit of [G]).
    """
    d2t = np.asarray(d2t, np.int64)
    if d2t.shape != (Vd,):
        return False, False
    t = np.arange(Vd, dtype=np.int64) + d2t
    valid = bool(np.all((t >= 0) & (t < Vt)))
    injective = valid and np.unique(t).size == Vd
    return valid, injective
