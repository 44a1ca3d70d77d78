"""GPU parity of the HIP draft step against the CPU oracle, through the C ABI.

Bars (from the draft-step spec):
  * logits: |z_gpu - z_oracle| <= 1e-3 * max|z_oracle| of the row;
  * Top-K: the slots are bit-exact when fed the oracle's logits (the same
    fp32 values on both sides); from the GPU's own logits they are bit-exact
    unless the oracle's K-th and (K+1)-th logits differ by less than the
    logit tolerance (then the set rule of gpu_util.check_topk_row applies);
  * walk: tokens and slots bit-exact when fed the oracle's unary and pairwise
    values (rounded to fp32, the oracle re-walking those fp32 values in
    fp64); a case whose oracle runner-up margin is below 1e-6 * max(|S|, 1)
    is listed as an exemption; path scores within 1e-4 * max(|S|, 1);
  * the whole step (GPU logits): tokens bit-exact and scores within 1e-4
    for every request none of whose rows uses the Top-K boundary exemption
    (a GPU candidate set that differs from the oracle's) and whose oracle
    runner-up margin is at least 1e-5 * max(|S|, 1); an exempt request's
    path must score within 1e-4 of the best path over the GPU's own
    candidates (oracle, fp64).  Full-size workloads check every request and
    allow at most a tenth of them to be exempt;
  * integer outputs (ids, target ids, slots) are compared exactly.
"""
import numpy as np
import pytest
import torch

import draft_inputs as di
from oracle import draft_step as O
from tests.gpu_util import (check_topk_row, dev, dev_bf16, logits_tol, offsets_of, pack_pair, record, require_gpu, say,
                            upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    from block_draft_markov_amd import api
    return api


def api():
    from block_draft_markov_amd import api as a
    return a


def f32(x):
    return np.asarray(x, dtype=np.float32)


# ============================================================ part 1: lm_head

LMHEAD_CASES = [
    # (name, M, H, V)          what it covers
    ("tiny", 5, 64, 1024),                    # the tiny workload
    ("ragged", 37, 136, 2051),                # M tail in a 16-row tile, H % 64 != 0, V % 16 and V % 4 != 0
    ("two_row_chunks", 300, 128, 5000),       # more than 256 rows: two row chunks
    ("one_row", 1, 64, 17),                   # a single row and a single partial tile
    ("rows_224", 224, 256, 20000),            # the 224-row tile of the 4B batch
    ("rows_240", 240, 512, 33333),            # the 240-row tile of the 27B / pruned batches
    ("rows_100_h200", 100, 200, 3001),        # batched rows, H not a multiple of 64 (column clamps)
    ("rows_65_h8", 65, 8, 257),               # smallest batched case: one partial step, one tile tail
    ("rows_480", 480, 192, 4133),             # two full 240-row chunks
]


@pytest.mark.parametrize("name,M,H,V", LMHEAD_CASES)
def test_lm_head_parity(name, M, H, V):
    say(f"lm_head {name}: M={M} H={H} V={V}")
    sh = di.custom_shape(name, R=M, L=1, H=H, Vd=V, K=min(64, V), r=4, seed=11 + M)
    inp = di.make_inputs(sh)
    z_gpu, lse_gpu = api().lm_head(dev_bf16(inp.hidden), dev_bf16(inp.lm_head))
    torch.cuda.synchronize()
    z_gpu = z_gpu.cpu().numpy().astype(np.float64)
    lse_gpu = lse_gpu.cpu().numpy().astype(np.float64)
    z = O.logits(inp.hidden, inp.lm_head)
    lse = O.row_lse(z)
    worst = 0.0
    for m in range(M):
        tol = logits_tol(z[m])
        err = np.max(np.abs(z_gpu[m] - z[m]))
        assert err <= tol, f"row {m}: max error {err} > {tol}"
        worst = max(worst, err / max(np.max(np.abs(z[m])), 1e-30))
        assert abs(lse_gpu[m] - lse[m]) <= tol
    say(f"  max relative logit error {worst:.3e}")
    assert worst < 1e-5   # fp32 accumulation of exact bf16 products: far inside the bar


def test_lm_head_full_qwen3_4b_single_request():
    """All 7 rows of the Qwen3-4B-shaped block at full vocabulary and hidden size."""
    inp = di.make_inputs(di.SHAPES["qwen3_4b_1"])
    say("lm_head qwen3_4b_1 full")
    z_gpu, lse_gpu = api().lm_head(dev_bf16(inp.hidden), dev_bf16(inp.lm_head))
    z_gpu = z_gpu.cpu().numpy().astype(np.float64)
    lse_gpu = lse_gpu.cpu().numpy()
    z = O.logits(inp.hidden, inp.lm_head)
    lse = O.row_lse(z)
    for m in range(inp.M):
        tol = logits_tol(z[m])
        assert np.max(np.abs(z_gpu[m] - z[m])) <= tol
        assert abs(lse_gpu[m] - lse[m]) <= tol


def test_row_lse_matches_oracle():
    rng = np.random.default_rng(4)
    z = (rng.standard_normal((9, 3001)) * 3).astype(np.float32)
    zt = torch.zeros((9, 3004), dtype=torch.float32, device="cuda")
    zt[:, :3001] = dev(z)
    lse = api().row_lse(zt[:, :3001]).cpu().numpy()
    ref = O.row_lse(z.astype(np.float64))
    assert np.max(np.abs(lse - ref)) <= 1e-5 * np.max(np.abs(ref))


# ============================================================ part 2: Top-K

def _topk_feed(z32: np.ndarray, K: int, d2t=None, Vt=None):
    """Run dflash_topk on fp32 logits (with the fp64 LSE of those values rounded to fp32)."""
    M, V = z32.shape
    ldz = V + (-V) % 4
    # the row padding past V holds values above every logit: they must never be read as logits
    zt = torch.full((M, ldz), 1e30, dtype=torch.float32, device="cuda")
    zt[:, :V] = dev(z32)
    lse = O.row_lse(z32.astype(np.float64))
    idx, tok, un = api().topk(zt[:, :V], dev(f32(lse)), K, d2t=dev(d2t), target_vocab=Vt)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), tok.cpu().numpy(), un.cpu().numpy(), f32(lse)


def _check_topk_exact(z32, K, d2t=None, Vt=None):
    idx, tok, un, lse32 = _topk_feed(z32, K, d2t, Vt)
    z64 = z32.astype(np.float64)
    cand = O.candidates(z64, K, d2t)
    assert np.array_equal(idx, cand.idx), "slots differ from the oracle's full sort"
    assert np.array_equal(tok, cand.tok), "target ids differ"
    want = np.take_along_axis(z32, cand.idx, 1).astype(np.float64) - lse32[:, None].astype(np.float64)
    assert np.max(np.abs(un - want)) <= 1e-6 * max(1.0, np.max(np.abs(want)))


TOPK_CASES = [
    # (name, M, V, K, kind)
    ("tiny", 5, 1024, 8, "normal"),
    ("k64", 7, 20000, 64, "normal"),
    ("k1", 4, 5000, 1, "normal"),
    ("v_eq_k", 3, 48, 48, "normal"),         # K = V_d: the 48-token draft vocabulary
    ("v_lt_chunk", 3, 300, 64, "normal"),    # a single short chunk
    ("v1", 3, 1, 1, "normal"),               # a one-token vocabulary: one partial tile of one logit
    ("v17", 2, 17, 17, "normal"),            # K = V_d inside one partial tile; V % 4 != 0
    ("ragged_v", 6, 70001, 64, "normal"),    # V % 4 != 0, last chunk partial
    ("ties_small_ints", 5, 9000, 64, "ints"),     # many exact ties: the radix fallback
    ("all_equal", 3, 5000, 64, "equal"),          # every logit equal: slots 0..K-1
    ("signed_zeros", 2, 4096, 64, "zeros"),       # -0.0 and +0.0 tie; the lower id wins
    ("qwen3_4b_rows", 4, 151936, 64, "normal"),
    ("dflash2_27b_rows", 3, 248100, 64, "normal"),
    ("many_rows", 224, 151936, 64, "normal"),     # the row count of the 4B batch: the large-chunk plan
    ("long_row", 2, 300000, 64, "normal"),        # 9375 tiles: more than the 8192 tile maxima kept in registers
    ("long_row_ties", 2, 300000, 64, "ints"),     # the same length with heavy ties: the exact path
    # many rows with ties, zeros, equal logits and short or long rows
    ("rows128_ties", 130, 9000, 64, "ints"),
    ("rows128_ragged_v", 128, 70001, 64, "normal"),
    ("rows128_zeros", 128, 4096, 64, "zeros"),
    ("rows128_equal", 128, 5000, 64, "equal"),
    ("rows128_v17", 160, 17, 17, "normal"),
    ("rows128_v1", 128, 1, 1, "normal"),
    ("rows128_8192_tiles", 128, 262144, 64, "ints"),   # the most tiles the LDS maxima hold
]


def _make_logits(M, V, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return f32(rng.standard_normal((M, V)))
    if kind == "ints":
        return f32(rng.integers(-3, 4, size=(M, V)))
    if kind == "equal":
        return np.full((M, V), 0.25, np.float32)
    if kind == "zeros":
        z = np.where(rng.random((M, V)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        z[:, ::7] = -1.0
        return z
    raise ValueError(kind)


@pytest.mark.parametrize("name,M,V,K,kind", TOPK_CASES)
def test_topk_fed_oracle_logits_bit_exact(name, M, V, K, kind):
    say(f"topk {name}: M={M} V={V} K={K} {kind}")
    z32 = _make_logits(M, V, kind, seed=sum(name.encode()))
    _check_topk_exact(z32, K)


def test_topk_pruned_d2t_remap():
    Vd, Vt = 114688, 248100
    sub = np.random.default_rng(5).permutation(Vt)[:Vd]
    d2t = (sub - np.arange(Vd)).astype(np.int64)
    z32 = _make_logits(5, Vd, "normal", 3)
    _check_topk_exact(z32, 64, d2t, Vt)


def test_topk_pruned_d2t_remap_many_rows():
    Vd, Vt = 114688, 248100
    sub = np.random.default_rng(6).permutation(Vt)[:Vd]
    d2t = (sub - np.arange(Vd)).astype(np.int64)
    z32 = _make_logits(130, Vd, "normal", 4)
    _check_topk_exact(z32, 64, d2t, Vt)


def test_topk_48_token_subset():
    sub = np.random.default_rng(9).permutation(200)[:48]
    d2t = (sub - np.arange(48)).astype(np.int64)
    _check_topk_exact(_make_logits(4, 48, "normal", 1), 48, d2t, 200)


# ============================================================ part 3: pair scores

PAIR_CASES = [
    # (name, R, L, K, r, gated, ragged)
    ("tiny", 1, 5, 8, 16, False, None),
    ("k64_r256", 3, 7, 64, 256, False, None),
    ("gated", 2, 15, 64, 256, True, None),
    ("k5_r100", 3, 4, 5, 100, True, None),     # K % 4 != 0, rank not a multiple of the 64-wide slice
    ("ragged", 4, 6, 16, 32, False, [3, 0, 6, 1]),
    ("r30_elementwise", 2, 5, 64, 30, True, None),   # rank not a multiple of 4: the element-wise gather
    ("r260_two_slices", 2, 4, 64, 260, False, None),  # a full 256-element slice, then 4 elements
    ("r520_three_slices", 1, 3, 33, 520, True, None),
]


@pytest.mark.parametrize("name,R,L,K,r,gated,ragged", PAIR_CASES)
def test_pair_scores_parity(name, R, L, K, r, gated, ragged):
    say(f"pair {name}")
    rng = np.random.default_rng(R * 100 + K)
    Vt, H = 3000, 64
    lengths = ragged if ragged is not None else [L] * R
    off = di.ragged_offsets(lengths)
    M = int(off[-1])
    tok = rng.integers(0, Vt, size=(M, K)).astype(np.int64)
    tables = f32(rng.standard_normal((2, Vt, r)) * 0.25)
    hidden = di.round_to_bf16_bits(f32(rng.standard_normal((M, H))))
    w = f32(rng.standard_normal(H) / 8) if gated else None
    last = rng.integers(0, Vt, size=R).astype(np.int64)
    pair = api().pair_scores(dev(tok), dev(tables), dev(last), gate_w=dev(w), hidden=dev_bf16(hidden),
                             row_offsets=dev(off) if ragged is not None else None, block_len=max(lengths))
    pair = pair.cpu().numpy().astype(np.float64)
    h64 = O.bf16_to_f64(hidden)
    for req in range(R):
        a = int(off[req])
        S = O.lattice_scores(tok[a:off[req + 1]], tables, h64[a:off[req + 1]], w, int(last[req]))
        for p, s in enumerate(S):
            got = pair[a + p, :1, :] if p == 0 else pair[a + p]
            scale = max(1.0, float(np.max(np.abs(s))))
            assert np.max(np.abs(got - s)) <= 1e-5 * scale, f"request {req} position {p}"
            if p == 0:
                assert np.all(pair[a, 1:, :] == 0.0)


@pytest.mark.parametrize("H,aligned", [(8, False), (64, False), (5120, True), (9000, True)])
def test_pair_scores_gate_hidden_sizes(H, aligned):
    """The gate w . h_p: a gate vector that is not 16-byte aligned (element loop), one round
    of 16-byte loads (5120) and more than one (9000)."""
    say(f"pair gate H={H} aligned={aligned}")
    rng = np.random.default_rng(H)
    R, L, K, r, Vt = 2, 3, 16, 64, 500
    M = R * L
    off = di.ragged_offsets([L] * R)
    tok = rng.integers(0, Vt, size=(M, K)).astype(np.int64)
    tables = f32(rng.standard_normal((2, Vt, r)) * 0.25)
    hidden = di.round_to_bf16_bits(f32(rng.standard_normal((M, H))))
    w = f32(rng.standard_normal(H) / np.sqrt(H))
    last = rng.integers(0, Vt, size=R).astype(np.int64)
    wd = dev(w) if aligned else dev(np.concatenate([np.zeros(1, np.float32), w]))[1:]   # 4 bytes past 16
    assert (wd.data_ptr() % 16 == 0) == aligned
    pair = api().pair_scores(dev(tok), dev(tables), dev(last), gate_w=wd, hidden=dev_bf16(hidden), block_len=L)
    pair = pair.cpu().numpy().astype(np.float64)
    h64 = O.bf16_to_f64(hidden)
    for req in range(R):
        a = int(off[req])
        S = O.lattice_scores(tok[a:a + L], tables, h64[a:a + L], w, int(last[req]))
        for p, s in enumerate(S):
            got = pair[a + p, :1, :] if p == 0 else pair[a + p]
            scale = max(1.0, float(np.max(np.abs(s))))
            assert np.max(np.abs(got - s)) <= 1e-5 * scale, f"request {req} position {p}"


# ============================================================ part 4: walk

def _walk_fed(u64, S_all, off, R, K, walk, L):
    """GPU walk fed the oracle's unary and pairwise values rounded to fp32."""
    M = u64.shape[0]
    u32 = f32(u64)
    pair32 = f32(pack_pair(S_all, off, M, K))
    tok = np.arange(M * K, dtype=np.int64).reshape(M, K) * 7 + 3    # distinct ids: token = f(row, slot)
    tokens, scores, slots = api().walk(dev(tok), dev(u32), dev(pair32), R, row_offsets=dev(off.astype(np.int32)),
                                       block_len=L, walk=walk)
    return tok, u32, pair32, tokens.cpu().numpy(), scores.cpu().numpy(), slots.cpu().numpy()


def _oracle_walk32(u32, pair32, off, R, walk):
    res = []
    for req in range(R):
        a, b = int(off[req]), int(off[req + 1])
        if b == a:
            res.append((np.zeros(0, np.int64), 0.0, np.inf))
            continue
        u = u32[a:b].astype(np.float64)
        S = [pair32[a, :1, :].astype(np.float64)] + [pair32[a + p].astype(np.float64) for p in range(1, b - a)]
        res.append(O.viterbi(u, S) if walk == "viterbi" else O.greedy(u, S))
    return res


def _check_walk(u64, S_all, off, R, K, L, walk):
    tok, u32, pair32, tokens, scores, slots = _walk_fed(u64, S_all, off, R, K, walk, L)
    exempt = 0
    for req, (path, score, margin) in enumerate(_oracle_walk32(u32, pair32, off, R, walk)):
        a, b = int(off[req]), int(off[req + 1])
        scale = max(1.0, abs(score))
        assert abs(scores[req] - score) <= 1e-4 * scale, f"request {req}: score {scores[req]} vs {score}"
        if b == a:
            continue
        if margin < 1e-6 * scale:
            exempt += 1
            continue
        assert list(slots[a:b]) == list(path), f"request {req}: slots differ"
        assert np.array_equal(tokens[a:b], tok[np.arange(a, b), path])
    return exempt


def _random_lattice(R, lengths, K, seed, scale_pair=1.0, ints=False):
    rng = np.random.default_rng(seed)
    M = sum(lengths)
    if ints:
        u = rng.integers(-3, 1, size=(M, K)).astype(np.float64)
    else:
        u = -np.sort(-rng.standard_normal((M, K)), axis=1) - 5.0
    S_all, a = [], 0
    for Lr in lengths:
        S = []
        for p in range(Lr):
            shape = (1, K) if p == 0 else (K, K)
            S.append(rng.integers(-2, 3, size=shape).astype(np.float64) if ints
                     else rng.standard_normal(shape) * scale_pair)
        S_all.append(S)
        a += Lr
    return u, S_all, di.ragged_offsets(lengths).astype(np.int64)


WALK_CASES = [
    # (name, lengths, K, kind)
    ("tiny", [5], 8, "normal"),
    ("batch_l7_k64", [7] * 32, 64, "normal"),
    ("batch_l15_k64", [15] * 16, 64, "normal"),
    ("l1", [1, 1, 1], 64, "normal"),
    ("k1", [6, 4], 1, "normal"),
    ("l100", [100, 37], 64, "normal"),          # the maximum block length
    ("ragged_with_empty", [3, 0, 9, 1, 0], 16, "normal"),
    ("exact_ties", [6] * 20, 4, "ints"),         # small integers: exact ties in fp32 and fp64
    ("exact_ties_k64", [7] * 8, 64, "ints"),
    # Viterbi blocks of up to 8 and up to 16 positions keep S in registers, longer ones stage it in LDS
    ("l8_k33", [8, 2, 8, 5], 33, "normal"),
    ("l8_and_l9", [8, 9, 8, 9], 64, "normal"),
    ("l16_and_l17", [16, 17, 3, 16], 64, "normal"),
    ("l16_k20", [16, 11, 16], 20, "normal"),
]


@pytest.mark.parametrize("walk", ["viterbi", "greedy"])
@pytest.mark.parametrize("name,lengths,K,kind", WALK_CASES)
def test_walk_fed_oracle_values_bit_exact(name, lengths, K, kind, walk):
    say(f"walk {name} {walk}")
    R = len(lengths)
    u, S_all, off = _random_lattice(R, lengths, K, seed=len(name) * 31 + K, ints=(kind == "ints"))
    exempt = _check_walk(u, S_all, off, R, K, max(max(lengths), 1), walk)
    say(f"  exemptions: {exempt}")
    assert exempt == 0 or kind == "ints"   # exact ties are compared bit for bit; margins 0 only there


# ============================================================ the whole step

def _staged(api_, d, inp, K, L, walk):
    z, lse = api_.lm_head(d["hidden"], d["lm_head"])
    idx, tok, un = api_.topk(z, lse, K, d2t=d["d2t"], target_vocab=inp.tables.shape[1])
    pair = api_.pair_scores(tok, d["tables"], d["last_tok"], gate_w=d["gate_w"], hidden=d["hidden"],
                            row_offsets=d["row_offsets"], block_len=L)
    tokens, scores, slots = api_.walk(tok, un, pair, len(inp.last_tok), row_offsets=d["row_offsets"],
                                      block_len=L, walk=walk)
    return z, lse, idx, tok, un, tokens, scores, slots


def _end_to_end(inp, sample_requests, walk="viterbi", name=None):
    """The fused step against the oracle on the given requests.

    A request is compared bit for bit (tokens, and the path score within
    1e-4 * max(|S|, 1)) unless one of its rows uses the Top-K boundary
    exemption (the GPU's candidate set differs from the oracle's), or the
    oracle's runner-up margin is below 1e-5 * max(|S|, 1) (then an fp32 rounding
    may pick the other path).  Exempt requests are re-walked by the oracle in
    fp64 on the GPU's own candidates: the GPU path must score within 1e-4 of
    that set's best.  Returns the counts.
    """
    api_ = api()
    s = inp.shape
    R, M, K = len(inp.last_tok), inp.M, s.K
    off = offsets_of(R, M, inp.row_offsets)
    L = int(np.max(np.diff(off))) if R else 1
    d = upload(inp)
    tokens, scores = api_.draft_block(d["hidden"], d["lm_head"], d["tables"], d["last_tok"], top_k=K, d2t=d["d2t"],
                                      gate_w=d["gate_w"], row_offsets=d["row_offsets"], block_len=L, walk=walk)
    tokens2, scores2 = api_.draft_block(d["hidden"], d["lm_head"], d["tables"], d["last_tok"], top_k=K,
                                        d2t=d["d2t"], gate_w=d["gate_w"], row_offsets=d["row_offsets"],
                                        block_len=L, walk=walk)
    # the opt-in logits filter (DFLASH_OPT_FILTER_LOGITS): the same tokens and scores bit for bit
    f_tokens, f_scores = api_.draft_block(d["hidden"], d["lm_head"], d["tables"], d["last_tok"], top_k=K,
                                          d2t=d["d2t"], gate_w=d["gate_w"], row_offsets=d["row_offsets"],
                                          block_len=L, walk=walk, filter_logits=True)
    z, lse, idx, tok, un, st_tokens, st_scores, st_slots = _staged(api_, d, inp, K, L, walk)
    lat_tokens, lat_scores = api_.lattice(tok, un, d["tables"], d["last_tok"], gate_w=d["gate_w"],
                                          hidden=d["hidden"], row_offsets=d["row_offsets"], block_len=L, walk=walk)
    torch.cuda.synchronize()
    tokens, scores = tokens.cpu().numpy(), scores.cpu().numpy()
    # deterministic, and the fused call equals the staged calls bit for bit
    assert np.array_equal(tokens, tokens2.cpu().numpy()) and np.array_equal(scores, scores2.cpu().numpy())
    assert np.array_equal(tokens, st_tokens.cpu().numpy())
    assert np.array_equal(scores, st_scores.cpu().numpy())
    assert np.array_equal(tokens, lat_tokens.cpu().numpy()) and np.array_equal(scores, lat_scores.cpu().numpy())
    assert np.array_equal(tokens, f_tokens.cpu().numpy()) and np.array_equal(scores, f_scores.cpu().numpy()), \
        "the logits filter changed the step's result"
    idx = idx.cpu().numpy().astype(np.int64)
    gtok = tok.cpu().numpy()
    slots = st_slots.cpu().numpy()
    owalk = O.WALK_VITERBI if walk == "viterbi" else O.WALK_GREEDY
    counts = dict(requests=0, req_exact=0, req_topk_exempt=0, req_margin_exempt=0, rows=0, rows_same=0,
                  rows_reorder=0, rows_differs=0)
    reqs = [r for r in sample_requests if off[r + 1] > off[r]]
    for req in sample_requests:
        if off[req + 1] == off[req]:
            assert scores[req] == 0.0
    if not reqs:
        return counts
    # the oracle's fp64 logits of every row of the sampled requests, in one product
    rows_all = np.concatenate([np.arange(off[r], off[r + 1]) for r in reqs])
    zo_all = O.logits(inp.hidden[rows_all], inp.lm_head)
    zg_all = z.cpu().numpy()[rows_all].astype(np.float64)
    base = 0
    for req in reqs:
        a, b = int(off[req]), int(off[req + 1])
        n = b - a
        rows = np.arange(a, b)
        zo, zg = zo_all[base:base + n], zg_all[base:base + n]
        base += n
        counts["requests"] += 1
        kinds = []
        for i in range(n):
            assert np.max(np.abs(zg[i] - zo[i])) <= logits_tol(zo[i]), f"request {req} row {i}: logits"
            kinds.append(check_topk_row(idx[a + i], zo[i], K))
        counts["rows"] += n
        for k in ("same", "reorder", "differs"):
            counts["rows_" + k] += kinds.count(k)
        sub = O.draft_from_logits(zo, K, inp.d2t, inp.tables, inp.hidden[rows], inp.gate_w,
                                  inp.last_tok[req:req + 1], walk=owalk)
        score, margin = sub.scores[0], sub.margins[0]
        scale = max(1.0, abs(score))
        if "differs" not in kinds and margin >= 1e-5 * scale:
            assert np.array_equal(tokens[a:b], sub.tokens), f"request {req}: tokens {tokens[a:b]} vs {sub.tokens}"
            assert abs(scores[req] - score) <= 1e-4 * scale, f"request {req}: score {scores[req]} vs {score}"
            counts["req_exact"] += 1
            continue
        counts["req_topk_exempt" if "differs" in kinds else "req_margin_exempt"] += 1
        # the GPU's own candidate set, re-walked by the oracle in fp64: same best score within 1e-4
        lse_o = O.row_lse(zo)
        cand = O.Candidates(idx[a:b], gtok[a:b], np.take_along_axis(zo, idx[a:b], 1) - lse_o[:, None], None, lse_o,
                            None)
        alt = O.walk_from_candidates(cand, inp.tables, inp.hidden[rows], inp.gate_w, inp.last_tok[req:req + 1],
                                     walk=owalk)
        gpu_path_score = O.path_score(cand.unary, alt.S[0], slots[a:b])
        assert abs(gpu_path_score - alt.scores[0]) <= 1e-4 * max(1.0, abs(alt.scores[0]))
        assert abs(scores[req] - alt.scores[0]) <= 1e-4 * max(1.0, abs(alt.scores[0]))
    record(name or s.name, walk=walk, **counts)
    return counts


def _assert_mostly_exact(c):
    """Exemptions are rare (fp32 logits are ~1e-6 relative from the oracle's): at least one
    request compared bit for bit, and at most a tenth of them (or one) exempt."""
    assert c["req_exact"] >= 1, c
    assert c["req_topk_exempt"] + c["req_margin_exempt"] <= max(1, c["requests"] // 10), c


def test_end_to_end_tiny():
    c = _end_to_end(di.make_inputs(di.SHAPES["tiny"]), [0])
    assert c["req_exact"] == 1


@pytest.mark.parametrize("walk", ["viterbi", "greedy"])
def test_end_to_end_tiny_stress_seeds(walk):
    exact = 0
    for seed in range(2000, 2040):
        sh = di.custom_shape("tiny_stress", R=1, L=5, H=64, Vd=1024, K=8, r=16, table_std=0.5, seed=seed,
                             weight_seed=seed)
        c = _end_to_end(di.make_inputs(sh), [0], walk, name=f"tiny_stress_{seed}")
        exact += c["req_exact"]
        assert c["req_exact"] + c["req_topk_exempt"] + c["req_margin_exempt"] == 1
    say(f"  {exact} of 40 requests outside every exemption, all bit-exact")
    assert exact >= 36


def test_end_to_end_gated_tiny_and_ragged():
    sh = di.custom_shape("gated_tiny", R=4, L=6, H=64, Vd=2000, K=16, r=16, gated=True, table_std=0.5, seed=7)
    inp = di.make_inputs(sh)
    _end_to_end(inp, range(4))
    inp.row_offsets = di.ragged_offsets([6, 0, 2, 5])
    inp.hidden = inp.hidden[:13].copy()
    _end_to_end(inp, range(4))


@pytest.mark.parametrize("name,Vd,K", [("vocab_1", 1, 1), ("vocab_17", 17, 17), ("vocab_33_k8", 33, 8)])
def test_end_to_end_tiny_vocabularies(name, Vd, K):
    """Vocabularies of one partial tile or two: every kernel of the fused step at its edge."""
    say(f"end-to-end {name}: V={Vd} K={K}")
    sh = di.custom_shape(name, R=3, L=4, H=64, Vd=Vd, K=K, r=8, table_std=0.5, seed=80 + Vd)
    _end_to_end(di.make_inputs(sh), [0, 1, 2])


def test_end_to_end_pruned_small_48():
    sh = di.custom_shape("pruned48", R=2, L=4, H=64, Vd=48, Vt=200, K=48, r=8, pruned=True, table_std=0.5, seed=9)
    _end_to_end(di.make_inputs(sh), [0, 1])


def test_end_to_end_qwen3_4b_single_request():
    c = _end_to_end(di.make_inputs(di.SHAPES["qwen3_4b_1"]), [0])
    assert c["req_exact"] + c["req_topk_exempt"] + c["req_margin_exempt"] == 1


def test_end_to_end_qwen3_4b_batch_all_requests():
    c = _end_to_end(di.make_inputs(di.SHAPES["qwen3_4b_32"]), range(32))
    _assert_mostly_exact(c)


def test_end_to_end_qwen3_4b_batch_greedy_all_requests():
    c = _end_to_end(di.make_inputs(di.SHAPES["qwen3_4b_32"]), range(32), walk="greedy")
    _assert_mostly_exact(c)


def test_end_to_end_dflash2_27b_all_requests():
    c = _end_to_end(di.make_inputs(di.SHAPES["dflash2_27b"]), range(16))
    _assert_mostly_exact(c)


def test_end_to_end_pruned_ocr_all_requests():
    c = _end_to_end(di.make_inputs(di.SHAPES["pruned_ocr"]), range(16))
    _assert_mostly_exact(c)


def _zero_hidden(inp):
    inp.hidden[:] = 0    # bf16 +0: every logit is 0, the whole row ties
    return inp


@pytest.mark.parametrize("name,R,L,V,zero", [
    ("batched_ragged_vocab", 20, 5, 5003, False),    # tile maxima path, partial last tile
    ("batched_ties_all_tiles", 13, 7, 40000, True),  # every tile ties: more than 1024 tiles kept -> exact path
    ("batched_ties_candidates", 17, 5, 3000, True),  # 94 tiles kept but 3000 tied logits -> exact path
    ("batched_long_rows", 10, 7, 300000, False),     # 9375 tiles per row: past the 8192 kept in registers
])
def test_end_to_end_batched_tile_maxima_paths(name, R, L, V, zero):
    """More than 64 rows: the Top-K reads only the tiles the lm_head tile maxima keep,
    or all logits when ties keep too many; either way the same candidates as the
    stand-alone Top-K over the full logits (checked bit for bit inside _end_to_end)."""
    say(f"end-to-end {name}: R={R} L={L} V={V} zero_hidden={zero}")
    sh = di.custom_shape(name, R=R, L=L, H=128, Vd=V, K=64, r=16, seed=70 + R)
    inp = di.make_inputs(sh)
    if zero:
        inp = _zero_hidden(inp)
    _end_to_end(inp, list(range(R)))


def _scale_rows_bf16(bits, rows, factor):
    """bf16 rows multiplied by a power of two (exact)."""
    x = O.bf16_to_f64(bits[rows]) * factor
    out = bits.copy()
    out[rows] = di.round_to_bf16_bits(x.astype(np.float32))
    return out


@pytest.mark.parametrize("V", [40003, 151936])
def test_end_to_end_filter_bound_is_tight(V):
    """The logits filter (DFLASH_OPT_FILTER_LOGITS; more than 64 rows and at least 512
    vocabulary tiles; _end_to_end runs the step with and without it): the lm_head writes only the groups
    of logits that reach a bound from the exact logits of 128 sampled tiles (tile
    floor(j T / 128), T tiles).  Here the W rows of the sampled tiles are scaled by 8, so
    every row's top K lies among them and the bound is the row's K-th largest logit itself:
    a sample logit one rounding above the main kernel's would drop a member of the top K.
    The filtered step must match the unfiltered stage entry points and the oracle."""
    sh = di.custom_shape(f"filter_tight_{V}", R=10, L=7, H=128, Vd=V, K=64, r=16, table_std=0.5, seed=90)
    inp = di.make_inputs(sh)
    T = (V + 31) // 32
    tiles = [(j * T) // 128 for j in range(128)]
    rows = np.concatenate([np.arange(t * 32, t * 32 + 32) for t in tiles])
    inp.lm_head = _scale_rows_bf16(inp.lm_head, rows, 8.0)
    z = O.logits(inp.hidden[:3], inp.lm_head)
    for m in range(3):   # the planted rows do hold each row's top K
        assert set(O.topk_slots(z[m], 64).tolist()) <= set(rows.tolist())
    c = _end_to_end(inp, list(range(10)))
    _assert_mostly_exact(c)


def test_empty_batch_is_a_no_op():
    sh = di.custom_shape("empty", R=0, L=3, H=64, Vd=1024, K=8, r=4, seed=1)
    inp = di.make_inputs(sh)
    d = upload(inp)
    tokens, scores = api().draft_block(d["hidden"], d["lm_head"], d["tables"], d["last_tok"], top_k=8, block_len=3)
    torch.cuda.synchronize()
    assert tokens.numel() == 0 and scores.numel() == 0


def test_request_isolation_on_gpu():
    sh = di.custom_shape("iso", R=3, L=4, H=64, Vd=3000, K=16, r=16, table_std=0.5, seed=21)
    inp = di.make_inputs(sh)
    d = upload(inp)
    t1, s1 = api().draft_block(d["hidden"], d["lm_head"], d["tables"], d["last_tok"], top_k=16)
    h2 = inp.hidden.copy()
    h2[4:8] = di.round_to_bf16_bits(f32(np.random.default_rng(2).standard_normal((4, 64))))
    t2, s2 = api().draft_block(dev_bf16(h2), d["lm_head"], d["tables"], d["last_tok"], top_k=16)
    t1, t2, s1, s2 = (x.cpu().numpy() for x in (t1, t2, s1, s2))
    keep = np.r_[0:4, 8:12]
    assert np.array_equal(t1[keep], t2[keep]) and s1[0] == s2[0] and s1[2] == s2[2]
