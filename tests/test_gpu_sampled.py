"""GPU parity of the sampled lattice walk (dflash_walk_sampled and
dflash_draft_block_sampled) against the oracle.

Fed the oracle's own fp32 unary and pair values, the walk takes the same fp32
steps as the oracle (fp32 row and temperature, weights rounded to fp32 from a
double exp, double sums in slot order, the caller's double uniforms), so the
drawn slots and the recorded proposals must agree exactly; a draw whose
U * total lies within 1e-12 * total of a running sum is exempt (counted,
expected 0).  The whole step computes its own unary and pair values in fp32:
there every position is re-drawn by the oracle from the GPU's candidates
(fp64 unary and pair values) and the GPU's previous slot, a draw with a
relative gap below 5e-5 is exempt, and the exemptions are counted and
bounded (see _sampled_end_to_end).
"""
import numpy as np
import pytest
import torch

import draft_inputs as di
from oracle import draft_step as O
from tests.gpu_util import check_topk_row, dev, dev_bf16, offsets_of, pack_pair, record, require_gpu, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def api():
    from block_draft_markov_amd import api as A
    return A


def f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _random_lattice(lengths, K, seed, ints=False):
    rng = np.random.default_rng(seed)
    M = sum(lengths)
    if ints:
        u = rng.integers(-3, 1, size=(M, K)).astype(np.float64)
    else:
        u = -np.sort(-rng.standard_normal((M, K)), axis=1) - 2.0
    S_all = []
    for Lr in lengths:
        S = []
        for p in range(Lr):
            shape = (1, K) if p == 0 else (K, K)
            S.append(rng.integers(-2, 3, size=shape).astype(np.float64) if ints else rng.standard_normal(shape))
        S_all.append(S)
    return u, S_all, di.ragged_offsets(lengths).astype(np.int64)


def _uniforms(M, seed):
    U = np.random.default_rng(seed).random(M)
    if M > 2:
        U[0] = 0.0
        U[-1] = np.nextafter(1.0, 0.0)
    return U


CASES = [
    # (name, lengths, K, integer scores, temperature)
    ("tiny", [5], 8, False, 1.0),
    ("batch_l7_k64", [7] * 32, 64, False, 1.0),
    ("batch_l15_k64_t07", [15] * 16, 64, False, 0.7),
    ("l1", [1, 1, 1], 64, False, 1.0),
    ("k1", [6, 4], 1, False, 1.0),
    ("l100", [100, 37], 64, False, 2.0),           # the maximum block length
    ("ragged_with_empty", [3, 0, 9, 1, 0], 16, False, 1.0),
    ("integer_scores", [6] * 20, 4, True, 1.0),    # equal weights: boundaries at exact fractions
]


@pytest.mark.parametrize("name,lengths,K,ints,T", CASES)
def test_sampled_walk_fed_oracle_values_exact(name, lengths, K, ints, T):
    say(f"sampled walk {name}: lengths {lengths[:6]}{'...' if len(lengths) > 6 else ''} K={K} T={T}")
    R = len(lengths)
    u64, S_all, off = _random_lattice(lengths, K, seed=len(name) * 17 + K, ints=ints)
    M = u64.shape[0]
    L = max(lengths)
    u32 = f32(u64)
    pair32 = f32(pack_pair(S_all, off, M, K))
    U = _uniforms(M, seed=M + K)
    tok = np.arange(M * K, dtype=np.int64).reshape(M, K) * 5 + 1
    tokens, scores, slots, q = api().walk_sampled(dev(tok), dev(u32), dev(pair32), R, dev(U), temperature=T,
                                                  row_offsets=dev(off.astype(np.int32)), block_len=L)
    torch.cuda.synchronize()
    tokens, scores, slots, q = tokens.cpu().numpy(), scores.cpu().numpy(), slots.cpu().numpy(), q.cpu().numpy()
    exempt = 0
    for req in range(R):
        a, b = int(off[req]), int(off[req + 1])
        if b == a:
            assert scores[req] == 0.0
            continue
        u = u32[a:b].astype(np.float64)
        S = [pair32[a, :1, :].astype(np.float64)] + [pair32[a + p].astype(np.float64) for p in range(1, b - a)]
        sw = O.sampled(u, S, U[a:b], temperature=T)
        if np.min(sw.gaps) < 1e-12:
            exempt += 1
            continue
        assert list(slots[a:b]) == list(sw.path), f"request {req}: slots differ"
        assert np.array_equal(tokens[a:b], tok[np.arange(a, b), sw.path])
        assert np.allclose(q[a:b], sw.q, rtol=1e-6, atol=0), f"request {req}: proposals differ"
        scale = max(1.0, abs(sw.score))
        assert abs(scores[req] - sw.score) <= 1e-4 * scale
    say(f"  exempt requests: {exempt}")


def _sampled_end_to_end(inp, sample_requests, T, seed, name=None):
    """The fused sampled step against the oracle on the given requests.

    Every position is re-drawn by the oracle (fp64 unary and pair values) from
    the GPU's candidates and the GPU's previous slot, with the same uniform.
    The drawn slot must be the GPU's unless U * total lies within 5e-5 * total
    of a running sum (fp32 rows are ~1e-6 relative from the oracle's; counted
    as a gap exemption).  A position whose GPU candidates are not the oracle's
    slots in the oracle's order (the Top-K boundary exemption, or ids closer
    than the logit error swapped) is counted separately; its draw is still
    checked on the GPU's candidates.
    """
    A = api()
    R, M, K = len(inp.last_tok), inp.M, inp.shape.K
    off = offsets_of(R, M, inp.row_offsets)
    L = int(np.max(np.diff(off))) if R else 1
    d = upload(inp)
    U = _uniforms(M, seed)
    Ud = dev(U)
    kw = dict(top_k=K, temperature=T, d2t=d["d2t"], gate_w=d["gate_w"], row_offsets=d["row_offsets"], block_len=L)
    tokens, scores, q = A.draft_block_sampled(d["hidden"], d["lm_head"], d["tables"], d["last_tok"], Ud, **kw)
    tokens2, scores2, q2 = A.draft_block_sampled(d["hidden"], d["lm_head"], d["tables"], d["last_tok"], Ud, **kw)
    tokens3, scores3, q3 = A.draft_block_sampled(d["hidden"], d["lm_head"], d["tables"], d["last_tok"], Ud,
                                                 filter_logits=True, **kw)
    # the staged calls: lm_head, Top-K, pair scores, then the sampled walk
    z, lse = A.lm_head(d["hidden"], d["lm_head"])
    idx, tok, un = A.topk(z, lse, K, d2t=d["d2t"], target_vocab=inp.tables.shape[1])
    pair = A.pair_scores(tok, d["tables"], d["last_tok"], gate_w=d["gate_w"], hidden=d["hidden"],
                         row_offsets=d["row_offsets"], block_len=L)
    st_tokens, st_scores, st_slots, st_q = A.walk_sampled(tok, un, pair, R, Ud, temperature=T,
                                                          row_offsets=d["row_offsets"], block_len=L)
    torch.cuda.synchronize()
    tokens, scores, q = tokens.cpu().numpy(), scores.cpu().numpy(), q.cpu().numpy()
    assert np.array_equal(tokens, tokens2.cpu().numpy()) and np.array_equal(q, q2.cpu().numpy())
    # the opt-in logits filter: the same draws bit for bit
    assert np.array_equal(tokens, tokens3.cpu().numpy()) and np.array_equal(q, q3.cpu().numpy())
    assert np.array_equal(scores, scores3.cpu().numpy())
    assert np.array_equal(tokens, st_tokens.cpu().numpy()) and np.array_equal(scores, st_scores.cpu().numpy())
    assert np.array_equal(q, st_q.cpu().numpy())
    idx, gtok, slots = idx.cpu().numpy().astype(np.int64), tok.cpu().numpy(), st_slots.cpu().numpy()
    counts = dict(positions=0, exact=0, gap_exempt=0, topk_exempt=0)
    reqs = [r for r in sample_requests if off[r + 1] > off[r]]
    for req in sample_requests:
        if off[req + 1] == off[req]:
            assert scores[req] == 0.0
    if not reqs:
        return counts
    rows_all = np.concatenate([np.arange(off[r], off[r + 1]) for r in reqs])
    zo_all = O.logits(inp.hidden[rows_all], inp.lm_head)
    base = 0
    for req in reqs:
        a, b = int(off[req]), int(off[req + 1])
        rows = np.arange(a, b)
        zo = zo_all[base:base + (b - a)]
        base += b - a
        kinds = [check_topk_row(idx[a + i], zo[i], K) for i in range(b - a)]
        lse = O.row_lse(zo)
        u_o = np.take_along_axis(zo, idx[a:b], 1) - lse[:, None]        # fp64 unary of the GPU's slots
        h = O.bf16_to_f64(inp.hidden[rows])
        S_o = O.lattice_scores(gtok[a:b], inp.tables, h, inp.gate_w, int(inp.last_tok[req]))
        for p in range(b - a):
            counts["positions"] += 1
            prev = 0 if p == 0 else int(slots[a + p - 1])
            row = S_o[p][prev:prev + 1] if p > 0 else S_o[0][:1]
            sw = O.sampled(u_o[p:p + 1], [row], U[a + p:a + p + 1], temperature=T)
            if kinds[p] != "same":
                counts["topk_exempt"] += 1
            if sw.gaps[0] < 5e-5:
                counts["gap_exempt"] += 1
            else:
                assert slots[a + p] == sw.path[0], f"request {req} position {p}: slot {slots[a + p]} vs {sw.path[0]}"
                counts["exact"] += kinds[p] == "same"
            assert np.max(np.abs(q[a + p] - sw.q[0])) <= 1e-5, f"request {req} position {p}: proposal"
            assert tokens[a + p] == gtok[a + p][slots[a + p]]
        gpu_score = O.path_score(u_o, S_o, slots[a:b])
        assert abs(scores[req] - gpu_score) <= 1e-4 * max(1.0, abs(gpu_score))
    record(name or inp.shape.name, sampled=True, temperature=T, **counts)
    n = counts["positions"]
    assert counts["exact"] >= 1, counts
    assert counts["gap_exempt"] <= max(3, n // 25), counts
    assert counts["topk_exempt"] <= max(1, n // 10), counts
    return counts


def test_sampled_end_to_end_tiny():
    inp = di.make_inputs(di.SHAPES["tiny_stress"])
    _sampled_end_to_end(inp, [0], T=1.0, seed=1)


@pytest.mark.parametrize("seed", range(4))
def test_sampled_end_to_end_tiny_seeds(seed):
    sh = di.custom_shape("tiny_s", R=1, L=5, H=64, Vd=1024, K=8, r=16, table_std=0.5, seed=3000 + seed)
    _sampled_end_to_end(di.make_inputs(sh), [0], T=0.8 + 0.2 * seed, seed=seed)


def test_sampled_end_to_end_gated_ragged():
    sh = di.custom_shape("gated_r", R=4, L=6, H=64, Vd=2000, K=16, r=32, gated=True, table_std=0.4, seed=71)
    inp = di.make_inputs(sh)
    inp.row_offsets = di.ragged_offsets([6, 0, 2, 5])
    inp.hidden = np.ascontiguousarray(inp.hidden[:13])
    _sampled_end_to_end(inp, range(4), T=1.0, seed=5)


def test_sampled_end_to_end_pruned_48():
    sh = di.custom_shape("pruned48", R=3, L=4, H=64, Vd=48, Vt=200, K=48, r=8, pruned=True, table_std=0.5, seed=19)
    _sampled_end_to_end(di.make_inputs(sh), range(3), T=1.0, seed=6)


def test_sampled_end_to_end_qwen3_4b_batch_all_requests():
    """The Qwen3-4B batch (32 requests x 7 rows), every request against the oracle."""
    inp = di.make_inputs(di.SHAPES["qwen3_4b_32"])
    _sampled_end_to_end(inp, range(32), T=1.0, seed=7)


def test_sampled_end_to_end_dflash2_27b_all_requests():
    """The gated 27B shape (16 requests x 15 rows, V 248100, H 5120), every request against the oracle."""
    inp = di.make_inputs(di.SHAPES["dflash2_27b"])
    _sampled_end_to_end(inp, range(16), T=1.0, seed=8)


def test_sampled_end_to_end_pruned_ocr_all_requests():
    """The pruned vocabulary (16 requests x 15 rows, 114688 -> 248100), every request against the oracle."""
    inp = di.make_inputs(di.SHAPES["pruned_ocr"])
    _sampled_end_to_end(inp, range(16), T=0.9, seed=9)
