"""GPU parity of the dense Markov walk (dflash_draft_dense) against the oracle.

Every row is checked on its own: the oracle's biased row x_p is built from
the previous token the GPU chose (last_tok at position 0), so one near tie
cannot derail the rest of a block.  Decision rule per row (the GPU takes the
argmax in fp32, the oracle in fp64): with v1 >= v2 the oracle's two best x of
the row and tau = 1e-3 max|x|, a gap v1 - v2 >= tau requires the oracle's id;
a smaller gap requires that the GPU's id reaches v1 - tau.  Values within
1e-5 of the row's scale.  When no row needed the exemption, the GPU's tokens
must also equal the oracle's own walk, chained through its own choices.
"""
import numpy as np
import pytest
import torch

import draft_inputs as di
from oracle import draft_step as O
from tests.gpu_util import dev, dev_bf16, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def api():
    from block_draft_markov_amd import api as A
    return A


def _ids_of(tok, d2t):
    if d2t is None:
        return tok.copy()
    inv = {int(i + d2t[i]): i for i in range(d2t.size)}
    return np.array([inv[int(t)] for t in tok], dtype=np.int64)


def _offsets(R, L, M, row_offsets):
    if row_offsets is not None:
        return np.asarray(row_offsets, np.int64)
    return np.arange(R + 1, dtype=np.int64) * L


def _run_gpu(inp, hidden, row_offsets, L, scale, cap):
    A = api()
    args = (dev_bf16(hidden), dev_bf16(inp.lm_head), dev(inp.tables), dev(inp.last_tok))
    kw = dict(d2t=dev(inp.d2t), row_offsets=dev(row_offsets), block_len=L, out_scale=scale, soft_cap=cap)
    tok, val = A.draft_dense(*args, **kw)
    tok2, val2 = A.draft_dense(*args, **kw)
    torch.cuda.synchronize()
    tok, val = tok.cpu().numpy(), val.cpu().numpy()
    assert np.array_equal(tok, tok2.cpu().numpy()) and np.array_equal(val, val2.cpu().numpy())   # deterministic
    return tok, val


def _check(inp, hidden, row_offsets, L, scale, cap, tok, val, rows=None):
    """Row-by-row rule; rows = the rows to check (all by default)."""
    R = inp.last_tok.size
    M = hidden.shape[0]
    off = _offsets(R, L, M, row_offsets)
    ids = _ids_of(tok, inp.d2t)
    want = list(range(M)) if rows is None else sorted(rows)
    Z = O.logits(hidden[want], inp.lm_head) if want else None
    zrow = {m: i for i, m in enumerate(want)}
    Vd = inp.lm_head.shape[0]
    Bt = np.asarray(inp.tables[1], np.float64)[O.draft_to_target(np.arange(Vd), inp.d2t)]
    counts = dict(exact=0, exempt=0)
    for req in range(R):
        a, b = int(off[req]), int(off[req + 1])
        for m in range(a, b):
            if m not in zrow:
                continue
            prev = int(inp.last_tok[req]) if m == a else int(tok[m - 1])
            z = Z[zrow[m]]
            zs = O.scale_cap(z, scale, cap)
            x = zs + Bt @ np.asarray(inp.tables[0][prev], np.float64)
            c, v, margin = O.dense_row(z, scale, cap, inp.d2t, inp.tables, prev)
            assert v == x[c]
            top2 = np.sort(x)[-2:] if Vd > 1 else np.array([-np.inf, x[0]])
            v1, v2 = top2[1], top2[0]
            tau = 1e-3 * float(np.max(np.abs(x)))
            g = int(ids[m])
            assert 0 <= g < Vd
            if v1 - v2 >= tau:
                assert g == c, f"row {m}: GPU id {g} != oracle id {c} (gap {v1 - v2} >= {tau})"
                counts["exact"] += 1
            else:
                assert x[g] >= v1 - tau, f"row {m}: GPU id {g} has x {x[g]} < {v1} - {tau}"
                counts["exempt"] += 1
            scale_v = max(float(np.max(np.abs(x))), float(np.max(np.abs(zs))), 1e-6)
            assert abs(float(val[m]) - x[g]) <= 1e-5 * scale_v, f"row {m}: value {val[m]} vs {x[g]}"
    return counts


def _whole_walk_equal(inp, hidden, row_offsets, scale, cap, tok):
    z = O.logits(hidden, inp.lm_head)
    res = O.dense_walk(z, scale, cap, inp.d2t, inp.tables, inp.last_tok, row_offsets)
    assert np.array_equal(res.tokens, tok)


def _case(name, R, L, H, V, Vt, r, *, lengths=None, scale=1.0, cap=0.0, table_std=0.25, zero_hidden=False,
          zero_tables=False, seed=0):
    say(f"dense {name}: R={R} L={L} H={H} V_d={V} V_t={Vt} r={r} lengths={lengths} scale={scale} cap={cap}")
    sh = di.custom_shape(name, R=R, L=L, H=H, Vd=V, Vt=Vt, K=min(64, V), r=r, pruned=Vt > V,
                         table_std=table_std, seed=seed)
    inp = di.make_inputs(sh)
    row_offsets = None
    hidden = inp.hidden
    if lengths is not None:
        row_offsets = di.ragged_offsets(lengths)
        hidden = np.ascontiguousarray(hidden[: int(row_offsets[-1])])
    if zero_hidden:
        hidden = np.zeros_like(hidden)
    if zero_tables:
        inp.tables[:] = 0
    return inp, hidden, row_offsets


CASES = [
    # name, R, L, H, V_d, V_t, r, lengths, scale, cap, table_std
    ("tiny", 1, 5, 64, 1024, 1024, 16, None, 1.0, 0.0, 0.02),
    ("tiny_strong_tables", 1, 5, 64, 1024, 1024, 16, None, 1.0, 0.0, 0.5),
    ("capped", 3, 7, 128, 3001, 3001, 32, None, 1.7, 5.0, 0.3),
    # 40 requests: two groups of 32, the second partial; ragged blocks with empty ones;
    # V = 5003: a ragged last tile of 256 ids; r = 20: scalar loads, rank padding
    ("ragged_two_groups", 40, 7, 64, 5003, 5003, 20, "ragged", 1.0, 0.0, 0.25),
    ("rank_300_two_chunks", 5, 4, 64, 2000, 2000, 300, None, 1.0, 30.0, 0.1),
    ("rank_1", 4, 6, 64, 777, 777, 1, None, 1.0, 0.0, 1.0),
    ("pruned_vocab", 6, 5, 64, 1500, 4000, 16, None, 1.0, 0.0, 0.4),
    ("block_len_100", 2, 100, 64, 1024, 1024, 16, [100, 37], 1.0, 0.0, 0.3),
    # the LDS-staged kernel at its largest rank (512, the deeper A buffer)
    ("rank_512_staged", 3, 4, 64, 1500, 1500, 512, None, 1.0, 0.0, 0.05),
    # ranks the staged kernel does not take: not a multiple of 4 (scalar loads of the
    # register-streamed kernel), and above 512 (its 16-byte loads, three rank chunks)
    ("rank_30_register_path", 3, 5, 64, 2003, 2003, 30, None, 1.0, 0.0, 0.2),
    ("rank_520_register_path", 3, 4, 64, 1500, 1500, 520, None, 1.7, 5.0, 0.05),
    # 9375 tiles: more than 256 workgroups of at most 32 tiles each
    ("vocab_300k_wide_grid", 2, 3, 64, 300000, 300000, 16, None, 1.0, 0.0, 0.3),
]


def _lengths(spec, R, L, seed):
    if spec != "ragged":
        return spec
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, L + 1, size=R)
    lens[0] = L
    return [int(x) for x in lens]


@pytest.mark.parametrize("name,R,L,H,V,Vt,r,lengths,scale,cap,std", CASES)
def test_draft_dense_parity(name, R, L, H, V, Vt, r, lengths, scale, cap, std):
    lens = _lengths(lengths, R, L, seed=R + L)
    inp, hidden, off = _case(name, R, L, H, V, Vt, r, lengths=lens, scale=scale, cap=cap, table_std=std,
                             seed=500 + R * 7 + r)
    tok, val = _run_gpu(inp, hidden, off, L, scale, cap)
    counts = _check(inp, hidden, off, L, scale, cap, tok, val)
    say(f"  {counts}")
    if counts["exempt"] == 0:
        _whole_walk_equal(inp, hidden, off, scale, cap, tok)


def test_draft_dense_zero_tables_is_the_headless_argmax():
    """With zero tables the bias vanishes: the dense walk takes the head-less argmax of every row."""
    inp, hidden, off = _case("zero_tables", 9, 7, 64, 3001, 3001, 16, zero_tables=True, scale=1.3, cap=4.0,
                             seed=77)
    tok, val = _run_gpu(inp, hidden, off, 7, 1.3, 4.0)
    counts = _check(inp, hidden, off, 7, 1.3, 4.0, tok, val)
    ids_o, tok_o, _ = O.argmax_rows(O.logits(hidden, inp.lm_head), 1.3, 4.0, inp.d2t)
    if counts["exempt"] == 0:
        assert np.array_equal(tok, tok_o)
    A = api()
    tok_a, val_a = A.draft_argmax(dev_bf16(hidden), dev_bf16(inp.lm_head), out_scale=1.3, soft_cap=4.0)
    torch.cuda.synchronize()
    # same logits kernel, same fp32 scale and cap, bias exactly 0: identical outputs
    assert np.array_equal(tok, tok_a.cpu().numpy())
    assert np.array_equal(val, val_a.cpu().numpy())


def test_draft_dense_all_tied_rows_take_id_zero():
    """Zero hidden states and zero tables: every x is 0 and the lowest id, 0, wins everywhere."""
    inp, hidden, off = _case("all_tied", 35, 3, 64, 2000, 2000, 8, zero_hidden=True, zero_tables=True, seed=9)
    tok, val = _run_gpu(inp, hidden, off, 3, 1.0, 0.0)
    assert np.all(tok == 0) and np.all(val == 0.0)


def test_draft_dense_empty_requests():
    """Requests without rows write nothing; total_rows = 0 launches nothing and succeeds."""
    inp, hidden, off = _case("empty", 4, 3, 64, 512, 512, 8, lengths=[0, 3, 0, 1], seed=11)
    tok, val = _run_gpu(inp, hidden, off, 3, 1.0, 0.0)
    counts = _check(inp, hidden, off, 3, 1.0, 0.0, tok, val)
    assert counts["exact"] + counts["exempt"] == 4
    inp0, hidden0, off0 = _case("none", 3, 2, 64, 512, 512, 8, lengths=[0, 0, 0], seed=12)
    A = api()
    tok0, _ = A.draft_dense(dev_bf16(hidden0), dev_bf16(inp0.lm_head), dev(inp0.tables), dev(inp0.last_tok),
                            row_offsets=dev(off0), block_len=2)
    torch.cuda.synchronize()
    assert tok0.numel() == 0


def test_draft_dense_qwen3_4b_batch_sampled_rows():
    """The Qwen3-4B batch (32 requests x 7 rows, r = 256) as timed: sampled rows against the oracle."""
    inp = di.make_inputs(di.SHAPES["qwen3_4b_32"])
    L = inp.shape.L
    tok, val = _run_gpu(inp, inp.hidden, None, L, 1.0, 30.0)
    rows = [0, 1, 6, 7 * 9 + 3, 7 * 17 + 6, 7 * 31, 7 * 31 + 5]
    say(f"dense qwen3_4b_32: rows {rows}")
    counts = _check(inp, inp.hidden, None, L, 1.0, 30.0, tok, val, rows=rows)
    say(f"  {counts}")


def test_draft_dense_pruned_ocr_sampled_rows():
    """The pruned-vocabulary shape (114688 draft ids mapped into 248100 targets, H 2048, 16 x 15 rows):
    B rows gathered by target id through d2t, sampled rows against the oracle."""
    inp = di.make_inputs(di.SHAPES["pruned_ocr"])
    L = inp.shape.L
    tok, val = _run_gpu(inp, inp.hidden, None, L, 1.0, 30.0)
    rows = [0, 1, 14, 15 * 7 + 8, 15 * 15 + 14]
    say(f"dense pruned_ocr: rows {rows}")
    counts = _check(inp, inp.hidden, None, L, 1.0, 30.0, tok, val, rows=rows)
    say(f"  {counts}")
