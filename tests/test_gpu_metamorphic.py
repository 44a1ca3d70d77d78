"""Metamorphic checks of the HIP draft step: transformations of the inputs that
must leave the drafted tokens unchanged, run through the C ABI on the GPU.

  * per-row logit shift: adding a constant to every logit of a row leaves the
    slots unchanged (compared bit for bit) and the tokens unchanged, since the
    log-sum-exp cancels the constant in the unary;
  * an all-zero d2t is the identity map: results bit-identical to d2t = NULL,
    for the Top-K lattice step, the head-less step and the dense walk;
  * pruned-vocabulary permutation: permuting the draft vocabulary (the rows of
    W and the d2t targets together) leaves the drafted target tokens unchanged
    (optimum-intel page "Support MiniCPM-OCR-1.0-DSpark", What does this PR
    do?: draft token i maps to target token i + d2t[i]; Tests: each input is
    read only in its own rows).

Token comparisons are exact.  Where the transformed step rounds differently
(the log-sum-exp of a permuted or shifted row is summed in another order), a
request whose runner-up margin, taken by the oracle's walk on the GPU's own
fp32 logits, is below 1e-5 * max(|S|, 1) is counted as exempt; at most a tenth
of the requests may be.
"""
import numpy as np
import pytest
import torch

import draft_inputs as di
from oracle import draft_step as O
from tests.gpu_util import dev, dev_bf16, offsets_of, record, require_gpu, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def api():
    from block_draft_markov_amd import api as A
    return A


def _margins(z_gpu, inp, K):
    """Oracle runner-up margins and scores of the walk over the GPU's own fp32 logits."""
    res = O.draft_from_logits(z_gpu.astype(np.float64), K, inp.d2t, inp.tables, inp.hidden, inp.gate_w,
                              inp.last_tok, inp.row_offsets)
    return res.margins, res.scores


def _compare_tokens(t1, t2, s1, s2, margins, scores, off, what):
    exempt = 0
    for req in range(len(off) - 1):
        a, b = int(off[req]), int(off[req + 1])
        scale = max(1.0, abs(scores[req]))
        assert abs(s1[req] - s2[req]) <= 1e-5 * scale, f"{what}: request {req} score {s1[req]} vs {s2[req]}"
        if margins[req] < 1e-5 * scale:
            exempt += 1
            continue
        assert np.array_equal(t1[a:b], t2[a:b]), f"{what}: request {req} tokens differ"
    R = len(off) - 1
    assert exempt <= max(1, R // 10), f"{what}: {exempt} of {R} requests exempt"
    return exempt


@pytest.mark.parametrize("name,R,L,H,V,K", [
    ("mid", 8, 7, 256, 20000, 64),
    ("qwen3_4b_rows", 4, 7, 2560, 151936, 64),
])
def test_per_row_logit_shift(name, R, L, H, V, K):
    """Logits on a 2^-10 grid plus per-row integer shifts: both are exact in fp32, so the
    shifted rows order exactly as the original ones."""
    A = api()
    rng = np.random.default_rng(len(name) + V)
    M = R * L
    z = (rng.integers(-4096, 4096, size=(M, V)) / 1024.0).astype(np.float32)
    shift = rng.integers(-40, 41, size=(M, 1)).astype(np.float32)
    z2 = z + shift
    assert np.array_equal(z2 - shift, z)      # the shift is exact
    Vt = V
    tables = (rng.standard_normal((2, Vt, 32)) * 0.4).astype(np.float32)
    last = rng.integers(0, Vt, size=R).astype(np.int64)
    out = []
    for zz in (z, z2):
        zt = dev(zz)
        lse = A.row_lse(zt)
        idx, tok, un = A.topk(zt, lse, K)
        tokens, scores = A.lattice(tok, un, dev(tables), dev(last), block_len=L)
        torch.cuda.synchronize()
        out.append((idx.cpu().numpy(), tok.cpu().numpy(), un.cpu().numpy(), tokens.cpu().numpy(),
                    scores.cpu().numpy()))
    (i1, k1, u1, t1, s1), (i2, k2, u2, t2, s2) = out
    assert np.array_equal(i1, i2) and np.array_equal(k1, k2), "slots changed under a per-row shift"
    assert np.max(np.abs(u1 - u2)) <= 1e-5
    # margins of the oracle's walk over these exact fp32 logits
    res = O.draft_from_logits(z.astype(np.float64), K, None, tables, np.zeros((M, 8), np.uint16), None, last)
    off = np.arange(R + 1) * L
    ex = _compare_tokens(t1, t2, s1, s2, res.margins, res.scores, off, "shift")
    record(f"shift_{name}", requests=R, exempt=ex)


@pytest.mark.parametrize("name,R,L,H,V", [("mid", 6, 5, 128, 9000), ("ragged_vocab", 4, 7, 64, 3001)])
def test_all_zero_d2t_is_null(name, R, L, H, V):
    A = api()
    sh = di.custom_shape(name, R=R, L=L, H=H, Vd=V, K=min(64, V), r=16, table_std=0.5, seed=30 + V)
    inp = di.make_inputs(sh)
    d = upload(inp)
    zero = torch.zeros(V, dtype=torch.int64, device="cuda")
    a = A.draft_block(d["hidden"], d["lm_head"], d["tables"], d["last_tok"], top_k=sh.K)
    b = A.draft_block(d["hidden"], d["lm_head"], d["tables"], d["last_tok"], top_k=sh.K, d2t=zero)
    g = A.draft_block(d["hidden"], d["lm_head"], d["tables"], d["last_tok"], top_k=sh.K, d2t=zero, walk="greedy")
    g0 = A.draft_block(d["hidden"], d["lm_head"], d["tables"], d["last_tok"], top_k=sh.K, walk="greedy")
    h0 = A.draft_argmax(d["hidden"], d["lm_head"], out_scale=1.5, soft_cap=3.0)
    h1 = A.draft_argmax(d["hidden"], d["lm_head"], d2t=zero, out_scale=1.5, soft_cap=3.0)
    n0 = A.draft_dense(d["hidden"], d["lm_head"], d["tables"], d["last_tok"], out_scale=1.0, soft_cap=0.0)
    n1 = A.draft_dense(d["hidden"], d["lm_head"], d["tables"], d["last_tok"], d2t=zero, out_scale=1.0, soft_cap=0.0)
    torch.cuda.synchronize()
    for x, y, what in ((a, b, "viterbi"), (g0, g, "greedy"), (h0, h1, "head-less"), (n0, n1, "dense")):
        for u, v in zip(x, y):
            assert torch.equal(u, v), f"{what}: zero d2t differs from no d2t"


def _permuted(inp, perm):
    """The same draft with draft id i renamed perm^-1[i]: W'[j] = W[perm[j]], and the
    target of draft id j is the target of perm[j]."""
    Vd = inp.lm_head.shape[0]
    tgt = np.arange(Vd, dtype=np.int64) + (inp.d2t if inp.d2t is not None else 0)
    out = di.DraftInputs(inp.shape, inp.hidden, np.ascontiguousarray(inp.lm_head[perm]), inp.tables, inp.last_tok,
                         (tgt[perm] - np.arange(Vd)).astype(np.int64), inp.gate_w, inp.row_offsets)
    return out


@pytest.mark.parametrize("shape", ["mid", "pruned_ocr"])
def test_pruned_vocabulary_permutation(shape):
    A = api()
    if shape == "mid":
        sh = di.custom_shape("perm_mid", R=8, L=15, H=256, Vd=30000, Vt=70000, K=64, r=32, pruned=True,
                             table_std=0.5, seed=44)
    else:
        sh = di.SHAPES["pruned_ocr"]
    inp = di.make_inputs(sh)
    perm = np.random.default_rng(3).permutation(sh.Vd)
    inp2 = _permuted(inp, perm)
    # the permuted draft maps to the same set of target ids
    assert np.array_equal(np.sort(np.arange(sh.Vd) + inp.d2t), np.sort(np.arange(sh.Vd) + inp2.d2t))
    res = []
    for x in (inp, inp2):
        d = upload(x)
        t, s = A.draft_block(d["hidden"], d["lm_head"], d["tables"], d["last_tok"], top_k=sh.K, d2t=d["d2t"])
        z, _ = A.lm_head(d["hidden"], d["lm_head"])
        torch.cuda.synchronize()
        res.append((t.cpu().numpy(), s.cpu().numpy(), z.cpu().numpy()))
        del d
    (t1, s1, z1), (t2, s2, z2) = res
    # the logits are the same numbers, renamed: each is one row of W against one hidden state
    assert np.array_equal(z2, z1[:, perm]), "permuted logits are not the original ones renamed"
    margins, scores = _margins(z1, inp, sh.K)
    off = offsets_of(len(inp.last_tok), inp.M, None)
    ex = _compare_tokens(t1, t2, s1, s2, margins, scores, off, "permutation")
    record(f"permutation_{shape}", requests=len(off) - 1, exempt=ex)
