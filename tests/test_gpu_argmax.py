"""GPU parity of the head-less draft step (dflash_draft_argmax) against the oracle.

Decision rule per row (the argmax is taken on fp32 z' on the GPU and on fp64
z' in the oracle): with v1 >= v2 the oracle's two best z' of the row and
tau = 1e-3 max|z'|, a gap v1 - v2 >= tau requires the oracle's id; a smaller
gap requires that the GPU's id reaches v1 - tau.  Values within 1e-5 max|z'|.
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


def _check(inp, rows, scale, cap, ids_gpu, tok_gpu, val_gpu):
    z = O.logits(inp.hidden[rows], inp.lm_head)
    ids_o, tok_o, val_o = O.argmax_rows(z, scale, cap, inp.d2t)
    zs = O.scale_cap(z, scale, cap)
    counts = dict(exact=0, exempt=0)
    for i, m in enumerate(rows):
        f = zs[i]
        top2 = np.sort(f)[-2:] if f.size > 1 else np.array([-np.inf, f[0]])
        v1, v2 = top2[1], top2[0]
        tau = 1e-3 * float(np.max(np.abs(f)))
        g = int(ids_gpu[m])
        assert 0 <= g < f.size
        if v1 - v2 >= tau:
            assert g == ids_o[i], f"row {m}: GPU id {g} != oracle id {ids_o[i]} (gap {v1 - v2} >= {tau})"
            counts["exact"] += 1
        else:
            assert f[g] >= v1 - tau, f"row {m}: GPU id {g} has z' {f[g]} < {v1} - {tau}"
            counts["exempt"] += 1
        want_tok = g + (int(inp.d2t[g]) if inp.d2t is not None else 0)
        assert int(tok_gpu[m]) == want_tok
        assert abs(float(val_gpu[m]) - v1) <= max(1e-5 * float(np.max(np.abs(f))), 1e-6)
    return counts


def _run(inp, scale, cap, rows=None):
    A = api()
    h, W = dev_bf16(inp.hidden), dev_bf16(inp.lm_head)
    d2t = dev(inp.d2t)
    tok, val = A.draft_argmax(h, W, d2t=d2t, target_vocab=inp.shape.Vt, out_scale=scale, soft_cap=cap)
    tok2, val2 = A.draft_argmax(h, W, d2t=d2t, target_vocab=inp.shape.Vt, out_scale=scale, soft_cap=cap)
    torch.cuda.synchronize()
    tok, val = tok.cpu().numpy(), val.cpu().numpy()
    assert np.array_equal(tok, tok2.cpu().numpy()) and np.array_equal(val, val2.cpu().numpy())   # deterministic
    ids = tok.copy()
    if inp.d2t is not None:
        # recover the draft id: the row's chosen target id maps back through the subset
        inv = {int(i + inp.d2t[i]): i for i in range(inp.d2t.size)}
        ids = np.array([inv[int(t)] for t in tok])
    rows = list(range(inp.M)) if rows is None else rows
    return _check(inp, rows, scale, cap, ids, tok, val)


CASES = [
    # name, R (rows), H, V_d, V_t (pruned when > V_d), scale, cap, zero hidden
    ("tiny_scan", 5, 64, 1024, 1024, 1.0, 0.0, False),
    ("tiny_cap", 5, 64, 1024, 1024, 1.7, 0.5, False),
    ("scan_64_rows", 64, 128, 3001, 3001, 0.9, 10.0, False),
    ("tiles_ragged", 100, 128, 5003, 5003, 1.3, 30.0, False),
    ("tiles_saturating", 70, 128, 3001, 3001, 100.0, 1.0, False),   # fp32 tanh saturates: ties at the cap
    ("tiles_all_tied", 80, 64, 40000, 40000, 2.0, 3.0, True),       # z = 0 everywhere: id 0
    ("scan_all_tied", 7, 64, 2000, 2000, 1.0, 0.0, True),
    ("tiles_pruned", 90, 64, 2000, 5000, 1.0, 0.0, False),
]


@pytest.mark.parametrize("name,R,H,V,Vt,scale,cap,zero", CASES)
def test_draft_argmax_parity(name, R, H, V, Vt, scale, cap, zero):
    say(f"argmax {name}: M={R} H={H} V_d={V} V_t={Vt} scale={scale} cap={cap} zero_hidden={zero}")
    sh = di.custom_shape(name, R=R, L=1, H=H, Vd=V, Vt=Vt, K=min(64, V), r=4, pruned=Vt > V, seed=300 + R)
    inp = di.make_inputs(sh)
    if zero:
        inp.hidden[:] = 0
    counts = _run(inp, scale, cap)
    say(f"  {counts}")


def test_draft_argmax_qwen3_4b_batch_sampled_rows():
    """The 224-row Qwen3-4B batch (tile path), 16 sampled rows against the oracle."""
    inp = di.make_inputs(di.SHAPES["qwen3_4b_32"])
    rows = list(range(0, inp.M, 14))
    say(f"argmax qwen3_4b_32: rows {rows}")
    counts = _run(inp, 1.25, 30.0, rows)
    say(f"  {counts}")


def test_draft_argmax_pruned_ocr_sampled_rows():
    """The pruned-vocabulary shape (d2t into 248100 targets), 12 sampled rows against the oracle."""
    inp = di.make_inputs(di.SHAPES["pruned_ocr"])
    rows = list(range(0, inp.M, 20))
    say(f"argmax pruned_ocr: rows {rows}")
    counts = _run(inp, 1.0, 30.0, rows)
    say(f"  {counts}")
