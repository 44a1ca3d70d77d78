"""The C ABI on the CPU: the library loads, exports every symbol that
include/*.h declares, and rejects bad arguments on the host before any launch
(no GPU is touched: every call here fails validation first)."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import block_draft_markov_amd as bdm
from block_draft_markov_amd._lib import Dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000          # a 256-byte aligned non-NULL address; never dereferenced (validation fails first)
FAKE_ODD = 0x100008      # 8-byte aligned only


def header_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(dflash_\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return bdm.load()


def dims(**kw):
    base = dict(num_requests=2, block_len=3, total_rows=6, hidden=64, draft_vocab=1024, target_vocab=1024,
                top_k=8, rank=16, walk=0)
    base.update(kw)
    return Dims(**base)


def err(lib):
    return lib.dflash_last_error().decode()


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert len(names) == 16, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    assert set(names) == set(bdm.SIGNATURES), "binding and header disagree"


def test_workspace_bytes_and_stride(lib):
    d = dims()
    n = lib.dflash_workspace_bytes(ctypes.byref(d))
    assert n > 0 and n % 256 == 0
    # grows with the rows and the vocabulary
    assert lib.dflash_workspace_bytes(ctypes.byref(dims(num_requests=4, total_rows=12))) > n
    assert lib.dflash_workspace_bytes(ctypes.byref(dims(draft_vocab=4096, target_vocab=4096))) > n
    assert lib.dflash_logits_stride(151936) == 151936
    assert lib.dflash_logits_stride(1023) == 1024
    assert lib.dflash_logits_stride(48) == 48
    # invalid dims -> 0 and a message
    assert lib.dflash_workspace_bytes(ctypes.byref(dims(top_k=0))) == 0
    assert "top_k" in err(lib)
    assert lib.dflash_workspace_bytes(None) == 0


@pytest.mark.parametrize("kw,code,word", [
    (dict(top_k=0), bdm.EINVAL, "top_k"),
    (dict(top_k=65, draft_vocab=100000, target_vocab=100000), bdm.EINVAL, "top_k"),
    (dict(top_k=49, draft_vocab=48, target_vocab=48), bdm.EINVAL, "top_k"),   # K <= min(64, V_d)
    (dict(block_len=0, total_rows=0), bdm.EINVAL, "block_len"),
    (dict(block_len=101, total_rows=202), bdm.EINVAL, "block_len"),
    (dict(hidden=60), bdm.EINVAL, "hidden"),
    (dict(hidden=0), bdm.EINVAL, "hidden"),
    (dict(draft_vocab=0), bdm.EINVAL, "draft_vocab"),
    (dict(target_vocab=1000), bdm.EINVAL, "target_vocab"),
    (dict(rank=0), bdm.EINVAL, "rank"),
    (dict(walk=2), bdm.EINVAL, "walk"),
    (dict(options=2), bdm.EINVAL, "options"),
    (dict(num_requests=-1), bdm.EINVAL, "num_requests"),
    (dict(total_rows=7), bdm.EINVAL, "total_rows"),
    (dict(total_rows=5), bdm.EINVAL, "row_offsets"),   # uniform blocks need M = R * L
])
def test_draft_block_rejects_bad_dims(lib, kw, code, word):
    d = dims(**kw)
    rc = lib.dflash_draft_block(ctypes.byref(d), FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, FAKE,
                                1 << 40, None)
    assert rc == code
    assert word in err(lib)


def test_draft_block_pointer_and_mode_rules(lib):
    d = dims()
    big = 1 << 40
    call = lambda **p: lib.dflash_draft_block(
        ctypes.byref(p.get("d", d)), p.get("hidden", FAKE), p.get("lm", FAKE), p.get("d2t", None),
        p.get("tables", FAKE), p.get("gate", None), p.get("last", FAKE), p.get("off", None), p.get("tok", FAKE),
        p.get("sc", FAKE), p.get("ws", FAKE), p.get("wsn", big), None)
    assert call(hidden=None) == bdm.EINVAL and "hidden" in err(lib)
    assert call(lm=None) == bdm.EINVAL and "lm_head" in err(lib)
    assert call(tables=None) == bdm.EINVAL and "tables" in err(lib)
    assert call(last=None) == bdm.EINVAL and "last_tok" in err(lib)
    assert call(tok=None) == bdm.EINVAL and "tokens" in err(lib)
    assert call(sc=None) == bdm.EINVAL and "scores" in err(lib)
    # a pruned vocabulary needs d2t
    dp = dims(target_vocab=4096)
    assert call(d=dp) == bdm.EINVAL and "d2t" in err(lib)
    # gated transitions with a pruned vocabulary are rejected
    assert call(d=dp, d2t=FAKE, gate=FAKE) == bdm.EUNSUPPORTED and "gate_w" in err(lib)
    # workspace
    assert call(ws=None) == bdm.EWORKSPACE
    need = lib.dflash_workspace_bytes(ctypes.byref(d))
    assert call(wsn=need - 1) == bdm.EWORKSPACE and str(need) in err(lib)
    assert call(ws=FAKE_ODD) == bdm.EINVAL and "aligned" in err(lib)
    # 16-byte alignment of the bf16 operands
    assert call(hidden=FAKE + 2) == bdm.EINVAL and "aligned" in err(lib)


@pytest.mark.parametrize("R,L,M", [(0, 3, 0), (2, 5, 0), (1, 1, 1), (400, 1, 400)])
def test_workspace_sizing_edge_rows(lib, R, L, M):
    # empty batches, a single row and more rows than one 256-row chunk size without faults
    n = lib.dflash_workspace_bytes(ctypes.byref(dims(num_requests=R, block_len=L, total_rows=M)))
    assert n >= 256 and n % 256 == 0


def test_empty_batch_returns_before_any_launch(lib):
    # M = 0 rows: nothing to launch, every array may be NULL; a NULL stream is never used
    d = dims(num_requests=0, block_len=3, total_rows=0)
    need = lib.dflash_workspace_bytes(ctypes.byref(d))
    assert lib.dflash_draft_block(ctypes.byref(d), None, FAKE, None, FAKE, None, None, None, None, None, FAKE,
                                  need, None) == bdm.OK


def test_stage_entry_points_validate(lib):
    d = dims()
    big = 1 << 40
    # lm_head: ldz must cover V_d and be a multiple of 4
    assert lib.dflash_lm_head(ctypes.byref(d), FAKE, FAKE, FAKE, 1022, FAKE, FAKE, big, None) == bdm.EINVAL
    assert "ldz" in err(lib)
    assert lib.dflash_lm_head(ctypes.byref(d), FAKE, FAKE, FAKE, 1026, FAKE, FAKE, big, None) == bdm.EINVAL
    assert lib.dflash_lm_head(ctypes.byref(d), FAKE, FAKE, None, 1024, FAKE, FAKE, big, None) == bdm.EINVAL
    assert "logits" in err(lib)
    assert lib.dflash_row_lse(ctypes.byref(d), FAKE, 1000, FAKE, None) == bdm.EINVAL
    assert lib.dflash_row_lse(ctypes.byref(d), FAKE, 1024, None, None) == bdm.EINVAL and "lse" in err(lib)
    # topk
    assert lib.dflash_topk(ctypes.byref(d), FAKE, 1024, FAKE, None, FAKE, FAKE, FAKE, FAKE, 16, None) == \
        bdm.EWORKSPACE
    assert lib.dflash_topk(ctypes.byref(dims(target_vocab=2000)), FAKE, 1024, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                           big, None) == bdm.EINVAL and "d2t" in err(lib)
    assert lib.dflash_topk(ctypes.byref(d), FAKE, 1024, FAKE, None, None, FAKE, FAKE, FAKE, big, None) == \
        bdm.EINVAL and "cand_idx" in err(lib)
    # pair scores: the gate reads the hidden states
    assert lib.dflash_pair_scores(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None) == bdm.EINVAL
    assert "hidden" in err(lib)
    assert lib.dflash_pair_scores(ctypes.byref(dims(total_rows=4)), FAKE, FAKE, None, None, FAKE, None, FAKE,
                                  None) == bdm.EINVAL
    # walk
    assert lib.dflash_walk(ctypes.byref(dims(walk=3)), FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None) == \
        bdm.EINVAL and "walk" in err(lib)
    assert lib.dflash_walk(ctypes.byref(d), FAKE, FAKE, None, None, FAKE, FAKE, None, None) == bdm.EINVAL
    assert "pair" in err(lib)


def test_check_d2t_host(lib):
    sub = np.random.default_rng(3).permutation(200)[:48]
    d2t = np.ascontiguousarray(sub - np.arange(48), dtype=np.int64)
    inj = ctypes.c_int(-1)
    assert lib.dflash_check_d2t(d2t.ctypes.data, 48, 200, ctypes.byref(inj)) == bdm.OK and inj.value == 1
    assert err(lib) == ""
    dup = d2t.copy()
    dup[1] = sub[0] - 1
    assert lib.dflash_check_d2t(dup.ctypes.data, 48, 200, ctypes.byref(inj)) == bdm.OK and inj.value == 0
    bad = d2t.copy()
    bad[7] = 500
    assert lib.dflash_check_d2t(bad.ctypes.data, 48, 200, ctypes.byref(inj)) == bdm.EINVAL
    assert "d2t[7]" in err(lib)
    neg = d2t.copy()
    neg[0] = -1   # maps draft 0 to target -1
    assert lib.dflash_check_d2t(neg.ctypes.data, 48, 200, ctypes.byref(inj)) == bdm.EINVAL
    assert lib.dflash_check_d2t(None, 48, 200, ctypes.byref(inj)) == bdm.EINVAL
    assert lib.dflash_check_d2t(d2t.ctypes.data, 48, 40, ctypes.byref(inj)) == bdm.EINVAL


def test_binding_check_d2t_matches_oracle():
    from block_draft_markov_amd import api
    from oracle import draft_step as O
    rng = np.random.default_rng(1)
    for _ in range(20):
        Vd, Vt = int(rng.integers(1, 60)), int(rng.integers(60, 120))
        t = rng.integers(0, Vt, size=Vd)
        d2t = t - np.arange(Vd)
        valid, inj = O.check_d2t(d2t, Vd, Vt)
        assert valid
        assert api.check_d2t(d2t, Vd, Vt) == inj


@pytest.mark.parametrize("src,kernel", [("lmhead.hip", "lmhead_dma_kernel"), ("dense.hip", "dense_lds_kernel")])
def test_m0_only_set_for_lds_dma(src, kernel):
    """The batched lm_head kernel and the LDS-staged dense walk kernel set m0 (a register
    the compiler reserves) in inline assembly right before each buffer_load ... lds.
    That is only sound while no compiler-generated code of the kernel relies on m0,
    which this checks in the gfx950 assembly: every line naming m0 is such a set, and
    the next line is an LDS-DMA load."""
    import re
    import shutil
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    from block_draft_markov_amd import build as B
    text = B.device_asm(src)
    kernels = re.findall(r"^(_Z\w*" + kernel + r"\w*):", text, re.M)
    assert kernels, f"no {kernel} in the assembly"
    for name in kernels:
        body = text[text.index(name + ":"):]
        body = body[:body.index(".Lfunc_end")]
        lines = [l.strip() for l in body.splitlines() if l.strip() and not l.strip().startswith(";")]
        for i, l in enumerate(lines):
            if re.search(r"\bm0\b", l):
                assert l.startswith("s_mov_b32 m0,"), f"{name}: m0 used by '{l}'"
                nxt = lines[i + 1]
                assert nxt.startswith("buffer_load_dwordx4") and nxt.endswith(" lds"), \
                    f"{name}: m0 set but followed by '{nxt}'"


def test_draft_argmax_validates(lib):
    d = dims()
    big = 1 << 40
    call = lambda **p: lib.dflash_draft_argmax(
        ctypes.byref(p.get("d", d)), p.get("hidden", FAKE), p.get("lm", FAKE), p.get("d2t", None),
        p.get("scale", 1.0), p.get("cap", 0.0), p.get("tok", FAKE), p.get("val", None), p.get("ws", FAKE),
        p.get("wsn", big), None)
    assert call(scale=0.0) == bdm.EINVAL and "out_scale" in err(lib)
    assert call(scale=-2.0) == bdm.EINVAL and "out_scale" in err(lib)
    assert call(scale=float("inf")) == bdm.EINVAL and "out_scale" in err(lib)
    assert call(scale=float("nan")) == bdm.EINVAL and "out_scale" in err(lib)
    assert call(cap=float("nan")) == bdm.EINVAL and "soft_cap" in err(lib)
    assert call(tok=None) == bdm.EINVAL and "tokens" in err(lib)
    assert call(hidden=None) == bdm.EINVAL and "hidden" in err(lib)
    assert call(d=dims(target_vocab=2000)) == bdm.EINVAL and "d2t" in err(lib)
    assert call(hidden=FAKE + 2) == bdm.EINVAL and "aligned" in err(lib)
    assert call(wsn=16) == bdm.EWORKSPACE
    assert call(d=dims(top_k=0)) == bdm.EINVAL and "top_k" in err(lib)


def test_draft_dense_validates(lib):
    d = dims()
    big = 1 << 40
    call = lambda **p: lib.dflash_draft_dense(
        ctypes.byref(p.get("d", d)), p.get("hidden", FAKE), p.get("lm", FAKE), p.get("d2t", None),
        p.get("tables", FAKE), p.get("last", FAKE), p.get("offs", None), p.get("scale", 1.0), p.get("cap", 0.0),
        p.get("tok", FAKE), p.get("val", None), p.get("ws", FAKE), p.get("wsn", big), None)
    assert call(scale=0.0) == bdm.EINVAL and "out_scale" in err(lib)
    assert call(scale=float("nan")) == bdm.EINVAL and "out_scale" in err(lib)
    assert call(cap=float("inf")) == bdm.EINVAL and "soft_cap" in err(lib)
    assert call(tables=None) == bdm.EINVAL and "tables" in err(lib)
    assert call(last=None) == bdm.EINVAL and "last_tok" in err(lib)
    assert call(tok=None) == bdm.EINVAL and "tokens" in err(lib)
    assert call(hidden=None) == bdm.EINVAL and "hidden" in err(lib)
    assert call(d=dims(target_vocab=2000)) == bdm.EINVAL and "d2t" in err(lib)
    assert call(lm=FAKE_ODD) == bdm.EINVAL and "aligned" in err(lib)
    assert call(d=dims(total_rows=5)) == bdm.EINVAL and "row_offsets" in err(lib)
    assert call(ws=None) == bdm.EWORKSPACE
    assert call(wsn=16) == bdm.EWORKSPACE
    assert call(d=dims(rank=0)) == bdm.EINVAL and "rank" in err(lib)


def test_sampled_entry_points_validate(lib):
    d = dims()
    big = 1 << 40
    blk = lambda **p: lib.dflash_draft_block_sampled(
        ctypes.byref(p.get("d", d)), p.get("hidden", FAKE), FAKE, None, FAKE, None, FAKE, None,
        p.get("uni", FAKE), p.get("temp", 1.0), p.get("tok", FAKE), p.get("sc", FAKE), None, p.get("ws", FAKE),
        p.get("wsn", big), None)
    assert blk(temp=0.0) == bdm.EINVAL and "temperature" in err(lib)
    assert blk(temp=-1.0) == bdm.EINVAL and "temperature" in err(lib)
    assert blk(temp=float("inf")) == bdm.EINVAL and "temperature" in err(lib)
    assert blk(temp=float("nan")) == bdm.EINVAL and "temperature" in err(lib)
    assert blk(uni=None) == bdm.EINVAL and "uniforms" in err(lib)
    assert blk(tok=None) == bdm.EINVAL and "tokens" in err(lib)
    assert blk(sc=None) == bdm.EINVAL and "scores" in err(lib)
    assert blk(d=dims(top_k=0)) == bdm.EINVAL and "top_k" in err(lib)
    assert blk(d=dims(total_rows=5)) == bdm.EINVAL and "row_offsets" in err(lib)
    assert blk(ws=None) == bdm.EWORKSPACE
    wlk = lambda **p: lib.dflash_walk_sampled(
        ctypes.byref(p.get("d", d)), FAKE, FAKE, FAKE, None, p.get("uni", FAKE), p.get("temp", 1.0),
        p.get("tok", FAKE), FAKE, None, None, None)
    assert wlk(temp=0.0) == bdm.EINVAL and "temperature" in err(lib)
    assert wlk(uni=None) == bdm.EINVAL and "uniforms" in err(lib)
    assert wlk(tok=None) == bdm.EINVAL and "tokens" in err(lib)
    assert wlk(d=dims(block_len=0, total_rows=0)) == bdm.EINVAL and "block_len" in err(lib)


def test_lattice_validates(lib):
    d = dims()
    big = 1 << 40
    call = lambda **p: lib.dflash_lattice(
        ctypes.byref(p.get("d", d)), p.get("tok", FAKE), p.get("un", FAKE), p.get("tables", FAKE),
        p.get("gate", None), p.get("hidden", None), p.get("last", FAKE), p.get("offs", None), p.get("out", FAKE),
        p.get("sc", FAKE), p.get("ws", FAKE), p.get("wsn", big), None)
    assert call(tok=None) == bdm.EINVAL and "cand_tok" in err(lib)
    assert call(un=None) == bdm.EINVAL and "unary" in err(lib)
    assert call(tables=None) == bdm.EINVAL and "tables" in err(lib)
    assert call(last=None) == bdm.EINVAL and "last_tok" in err(lib)
    assert call(out=None) == bdm.EINVAL and "tokens" in err(lib)
    assert call(sc=None) == bdm.EINVAL and "scores" in err(lib)
    # the gate reads the hidden states
    assert call(gate=FAKE) == bdm.EINVAL and "hidden" in err(lib)
    assert call(d=dims(walk=5)) == bdm.EINVAL and "walk" in err(lib)
    assert call(d=dims(total_rows=5)) == bdm.EINVAL and "row_offsets" in err(lib)
    assert call(ws=None) == bdm.EWORKSPACE
    assert call(wsn=16) == bdm.EWORKSPACE
    assert call(ws=FAKE_ODD) == bdm.EINVAL and "aligned" in err(lib)
    # no rows: nothing to launch
    d0 = dims(num_requests=0, total_rows=0)
    assert lib.dflash_lattice(ctypes.byref(d0), None, None, FAKE, None, None, None, None, None, None, FAKE,
                              lib.dflash_workspace_bytes(ctypes.byref(d0)), None) == bdm.OK


def test_lattice_noalloc_validates_before_touching_the_gpu(lib):
    from block_draft_markov_amd._lib import LATTICE_NOALLOC_MAX_BYTES
    call = lambda d, **p: lib.dflash_lattice_noalloc(
        ctypes.byref(d), p.get("tok", FAKE), p.get("un", FAKE), p.get("tables", FAKE), p.get("gate", None),
        p.get("hidden", None), p.get("last", FAKE), None, p.get("out", FAKE), p.get("sc", FAKE), None)
    # more rows than the static scratch holds at K = 64: rejected with the limit in the message
    rows = LATTICE_NOALLOC_MAX_BYTES // (64 * 64 * 4) + 1
    big = dims(num_requests=rows, block_len=1, total_rows=rows, draft_vocab=64, target_vocab=100, top_k=64)
    assert call(big) == bdm.EINVAL and "static scratch" in err(lib)
    fits = dims(num_requests=rows - 1, block_len=1, total_rows=rows - 1, draft_vocab=64, target_vocab=100, top_k=64)
    assert call(fits, tok=None) == bdm.EINVAL and "cand_tok" in err(lib)
    assert call(dims(), gate=FAKE) == bdm.EINVAL and "hidden" in err(lib)
    assert call(dims(walk=4)) == bdm.EINVAL and "walk" in err(lib)
    # no requests: nothing to launch, no device touched
    assert lib.dflash_lattice_noalloc(ctypes.byref(dims(num_requests=0, total_rows=0)), None, None, FAKE, None,
                                      None, None, None, None, None, None) == bdm.OK
    h = open(os.path.join(ROOT, "include", "dflash_draft.h")).read()
    assert f"DFLASH_LATTICE_NOALLOC_MAX_BYTES (16u << 20)" in h and LATTICE_NOALLOC_MAX_BYTES == 16 << 20


# ---------------------------------------------------------------- the binding's host checks
# The C ABI trusts sizes, so the binding checks every tensor before any call.
# CPU tensors suffice: shape and dtype checks come first, the device check last.

torch = pytest.importorskip("torch")


def _bf(*shape):
    return torch.zeros(shape, dtype=torch.int16)


def _step_args(M=6, H=64, Vd=1024, Vt=1024, r=16, R=2):
    return dict(hidden=_bf(M, H), lm_head_w=_bf(Vd, H), tables=torch.zeros((2, Vt, r)),
                last_tok=torch.zeros(R, dtype=torch.int64))


@pytest.mark.parametrize("change,exc,word", [
    (dict(lm_head_w=_bf(1024, 32)), ValueError, "lm_head"),                     # W narrower than H
    (dict(tables=torch.zeros((1, 1024, 16))), ValueError, "tables"),            # one table instead of two
    (dict(tables=torch.zeros((2, 1024, 16), dtype=torch.float64)), TypeError, "tables"),
    (dict(hidden=torch.zeros((6, 64))), TypeError, "hidden"),                  # fp32 hidden
    (dict(d2t=torch.zeros(1000, dtype=torch.int64)), ValueError, "d2t"),        # d2t of the wrong length
    (dict(gate_w=torch.zeros(32)), ValueError, "gate_w"),                       # gate of the wrong length
    (dict(last_tok=torch.zeros(2, dtype=torch.int32)), TypeError, "last_tok"),
    (dict(row_offsets=torch.zeros(2, dtype=torch.int32)), ValueError, "row_offsets"),   # needs R + 1 entries
    (dict(hidden=_bf(5, 64)), ValueError, "uniform blocks"),                    # 5 rows over 2 requests
    (dict(block_len=4), ValueError, "block_len"),                               # uniform blocks of 3
    (dict(out=(torch.zeros(5, dtype=torch.int64), torch.zeros(2))), ValueError, "tokens"),
    (dict(out=(torch.zeros(6, dtype=torch.int64), torch.zeros(2, dtype=torch.float64))), TypeError, "scores"),
    (dict(hidden=_bf(6, 64).t().contiguous().t()), ValueError, "contiguous"),
    (dict(), ValueError, "GPU"),                                               # shapes fine: CPU tensors refused
])
def test_binding_rejects_mismatched_tensors(change, exc, word):
    from block_draft_markov_amd import api
    args = _step_args()
    kw = dict(top_k=8)
    for k, v in change.items():
        (args if k in args else kw)[k] = v
    with pytest.raises(exc, match=word):
        api.draft_block(args.pop("hidden"), args.pop("lm_head_w"), args.pop("tables"), args.pop("last_tok"), **kw)


def test_binding_ragged_offsets_checked_on_the_host():
    from block_draft_markov_amd import api
    a = _step_args(M=7)
    off = torch.tensor([0, 5, 7], dtype=torch.int32)
    with pytest.raises(ValueError, match="longer than block_len"):
        api.draft_block(a["hidden"], a["lm_head_w"], a["tables"], a["last_tok"], top_k=8, row_offsets=off,
                        block_len=3)
    with pytest.raises(ValueError, match="non-decreasing"):
        api.draft_block(a["hidden"], a["lm_head_w"], a["tables"], a["last_tok"], top_k=8,
                        row_offsets=torch.tensor([0, 5, 4], dtype=torch.int32))
    with pytest.raises(ValueError, match="exceeds"):
        api.draft_block(a["hidden"], a["lm_head_w"], a["tables"], a["last_tok"], top_k=8,
                        row_offsets=torch.tensor([0, 5, 9], dtype=torch.int32))
    # well-formed offsets pass the host checks and stop only at the device check
    with pytest.raises(ValueError, match="GPU"):
        api.draft_block(a["hidden"], a["lm_head_w"], a["tables"], a["last_tok"], top_k=8, row_offsets=off)


def test_binding_stage_entry_points_check_shapes():
    from block_draft_markov_amd import api
    tok = torch.zeros((6, 8), dtype=torch.int64)
    un = torch.zeros((6, 8))
    tables = torch.zeros((2, 100, 16))
    last = torch.zeros(2, dtype=torch.int64)
    with pytest.raises(ValueError, match="unary"):
        api.lattice(tok, torch.zeros((6, 7)), tables, last)
    with pytest.raises(ValueError, match="hidden is required"):
        api.lattice(tok, un, tables, last, gate_w=torch.zeros(64))
    with pytest.raises(ValueError, match="gate_w"):
        api.lattice(tok, un, tables, last, gate_w=torch.zeros(32), hidden=_bf(6, 64))
    with pytest.raises(ValueError, match="pair"):
        api.walk(tok, un, torch.zeros((6, 8, 7)), 2)
    with pytest.raises(ValueError, match="uniforms"):
        api.walk_sampled(tok, un, torch.zeros((6, 8, 8)), 2, torch.zeros(5, dtype=torch.float64))
    with pytest.raises(ValueError, match="lse"):
        api.topk(torch.zeros((6, 1024)), torch.zeros(5), 8)
    with pytest.raises(ValueError, match="d2t"):
        api.topk(torch.zeros((6, 1024)), torch.zeros(6), 8, d2t=torch.zeros(1023, dtype=torch.int64))
    with pytest.raises(ValueError, match="out"):
        api.lm_head(_bf(6, 64), _bf(1024, 64), out=torch.zeros((6, 1000)))
    with pytest.raises(ValueError, match="lm_head"):
        api.draft_argmax(_bf(6, 64), _bf(1024, 48))
    with pytest.raises(ValueError, match="values"):
        api.draft_argmax(_bf(6, 64), _bf(1024, 64), out=(torch.zeros(6, dtype=torch.int64), torch.zeros(4)))
    with pytest.raises(ValueError, match="tables"):
        api.draft_dense(_bf(6, 64), _bf(1024, 64), torch.zeros((3, 1024, 16)), last)
    with pytest.raises(TypeError, match="uniforms"):
        api.draft_block_sampled(_bf(6, 64), _bf(1024, 64), torch.zeros((2, 1024, 16)), last,
                                torch.zeros(6, dtype=torch.float32), top_k=8)
