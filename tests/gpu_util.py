"""Helpers of the GPU parity tests: upload seeded inputs, pack oracle values for
the stage entry points, and the comparison rules.  Imports the oracle (tests
only) and the binding; never the other way round."""
import sys

import numpy as np
import pytest
import torch

from oracle import draft_step as O


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import block_draft_markov_amd as bdm
    bdm.load()   # raises when the HIP library is missing


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def dev(x, dtype=None):
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def upload(inp):
    """numpy DraftInputs -> dict of device tensors."""
    return dict(
        hidden=dev_bf16(inp.hidden),
        lm_head=dev_bf16(inp.lm_head),
        tables=dev(inp.tables),
        last_tok=dev(inp.last_tok),
        d2t=dev(inp.d2t),
        gate_w=dev(inp.gate_w),
        row_offsets=dev(inp.row_offsets),
    )


def pack_pair(S_all, offsets, M, K):
    """Oracle transition matrices -> the [M, K, K] fp32 layout of dflash_pair_scores."""
    pair = np.zeros((M, K, K), np.float64)
    for r, S in enumerate(S_all):
        a = int(offsets[r])
        for p, s in enumerate(S):
            if p == 0:
                pair[a, 0, :] = s[0]
            else:
                pair[a + p] = s
    return pair


def offsets_of(R, M, row_offsets):
    if row_offsets is not None:
        return np.asarray(row_offsets, np.int64)
    L = M // R if R else 0
    return np.arange(R + 1, dtype=np.int64) * L


def logits_tol(z_orc_row: np.ndarray) -> float:
    """Logit tolerance of a row: 1e-3 * max |z| of the oracle row."""
    return 1e-3 * float(np.max(np.abs(z_orc_row)))


def check_topk_row(gpu_idx: np.ndarray, z_orc_row: np.ndarray, K: int):
    """Top-K set rule.  Returns 'exact' or 'exempt'; raises AssertionError on a violation.

    With tau = 1e-3 max|z| and v_1 >= v_2 >= ... the oracle's sorted row: if
    v_K - v_{K+1} >= tau the GPU slot set must equal the oracle's (and the
    slots be in logit order up to 1e-5 max|z|).
    Otherwise every id with z > v_{K+1} + tau must be among the GPU slots and
    every GPU slot must have z >= v_K - tau.
    """
    order = O.topk_slots(z_orc_row, min(K + 1, z_orc_row.size))
    tau = logits_tol(z_orc_row)
    vK = z_orc_row[order[K - 1]]
    vK1 = z_orc_row[order[K]] if z_orc_row.size > K else -np.inf
    fine = 1e-2 * tau    # ~1e-5 max|z|: well above the fp32 error of the GPU logits (~1e-6 relative)
    # slot order: non-increasing in the oracle's logits up to the fine tolerance
    zg = z_orc_row[gpu_idx]
    assert np.all(zg[:-1] >= zg[1:] - fine), "GPU slots are not in logit order"
    if vK - vK1 >= tau:
        assert set(gpu_idx.tolist()) == set(order[:K].tolist()), "Top-K set differs outside the tie tolerance"
        return "exact"
    # Stricter than the bar: fp32 logits are within ~1e-6 relative, so a gap of
    # 1e-5 max|z| already decides the set; the order within it may still differ
    # only where two candidates are that close.
    if vK - vK1 >= fine:
        assert set(gpu_idx.tolist()) == set(order[:K].tolist()), "Top-K set differs at a gap above 1e-5 max|z|"
    must = np.flatnonzero(z_orc_row > vK1 + tau)
    assert set(must) <= set(gpu_idx.tolist())
    assert np.all(z_orc_row[gpu_idx] >= vK - tau)
    assert len(set(gpu_idx.tolist())) == K
    return "exempt"
