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


def check_topk_row(gpu_idx: np.ndarray, z_orc_row: np.ndarray, K: int) -> str:
    """Top-K set rule for one row.  Raises AssertionError on a violation; returns

      'same'    the GPU slots are the oracle's slots, in the oracle's order;
      'reorder' the same K ids, in another order (only ids within the fine
                tolerance of each other may swap);
      'differs' another set: allowed only where the oracle's K-th and (K+1)-th
                logits are closer than tau = 1e-3 max|z| (the Top-K boundary
                exemption), and then every id with z > v_{K+1} + tau must be
                among the GPU slots and every GPU slot must have z >= v_K - tau.

    Stricter than the bar: the fp32 logits are within ~1e-6 relative, so a gap
    of 1e-5 max|z| (`fine`) already decides the set.
    """
    order = O.topk_slots(z_orc_row, min(K + 1, z_orc_row.size))
    tau = logits_tol(z_orc_row)
    vK = z_orc_row[order[K - 1]]
    vK1 = z_orc_row[order[K]] if z_orc_row.size > K else -np.inf
    fine = 1e-2 * tau
    ids = gpu_idx.tolist()
    assert len(set(ids)) == K, "duplicate GPU slots"
    zg = z_orc_row[gpu_idx]
    assert np.all(zg[:-1] >= zg[1:] - fine), "GPU slots are not in logit order"
    same_set = set(ids) == set(order[:K].tolist())
    if vK - vK1 >= fine:
        assert same_set, f"Top-K set differs at a boundary gap of {vK - vK1:.3e} (>= {fine:.3e})"
    if not same_set:
        must = np.flatnonzero(z_orc_row > vK1 + tau)
        assert set(must.tolist()) <= set(ids)
        assert np.all(zg >= vK - tau)
        return "differs"
    return "same" if np.array_equal(gpu_idx, order[:K]) else "reorder"


def record(test: str, **counts) -> None:
    """Append a parity record (a JSON line) to $PARITY_LOG when that variable is set,
    so that exact and exempt counts survive a quiet pytest run."""
    import json
    import os
    path = os.environ.get("PARITY_LOG")
    say(f"  {test}: {counts}")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(dict(test=test, **counts)) + "\n")
