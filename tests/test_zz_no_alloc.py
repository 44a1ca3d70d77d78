"""dflash_lattice_noalloc (S in the library's static device scratch) against
dflash_lattice (S in a caller workspace), through the C ABI: identical tokens
and scores, bit for bit (the same kernels run on the same inputs), on two calls
in a row, the second with a smaller input that leaves the first call's values
in the scratch beyond its own."""
import numpy as np
import pytest
import torch

import draft_inputs as di
from tests.gpu_util import dev, dev_bf16, record, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _case(R, L, K, Vt, r, gated, seed, ragged=None):
    rng = np.random.default_rng(seed)
    lengths = ragged if ragged is not None else [L] * R
    off = di.ragged_offsets(lengths)
    M = int(off[-1])
    tok = rng.integers(0, Vt, size=(M, K)).astype(np.int64)
    un = (-np.sort(-rng.standard_normal((M, K)), axis=1) - 4.0).astype(np.float32)
    tables = (rng.standard_normal((2, Vt, r)) * 0.25).astype(np.float32)
    hidden = di.round_to_bf16_bits(rng.standard_normal((M, 64)).astype(np.float32))
    w = (rng.standard_normal(64) / 8).astype(np.float32) if gated else None
    last = rng.integers(0, Vt, size=R).astype(np.int64)
    return dict(cand_tok=dev(tok), unary=dev(un), tables=dev(tables), last_tok=dev(last), gate_w=dev(w),
                hidden=dev_bf16(hidden) if gated else None,
                row_offsets=dev(off) if ragged is not None else None, block_len=max(lengths))


def _both(c, walk):
    from block_draft_markov_amd import api
    args = (c["cand_tok"], c["unary"], c["tables"], c["last_tok"])
    kw = dict(gate_w=c["gate_w"], hidden=c["hidden"], row_offsets=c["row_offsets"], block_len=c["block_len"],
              walk=walk)
    t1, s1 = api.lattice(*args, **kw)
    t2, s2 = api.lattice_noalloc(*args, **kw)
    torch.cuda.synchronize()
    return t1.cpu().numpy(), s1.cpu().numpy(), t2.cpu().numpy(), s2.cpu().numpy()


@pytest.mark.parametrize("walk", ["viterbi", "greedy"])
def test_noalloc_lattice_matches_workspace_lattice(walk):
    big = _case(R=16, L=15, K=64, Vt=5000, r=256, gated=True, seed=1)      # the 27B block shape: 3.9 MB of S
    small = _case(R=3, L=4, K=16, Vt=700, r=32, gated=False, seed=2, ragged=[4, 0, 3])
    for name, c in (("big", big), ("small", small)):
        t1, s1, t2, s2 = _both(c, walk)
        assert np.array_equal(t1, t2), f"{name}: tokens differ"
        assert np.array_equal(s1, s2), f"{name}: scores differ"
        record(f"noalloc_{name}_{walk}", rows=int(t1.size), requests=int(s1.size))
    # the request without rows scores 0
    assert s2[1] == 0.0


def test_noalloc_lattice_rejects_more_than_its_scratch():
    from block_draft_markov_amd import api, DFlashError
    from block_draft_markov_amd._lib import LATTICE_NOALLOC_MAX_BYTES
    c = _case(R=2, L=1, K=64, Vt=100, r=8, gated=False, seed=3)
    rows = LATTICE_NOALLOC_MAX_BYTES // (64 * 64 * 4) + 1
    tok = torch.zeros((rows, 64), dtype=torch.int64, device="cuda")
    un = torch.zeros((rows, 64), dtype=torch.float32, device="cuda")
    last = torch.zeros(rows, dtype=torch.int64, device="cuda")
    with pytest.raises(DFlashError, match="static scratch"):
        api.lattice_noalloc(tok, un, c["tables"], last, block_len=1)
