"""Seeded synthetic inputs for the draft step (block of draft hidden states ->
drafted tokens).

This module only draws random numbers and lays them out; it holds none of the
draft step's arithmetic.  Both the CPU oracle (``oracle/``) and the HIP path
(``block_draft_markov_amd``) are fed from here, so that they see identical
bytes.

Workload shapes follow the pages: block lengths 7 and 15 are the
``num_assistant_tokens`` values of the validation tables of the openvino.genai
page ("Add DSpark and DFlash v2 drafts ...", Validation); the pruned draft
vocabulary of 114,688 out of 248,100 target tokens, mapped through d2t as
"draft token i -> target token i + d2t[i]", is from the optimum-intel page
"Support MiniCPM-OCR-1.0-DSpark" (What does this PR do?).  Real draft logits
and checkpoints are not used: weights and hidden states are random.

Conventions (stated once, used everywhere):
  * "N(0, s)" means a normal with standard deviation s.
  * lm_head and hidden states are drawn in fp32 and rounded to bf16 with
    round-to-nearest-even; they are handed around as uint16 bit patterns.
  * tables are fp32 [2, V_t, r]: index 0 is A (the "previous token" table),
    index 1 is B (the "next token" table).
  * Large arrays are drawn in chunks of 2**22 elements; chunk c of stream s
    uses PCG64(SeedSequence([seed, s, c])), so the bytes do not depend on the
    number of threads used to draw them.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

_CHUNK = 1 << 22


@dataclasses.dataclass(frozen=True)
class Shape:
    """Sizes of one draft-step workload.

    R requests, each a block of L rows (M = R*L packed rows), hidden size H,
    draft vocabulary V_d, target vocabulary V_t, Top-K K, table rank r.
    """
    name: str
    R: int
    L: int
    H: int
    Vd: int
    Vt: int
    K: int
    r: int
    gated: bool = False
    pruned: bool = False
    table_std: float = 0.25
    seed: int = 0
    weight_seed: int = 0   # seed of lm_head / tables / gate (shared by shapes of one model)
    subset_seed: int = 0   # seed of the pruned-vocabulary subset

    @property
    def M(self) -> int:
        return self.R * self.L


def _k(vd: int) -> int:
    # K of the candidate scorer is at most one candidate per draft token:
    # min(64, draft vocabulary) (optimum-intel page "Support MiniCPM-OCR-1.0-DSpark",
    # What does this PR do?, Markov head bullet).
    return min(64, vd)


SHAPES = {
    # 1 request, L=5, H=64, V=1024, K=8, r=16; tables N(0, 0.02)
    "tiny": Shape("tiny", 1, 5, 64, 1024, 1024, 8, 16, table_std=0.02, seed=0, weight_seed=0),
    # as tiny, with tables N(0, 0.5) so that the pairwise term changes the walk
    "tiny_stress": Shape("tiny_stress", 1, 5, 64, 1024, 1024, 8, 16, table_std=0.5, seed=2000,
                         weight_seed=2000),
    # Qwen3-4B-shaped DSpark block, one request
    "qwen3_4b_1": Shape("qwen3_4b_1", 1, 7, 2560, 151936, 151936, 64, 256, seed=1, weight_seed=1),
    # Qwen3-4B-shaped batch: 32 requests x 7 rows, same weights as the single request
    "qwen3_4b_32": Shape("qwen3_4b_32", 32, 7, 2560, 151936, 151936, 64, 256, seed=2, weight_seed=1),
    # 27B-shaped DFlash v2 block with gated transitions
    "dflash2_27b": Shape("dflash2_27b", 16, 15, 5120, 248100, 248100, 64, 256, gated=True, seed=3,
                         weight_seed=3),
    # pruned-vocabulary DSpark draft: 114,688 draft tokens mapped into 248,100 target tokens
    "pruned_ocr": Shape("pruned_ocr", 16, 15, 2048, 114688, 248100, 64, 256, pruned=True, seed=4,
                        weight_seed=4, subset_seed=5),
}


def custom_shape(name="custom", *, R, L, H, Vd, Vt=None, K=None, r, gated=False, pruned=False,
                 table_std=0.25, seed=0, weight_seed=None, subset_seed=None) -> Shape:
    Vt = Vd if Vt is None else Vt
    K = _k(Vd) if K is None else K
    return Shape(name, R, L, H, Vd, Vt, K, r, gated, pruned, table_std, seed,
                 seed if weight_seed is None else weight_seed,
                 seed + 1 if subset_seed is None else subset_seed)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal_f32(n: int, std: float, seed: int, stream: int) -> np.ndarray:
    """n draws of N(0, std) in fp32, chunked so the result is thread-count independent."""
    out = np.empty(n, dtype=np.float32)
    chunks = [(c, c * _CHUNK, min(n, (c + 1) * _CHUNK)) for c in range((n + _CHUNK - 1) // _CHUNK)]

    def fill(job):
        c, lo, hi = job
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, c])))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            np.multiply(out[lo:hi], np.float32(std), out=out[lo:hi])

    if len(chunks) <= 1:
        for j in chunks:
            fill(j)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, chunks))
    return out


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs here are finite, so the NaN case is not handled.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 24

    def conv(lo):
        u = flat[lo:lo + step].view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        out[lo:lo + step] = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)

    starts = list(range(0, flat.size, step))
    if len(starts) <= 1:
        for s in starts:
            conv(s)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(conv, starts))
    return out.reshape(x.shape)


def bf16_bits(shape, std: float, seed: int, stream: int) -> np.ndarray:
    n = int(np.prod(shape))
    return round_to_bf16_bits(_normal_f32(n, std, seed, stream)).reshape(shape)


# stream ids: one per tensor, so that tensors are independent
_S_HIDDEN, _S_LMHEAD, _S_TABLE_A, _S_TABLE_B, _S_GATE, _S_LAST = 1, 2, 3, 4, 5, 6


@dataclasses.dataclass
class DraftInputs:
    """One synthetic draft-step workload, host side (numpy)."""
    shape: Shape
    hidden: np.ndarray            # uint16 bf16 bits [M, H]
    lm_head: np.ndarray           # uint16 bf16 bits [V_d, H] (nn.Linear layout)
    tables: np.ndarray            # float32 [2, V_t, r]  (A = prev, B = next)
    last_tok: np.ndarray          # int64 [R]
    d2t: Optional[np.ndarray]     # int64 [V_d] or None
    gate_w: Optional[np.ndarray]  # float32 [H] or None
    row_offsets: Optional[np.ndarray] = None  # int32 [R+1] or None (uniform blocks)

    @property
    def M(self) -> int:
        return int(self.hidden.shape[0])


def make_inputs(shape: Shape, *, with_lm_head: bool = True) -> DraftInputs:
    """Draw the inputs of ``shape`` (see the module docstring for the recipe)."""
    s = shape
    hidden = bf16_bits((s.M, s.H), 1.0, s.seed, _S_HIDDEN)
    lm_head = (bf16_bits((s.Vd, s.H), 0.02, s.weight_seed, _S_LMHEAD) if with_lm_head
               else np.zeros((0, s.H), np.uint16))
    d2t = None
    if s.pruned:
        sub = np.random.Generator(np.random.PCG64(s.subset_seed)).permutation(s.Vt)[: s.Vd]
        d2t = (sub - np.arange(s.Vd)).astype(np.int64)
        rows = sub
    else:
        rows = None
    tables = np.zeros((2, s.Vt, s.r), dtype=np.float32)
    nrows = s.Vt if rows is None else s.Vd
    a = _normal_f32(nrows * s.r, s.table_std, s.weight_seed, _S_TABLE_A).reshape(nrows, s.r)
    b = _normal_f32(nrows * s.r, s.table_std, s.weight_seed, _S_TABLE_B).reshape(nrows, s.r)
    if rows is None:
        tables[0], tables[1] = a, b
    else:
        # the next-token table is zero for target tokens outside the draft vocabulary
        tables[0, rows], tables[1, rows] = a, b
    gate_w = None
    if s.gated:
        gate_w = _normal_f32(s.H, 1.0 / np.sqrt(s.H), s.weight_seed, _S_GATE)
    last_tok = np.random.Generator(np.random.PCG64([s.seed, _S_LAST])).integers(
        0, s.Vt, size=s.R, dtype=np.int64)
    return DraftInputs(s, hidden, lm_head, tables, last_tok, d2t, gate_w)


def ragged_offsets(lengths) -> np.ndarray:
    """row_offsets [R+1] (int32) of packed blocks with the given lengths."""
    off = np.zeros(len(lengths) + 1, dtype=np.int32)
    off[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return off


def dyadic(shape, *, lo: int, hi: int, exp: int, seed: int) -> np.ndarray:
    """Small integers in [lo, hi] times 2**-exp, as float32.

    Sums and products of a few such values are exact in fp32 and fp64, which
    makes exact ties reproducible on both sides.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    return (g.integers(lo, hi + 1, size=shape).astype(np.float32) * np.float32(2.0 ** -exp))
