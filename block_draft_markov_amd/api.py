"""Python binding of the draft-step library: argument marshalling only.

Every function takes torch tensors that already live on the GPU, allocates
its outputs (and a workspace) with torch, and calls the C entry point of the
same name on torch's current stream.  No arithmetic of the draft step happens
here.  bf16 inputs may be torch.bfloat16 or 16-bit integer tensors holding
bf16 bit patterns.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from ._lib import (DFlashError, Dims, WALK_GREEDY, WALK_VITERBI, check, load)

__all__ = ["Dims", "DFlashError", "make_dims", "workspace_bytes", "logits_stride", "draft_block", "lm_head",
           "row_lse", "topk", "pair_scores", "walk", "check_d2t", "Workspace"]

_WALKS = {"viterbi": WALK_VITERBI, "greedy": WALK_GREEDY, WALK_VITERBI: WALK_VITERBI, WALK_GREEDY: WALK_GREEDY}


def make_dims(*, R: int, L: int, M: int, H: int, Vd: int, Vt: Optional[int] = None, K: int, r: int = 1,
              walk="viterbi") -> Dims:
    return Dims(int(R), int(L), int(M), int(H), int(Vd), int(Vd if Vt is None else Vt), int(K), int(r),
                _WALKS[walk])


def workspace_bytes(d: Dims) -> int:
    n = load().dflash_workspace_bytes(ctypes.byref(d))
    if n == 0:
        raise DFlashError(-1, load().dflash_last_error().decode())
    return int(n)


def logits_stride(Vd: int) -> int:
    return int(load().dflash_logits_stride(int(Vd)))


class Workspace:
    """A reusable device workspace (grown on demand, 256-byte aligned)."""

    def __init__(self, device=None):
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self._buf = None

    def get(self, nbytes: int) -> Tuple[int, int]:
        if self._buf is None or self._buf.numel() < nbytes + 256:
            self._buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        base = self._buf.data_ptr()
        aligned = (base + 255) // 256 * 256
        return aligned, nbytes


_default_ws = {}


def _ws(ws: Optional[Workspace], device) -> Workspace:
    if ws is not None:
        return ws
    key = torch.device(device).index
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr() if t.numel() else None


def _bf16(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 (torch.bfloat16 or 16-bit bit patterns), got {t.dtype}")
    return t


def _expect(t: Optional[torch.Tensor], dtype, name: str):
    if t is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def draft_block(hidden: torch.Tensor, lm_head_w: torch.Tensor, tables: torch.Tensor, last_tok: torch.Tensor, *,
                top_k: int, d2t: Optional[torch.Tensor] = None, gate_w: Optional[torch.Tensor] = None,
                row_offsets: Optional[torch.Tensor] = None, block_len: Optional[int] = None, walk="viterbi",
                workspace: Optional[Workspace] = None, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """The whole draft step: (tokens int64 [M], scores fp32 [R])."""
    _bf16(hidden, "hidden"), _bf16(lm_head_w, "lm_head")
    _expect(tables, torch.float32, "tables"), _expect(last_tok, torch.int64, "last_tok")
    _expect(d2t, torch.int64, "d2t"), _expect(gate_w, torch.float32, "gate_w")
    _expect(row_offsets, torch.int32, "row_offsets")
    M, H = hidden.shape
    Vd = lm_head_w.shape[0]
    Vt, r = tables.shape[1], tables.shape[2]
    R = last_tok.shape[0]
    L = block_len if block_len is not None else (M // R if R else 1)
    d = make_dims(R=R, L=L, M=M, H=H, Vd=Vd, Vt=Vt, K=top_k, r=r, walk=walk)
    dev = hidden.device
    if out is None:
        tokens = torch.empty(M, dtype=torch.int64, device=dev)
        scores = torch.empty(R, dtype=torch.float32, device=dev)
    else:
        tokens, scores = out
    wsp, wsn = _ws(workspace, dev).get(workspace_bytes(d))
    check(load().dflash_draft_block(ctypes.byref(d), _ptr(hidden), _ptr(lm_head_w), _ptr(d2t), _ptr(tables),
                                    _ptr(gate_w), _ptr(last_tok), _ptr(row_offsets), _ptr(tokens), _ptr(scores),
                                    wsp, wsn, _stream(dev)))
    return tokens, scores


def draft_block_sampled(hidden: torch.Tensor, lm_head_w: torch.Tensor, tables: torch.Tensor,
                        last_tok: torch.Tensor, uniforms: torch.Tensor, *, top_k: int, temperature: float = 1.0,
                        d2t: Optional[torch.Tensor] = None, gate_w: Optional[torch.Tensor] = None,
                        row_offsets: Optional[torch.Tensor] = None, block_len: Optional[int] = None,
                        workspace: Optional[Workspace] = None, with_q: bool = True):
    """The whole step with the sampled walk: (tokens int64 [M], scores fp32 [R], q float64 [M, K] or None)."""
    _bf16(hidden, "hidden"), _bf16(lm_head_w, "lm_head")
    _expect(tables, torch.float32, "tables"), _expect(last_tok, torch.int64, "last_tok")
    _expect(d2t, torch.int64, "d2t"), _expect(gate_w, torch.float32, "gate_w")
    _expect(row_offsets, torch.int32, "row_offsets"), _expect(uniforms, torch.float64, "uniforms")
    M, H = hidden.shape
    Vd = lm_head_w.shape[0]
    Vt, r = tables.shape[1], tables.shape[2]
    R = last_tok.shape[0]
    L = block_len if block_len is not None else (M // R if R else 1)
    d = make_dims(R=R, L=L, M=M, H=H, Vd=Vd, Vt=Vt, K=top_k, r=r)
    dev = hidden.device
    tokens = torch.empty(M, dtype=torch.int64, device=dev)
    scores = torch.empty(R, dtype=torch.float32, device=dev)
    q = torch.empty((M, top_k), dtype=torch.float64, device=dev) if with_q else None
    wsp, wsn = _ws(workspace, dev).get(workspace_bytes(d))
    check(load().dflash_draft_block_sampled(ctypes.byref(d), _ptr(hidden), _ptr(lm_head_w), _ptr(d2t), _ptr(tables),
                                            _ptr(gate_w), _ptr(last_tok), _ptr(row_offsets), _ptr(uniforms),
                                            float(temperature), _ptr(tokens), _ptr(scores), _ptr(q), wsp, wsn,
                                            _stream(dev)))
    return tokens, scores, q


def draft_argmax(hidden: torch.Tensor, lm_head_w: torch.Tensor, *, d2t: Optional[torch.Tensor] = None,
                 target_vocab: Optional[int] = None, out_scale: float = 1.0, soft_cap: float = 0.0,
                 workspace: Optional[Workspace] = None, with_values: bool = True,
                 out: Optional[Tuple[torch.Tensor, Optional[torch.Tensor]]] = None):
    """Head-less draft step: (tokens int64 [M], winning scaled/capped logits fp32 [M] or None)."""
    _bf16(hidden, "hidden"), _bf16(lm_head_w, "lm_head"), _expect(d2t, torch.int64, "d2t")
    M, H = hidden.shape
    Vd = lm_head_w.shape[0]
    Vt = target_vocab if target_vocab is not None else Vd
    d = make_dims(R=M, L=1, M=M, H=H, Vd=Vd, Vt=Vt, K=min(64, Vd))
    dev = hidden.device
    if out is None:
        tokens = torch.empty(M, dtype=torch.int64, device=dev)
        values = torch.empty(M, dtype=torch.float32, device=dev) if with_values else None
    else:
        tokens, values = out
    wsp, wsn = _ws(workspace, dev).get(workspace_bytes(d))
    check(load().dflash_draft_argmax(ctypes.byref(d), _ptr(hidden), _ptr(lm_head_w), _ptr(d2t), float(out_scale),
                                     float(soft_cap), _ptr(tokens), _ptr(values), wsp, wsn, _stream(dev)))
    return tokens, values


def draft_dense(hidden: torch.Tensor, lm_head_w: torch.Tensor, tables: torch.Tensor, last_tok: torch.Tensor, *,
                d2t: Optional[torch.Tensor] = None, row_offsets: Optional[torch.Tensor] = None,
                block_len: Optional[int] = None, out_scale: float = 1.0, soft_cap: float = 0.0,
                workspace: Optional[Workspace] = None, with_values: bool = True,
                out: Optional[Tuple[torch.Tensor, Optional[torch.Tensor]]] = None):
    """Dense Markov walk: (tokens int64 [M], winning biased values fp32 [M] or None)."""
    _bf16(hidden, "hidden"), _bf16(lm_head_w, "lm_head")
    _expect(tables, torch.float32, "tables"), _expect(last_tok, torch.int64, "last_tok")
    _expect(d2t, torch.int64, "d2t"), _expect(row_offsets, torch.int32, "row_offsets")
    M, H = hidden.shape
    Vd = lm_head_w.shape[0]
    Vt, r = tables.shape[1], tables.shape[2]
    R = last_tok.shape[0]
    L = block_len if block_len is not None else (M // R if R else 1)
    d = make_dims(R=R, L=L, M=M, H=H, Vd=Vd, Vt=Vt, K=min(64, Vd), r=r)
    dev = hidden.device
    if out is None:
        tokens = torch.empty(M, dtype=torch.int64, device=dev)
        values = torch.empty(M, dtype=torch.float32, device=dev) if with_values else None
    else:
        tokens, values = out
    wsp, wsn = _ws(workspace, dev).get(workspace_bytes(d))
    check(load().dflash_draft_dense(ctypes.byref(d), _ptr(hidden), _ptr(lm_head_w), _ptr(d2t), _ptr(tables),
                                    _ptr(last_tok), _ptr(row_offsets), float(out_scale), float(soft_cap),
                                    _ptr(tokens), _ptr(values), wsp, wsn, _stream(dev)))
    return tokens, values


def lm_head(hidden: torch.Tensor, lm_head_w: torch.Tensor, *, workspace: Optional[Workspace] = None,
            with_lse: bool = True, out: Optional[torch.Tensor] = None):
    """Part 1: (logits fp32 [M, V_d] (a view of rows of stride dflash_logits_stride), lse fp32 [M] or None)."""
    _bf16(hidden, "hidden"), _bf16(lm_head_w, "lm_head")
    M, H = hidden.shape
    Vd = lm_head_w.shape[0]
    d = make_dims(R=M, L=1, M=M, H=H, Vd=Vd, K=min(64, Vd))
    ldz = logits_stride(Vd)
    dev = hidden.device
    z = torch.empty((M, ldz), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty(M, dtype=torch.float32, device=dev) if with_lse else None
    wsp, wsn = _ws(workspace, dev).get(workspace_bytes(d))
    check(load().dflash_lm_head(ctypes.byref(d), _ptr(hidden), _ptr(lm_head_w), _ptr(z), ldz, _ptr(lse), wsp, wsn,
                                _stream(dev)))
    return z[:, :Vd], lse


def _rows(logits: torch.Tensor):
    """(M, V_d, row stride) of a logits tensor whose rows are contiguous."""
    if logits.dtype != torch.float32 or not logits.is_cuda or logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be a CUDA float32 [M, V] tensor with contiguous rows")
    M, Vd = logits.shape
    return M, Vd, (logits.stride(0) if M > 0 else Vd + (-Vd) % 4)


def row_lse(logits: torch.Tensor) -> torch.Tensor:
    M, Vd, ldz = _rows(logits)
    d = make_dims(R=M, L=1, M=M, H=8, Vd=Vd, K=min(64, Vd))
    lse = torch.empty(M, dtype=torch.float32, device=logits.device)
    check(load().dflash_row_lse(ctypes.byref(d), logits.data_ptr() if M else None, ldz, _ptr(lse),
                                _stream(logits.device)))
    return lse


def topk(logits: torch.Tensor, lse: torch.Tensor, top_k: int, *, d2t: Optional[torch.Tensor] = None,
         target_vocab: Optional[int] = None, workspace: Optional[Workspace] = None):
    """Part 2: (cand_idx int32 [M, K], cand_tok int64 [M, K], unary fp32 [M, K])."""
    _expect(lse, torch.float32, "lse"), _expect(d2t, torch.int64, "d2t")
    M, Vd, ldz = _rows(logits)
    d = make_dims(R=M, L=1, M=M, H=8, Vd=Vd, Vt=target_vocab, K=top_k)
    dev = logits.device
    idx = torch.empty((M, top_k), dtype=torch.int32, device=dev)
    tok = torch.empty((M, top_k), dtype=torch.int64, device=dev)
    un = torch.empty((M, top_k), dtype=torch.float32, device=dev)
    wsp, wsn = _ws(workspace, dev).get(workspace_bytes(d))
    check(load().dflash_topk(ctypes.byref(d), logits.data_ptr() if M else None, ldz, _ptr(lse), _ptr(d2t),
                             _ptr(idx), _ptr(tok), _ptr(un), wsp, wsn, _stream(dev)))
    return idx, tok, un


def pair_scores(cand_tok: torch.Tensor, tables: torch.Tensor, last_tok: torch.Tensor, *,
                gate_w: Optional[torch.Tensor] = None, hidden: Optional[torch.Tensor] = None,
                row_offsets: Optional[torch.Tensor] = None, block_len: Optional[int] = None) -> torch.Tensor:
    """Part 3: pair fp32 [M, K, K]."""
    _expect(cand_tok, torch.int64, "cand_tok"), _expect(tables, torch.float32, "tables")
    _expect(last_tok, torch.int64, "last_tok"), _expect(gate_w, torch.float32, "gate_w")
    _expect(row_offsets, torch.int32, "row_offsets")
    M, K = cand_tok.shape
    R = last_tok.shape[0]
    Vt, r = tables.shape[1], tables.shape[2]
    L = block_len if block_len is not None else (M // R if R else 1)
    H = hidden.shape[1] if hidden is not None else 8
    d = make_dims(R=R, L=L, M=M, H=H, Vd=max(K, 1), Vt=Vt, K=K, r=r)
    pair = torch.empty((M, K, K), dtype=torch.float32, device=cand_tok.device)
    check(load().dflash_pair_scores(ctypes.byref(d), _ptr(cand_tok), _ptr(tables), _ptr(gate_w), _ptr(hidden),
                                    _ptr(last_tok), _ptr(row_offsets), _ptr(pair), _stream(cand_tok.device)))
    return pair


def walk(cand_tok: torch.Tensor, unary: torch.Tensor, pair: torch.Tensor, R: int, *,
         row_offsets: Optional[torch.Tensor] = None, block_len: Optional[int] = None, walk="viterbi"):
    """Part 4: (tokens int64 [M], scores fp32 [R], slots int32 [M])."""
    _expect(cand_tok, torch.int64, "cand_tok"), _expect(unary, torch.float32, "unary")
    _expect(pair, torch.float32, "pair"), _expect(row_offsets, torch.int32, "row_offsets")
    M, K = cand_tok.shape
    L = block_len if block_len is not None else (M // R if R else 1)
    d = make_dims(R=R, L=L, M=M, H=8, Vd=K, K=K, walk=walk)
    dev = cand_tok.device
    tokens = torch.empty(M, dtype=torch.int64, device=dev)
    scores = torch.empty(R, dtype=torch.float32, device=dev)
    slots = torch.empty(M, dtype=torch.int32, device=dev)
    check(load().dflash_walk(ctypes.byref(d), _ptr(cand_tok), _ptr(unary), _ptr(pair), _ptr(row_offsets),
                             _ptr(tokens), _ptr(scores), _ptr(slots), _stream(dev)))
    return tokens, scores, slots


def walk_sampled(cand_tok: torch.Tensor, unary: torch.Tensor, pair: torch.Tensor, R: int, uniforms: torch.Tensor, *,
                 temperature: float = 1.0, row_offsets: Optional[torch.Tensor] = None,
                 block_len: Optional[int] = None, with_q: bool = True):
    """Part 4, sampled: (tokens int64 [M], scores fp32 [R], slots int32 [M], q float64 [M, K] or None)."""
    _expect(cand_tok, torch.int64, "cand_tok"), _expect(unary, torch.float32, "unary")
    _expect(pair, torch.float32, "pair"), _expect(row_offsets, torch.int32, "row_offsets")
    _expect(uniforms, torch.float64, "uniforms")
    M, K = cand_tok.shape
    L = block_len if block_len is not None else (M // R if R else 1)
    d = make_dims(R=R, L=L, M=M, H=8, Vd=K, K=K)
    dev = cand_tok.device
    tokens = torch.empty(M, dtype=torch.int64, device=dev)
    scores = torch.empty(R, dtype=torch.float32, device=dev)
    slots = torch.empty(M, dtype=torch.int32, device=dev)
    q = torch.empty((M, K), dtype=torch.float64, device=dev) if with_q else None
    check(load().dflash_walk_sampled(ctypes.byref(d), _ptr(cand_tok), _ptr(unary), _ptr(pair), _ptr(row_offsets),
                                     _ptr(uniforms), float(temperature), _ptr(tokens), _ptr(scores), _ptr(slots),
                                     _ptr(q), _stream(dev)))
    return tokens, scores, slots, q


def check_d2t(d2t_host, Vd: int, Vt: int) -> bool:
    """Host-side d2t check (once, at set-up): raises if a target id is out of range; returns injectivity."""
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(d2t_host, dtype=np.int64))
    if arr.shape != (Vd,):
        raise DFlashError(-1, f"d2t has shape {arr.shape}, expected ({Vd},)")
    inj = ctypes.c_int(0)
    check(load().dflash_check_d2t(arr.ctypes.data, int(Vd), int(Vt), ctypes.byref(inj)))
    return bool(inj.value)
