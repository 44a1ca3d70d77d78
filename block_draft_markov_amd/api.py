"""Python binding of the draft-step library: argument marshalling only.

Every function takes torch tensors that already live on the GPU, allocates
its outputs (and a workspace) with torch, and calls the C entry point of the
same name on torch's current stream.  No arithmetic of the draft step happens
here.  bf16 inputs may be torch.bfloat16 or 16-bit integer tensors holding
bf16 bit patterns.

The C ABI trusts the sizes it is given, so every tensor's dtype, shape,
contiguity and device is checked here, on the host, before any call: a
mismatch raises TypeError or ValueError and nothing is launched.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import torch

from ._lib import (DFlashError, Dims, MAX_BLOCK_LEN, OPT_FILTER_LOGITS, WALK_GREEDY, WALK_VITERBI, check, load)

__all__ = ["Dims", "DFlashError", "make_dims", "workspace_bytes", "logits_stride", "draft_block",
           "draft_block_sampled", "draft_argmax", "draft_dense", "lm_head", "row_lse", "topk", "pair_scores",
           "walk", "walk_sampled", "lattice", "lattice_noalloc", "check_d2t", "Workspace"]

_WALKS = {"viterbi": WALK_VITERBI, "greedy": WALK_GREEDY, WALK_VITERBI: WALK_VITERBI, WALK_GREEDY: WALK_GREEDY}

_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_I64 = (torch.int64,)
_I32 = (torch.int32,)
_F32 = (torch.float32,)
_F64 = (torch.float64,)


def make_dims(*, R: int, L: int, M: int, H: int, Vd: int, Vt: Optional[int] = None, K: int, r: int = 1,
              walk="viterbi", filter_logits: bool = False) -> Dims:
    if walk not in _WALKS:
        raise ValueError(f"walk must be 'viterbi' or 'greedy', got {walk!r}")
    return Dims(int(R), int(L), int(M), int(H), int(Vd), int(Vd if Vt is None else Vt), int(K), int(r),
                _WALKS[walk], OPT_FILTER_LOGITS if filter_logits else 0)


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
        if ws.device != torch.device(device):
            raise ValueError(f"workspace is on {ws.device}, the tensors on {device}")
        return ws
    key = torch.device(device).index
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


# ------------------------------------------------------------------ validation

def _dtype_names(dtypes) -> str:
    return " or ".join(str(d).replace("torch.", "") for d in dtypes)


def _arg(t, name: str, dtypes: Sequence[torch.dtype], shape: Sequence[Optional[int]],
         optional: bool = False) -> Optional[torch.Tensor]:
    """Check dtype, shape (None = any extent) and contiguity of one tensor argument."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be {_dtype_names(dtypes)}, got {t.dtype}")
    if t.dim() != len(shape) or any(s is not None and s != n for s, n in zip(shape, t.shape)):
        want = "[" + ", ".join("*" if s is None else str(s) for s in shape) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on_device(dev: torch.device, **tensors) -> None:
    """Every given tensor lives on the GPU device `dev`."""
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on the GPU, got {dev}")
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _block_len(R: int, M: int, row_offsets: Optional[torch.Tensor], block_len: Optional[int]) -> int:
    """Rows per request: M / R for uniform blocks; with row_offsets the longest block.

    Ragged offsets are checked on a host copy (non-decreasing from a value
    >= 0 up to at most M, every block at most block_len rows when given),
    since the kernels walk at most block_len rows of a request.
    """
    if row_offsets is None:
        if R == 0:
            if M != 0:
                raise ValueError(f"{M} rows but no requests")
            return int(block_len) if block_len is not None else 1
        if M % R != 0:
            raise ValueError(f"{M} rows do not split into {R} uniform blocks; pass row_offsets")
        L = M // R
        if block_len is not None and int(block_len) != L:
            raise ValueError(f"block_len = {block_len} but uniform blocks of {M} rows over {R} requests have {L}")
        return max(L, 1)
    off = row_offsets.detach().to("cpu", non_blocking=False).tolist()
    if off and off[0] < 0:
        raise ValueError(f"row_offsets[0] = {off[0]} < 0")
    if any(b < a for a, b in zip(off, off[1:])):
        raise ValueError("row_offsets must be non-decreasing")
    if off and off[-1] > M:
        raise ValueError(f"row_offsets[-1] = {off[-1]} exceeds the {M} rows")
    longest = max([b - a for a, b in zip(off, off[1:])] + [1])
    if block_len is None:
        return longest
    if longest > int(block_len):
        raise ValueError(f"a block of {longest} rows is longer than block_len = {block_len}")
    return int(block_len)


def _check_block_len(L: int) -> None:
    if not 1 <= L <= MAX_BLOCK_LEN:
        raise ValueError(f"block length {L} outside [1, {MAX_BLOCK_LEN}]")


def _outs(out, dev, specs):
    """Caller-supplied output tensors (checked like inputs) or new ones."""
    if out is None:
        return tuple(None if s is None else torch.empty(s[2], dtype=s[1][0], device=dev) for s in specs)
    if len(out) != len(specs):
        raise ValueError(f"out must hold {len(specs)} tensors")
    res = []
    for t, s in zip(out, specs):
        if s is None:
            res.append(None)
            continue
        name, dtypes, shape, optional = s
        t = _arg(t, name, dtypes, shape, optional)
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
        res.append(t)
    return tuple(res)


def _lattice_args(hidden, lm_head_w, tables, last_tok, d2t, gate_w, row_offsets):
    """Shapes shared by the whole-step entry points: (M, H, Vd, Vt, r, R)."""
    _arg(hidden, "hidden", _BF16, (None, None))
    M, H = hidden.shape
    _arg(lm_head_w, "lm_head", _BF16, (None, H))
    Vd = lm_head_w.shape[0]
    _arg(tables, "tables", _F32, (2, None, None))
    Vt, r = tables.shape[1], tables.shape[2]
    _arg(last_tok, "last_tok", _I64, (None,))
    R = last_tok.shape[0]
    _arg(d2t, "d2t", _I64, (Vd,), optional=True)
    _arg(gate_w, "gate_w", _F32, (H,), optional=True)
    _arg(row_offsets, "row_offsets", _I32, (R + 1,), optional=True)
    return M, H, Vd, Vt, r, R


# ------------------------------------------------------------------ entry points

def draft_block(hidden: torch.Tensor, lm_head_w: torch.Tensor, tables: torch.Tensor, last_tok: torch.Tensor, *,
                top_k: int, d2t: Optional[torch.Tensor] = None, gate_w: Optional[torch.Tensor] = None,
                row_offsets: Optional[torch.Tensor] = None, block_len: Optional[int] = None, walk="viterbi",
                workspace: Optional[Workspace] = None, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                filter_logits: bool = False):
    """The whole draft step: (tokens int64 [M], scores fp32 [R]).  filter_logits: DFLASH_OPT_FILTER_LOGITS."""
    M, H, Vd, Vt, r, R = _lattice_args(hidden, lm_head_w, tables, last_tok, d2t, gate_w, row_offsets)
    dev = hidden.device
    tokens, scores = _outs(out, dev, [("tokens", _I64, (M,), False), ("scores", _F32, (R,), False)])
    L = _block_len(R, M, row_offsets, block_len)
    _check_block_len(L)
    _on_device(dev, lm_head=lm_head_w, tables=tables, last_tok=last_tok, d2t=d2t, gate_w=gate_w,
               row_offsets=row_offsets)
    d = make_dims(R=R, L=L, M=M, H=H, Vd=Vd, Vt=Vt, K=top_k, r=r, walk=walk, filter_logits=filter_logits)
    wsp, wsn = _ws(workspace, dev).get(workspace_bytes(d))
    check(load().dflash_draft_block(ctypes.byref(d), _ptr(hidden), _ptr(lm_head_w), _ptr(d2t), _ptr(tables),
                                    _ptr(gate_w), _ptr(last_tok), _ptr(row_offsets), _ptr(tokens), _ptr(scores),
                                    wsp, wsn, _stream(dev)))
    return tokens, scores


def draft_block_sampled(hidden: torch.Tensor, lm_head_w: torch.Tensor, tables: torch.Tensor,
                        last_tok: torch.Tensor, uniforms: torch.Tensor, *, top_k: int, temperature: float = 1.0,
                        d2t: Optional[torch.Tensor] = None, gate_w: Optional[torch.Tensor] = None,
                        row_offsets: Optional[torch.Tensor] = None, block_len: Optional[int] = None,
                        workspace: Optional[Workspace] = None, with_q: bool = True, filter_logits: bool = False):
    """The whole step with the sampled walk: (tokens int64 [M], scores fp32 [R], q float64 [M, K] or None)."""
    M, H, Vd, Vt, r, R = _lattice_args(hidden, lm_head_w, tables, last_tok, d2t, gate_w, row_offsets)
    _arg(uniforms, "uniforms", _F64, (M,))
    dev = hidden.device
    L = _block_len(R, M, row_offsets, block_len)
    _check_block_len(L)
    _on_device(dev, lm_head=lm_head_w, tables=tables, last_tok=last_tok, d2t=d2t, gate_w=gate_w,
               row_offsets=row_offsets, uniforms=uniforms)
    d = make_dims(R=R, L=L, M=M, H=H, Vd=Vd, Vt=Vt, K=top_k, r=r, filter_logits=filter_logits)
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
    _arg(hidden, "hidden", _BF16, (None, None))
    M, H = hidden.shape
    _arg(lm_head_w, "lm_head", _BF16, (None, H))
    Vd = lm_head_w.shape[0]
    _arg(d2t, "d2t", _I64, (Vd,), optional=True)
    dev = hidden.device
    Vt = target_vocab if target_vocab is not None else Vd
    specs = [("tokens", _I64, (M,), False), ("values", _F32, (M,), True) if with_values or out is not None else None]
    tokens, values = _outs(out, dev, specs)
    _on_device(dev, lm_head=lm_head_w, d2t=d2t)
    d = make_dims(R=M, L=1, M=M, H=H, Vd=Vd, Vt=Vt, K=min(64, max(Vd, 1)))
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
    M, H, Vd, Vt, r, R = _lattice_args(hidden, lm_head_w, tables, last_tok, d2t, None, row_offsets)
    dev = hidden.device
    specs = [("tokens", _I64, (M,), False), ("values", _F32, (M,), True) if with_values or out is not None else None]
    tokens, values = _outs(out, dev, specs)
    L = _block_len(R, M, row_offsets, block_len)
    _check_block_len(L)
    _on_device(dev, lm_head=lm_head_w, tables=tables, last_tok=last_tok, d2t=d2t, row_offsets=row_offsets)
    d = make_dims(R=R, L=L, M=M, H=H, Vd=Vd, Vt=Vt, K=min(64, max(Vd, 1)), r=r)
    wsp, wsn = _ws(workspace, dev).get(workspace_bytes(d))
    check(load().dflash_draft_dense(ctypes.byref(d), _ptr(hidden), _ptr(lm_head_w), _ptr(d2t), _ptr(tables),
                                    _ptr(last_tok), _ptr(row_offsets), float(out_scale), float(soft_cap),
                                    _ptr(tokens), _ptr(values), wsp, wsn, _stream(dev)))
    return tokens, values


def lm_head(hidden: torch.Tensor, lm_head_w: torch.Tensor, *, workspace: Optional[Workspace] = None,
            with_lse: bool = True, out: Optional[torch.Tensor] = None):
    """Part 1: (logits fp32 [M, V_d] (a view of rows of stride dflash_logits_stride, or of out's
    row stride), lse fp32 [M] or None).  out: fp32 [M, >= V_d] with contiguous rows and a row
    stride that is a multiple of 4."""
    _arg(hidden, "hidden", _BF16, (None, None))
    M, H = hidden.shape
    _arg(lm_head_w, "lm_head", _BF16, (None, H))
    Vd = lm_head_w.shape[0]
    dev = hidden.device
    if out is None:
        _on_device(dev, lm_head=lm_head_w)
        z = torch.empty((M, logits_stride(Vd)), dtype=torch.float32, device=dev)
        ldz = z.stride(0)
    else:
        if not isinstance(out, torch.Tensor) or out.dtype != torch.float32 or out.dim() != 2:
            raise TypeError("out must be a float32 [M, >= V_d] tensor")
        if out.shape[0] != M or out.shape[1] < Vd or out.stride(1) != 1:
            raise ValueError(f"out has shape {list(out.shape)} and strides {out.stride()}; expected [{M}, >= {Vd}] "
                             "with contiguous rows")
        if out.device != dev:
            raise ValueError(f"out is on {out.device}, expected {dev}")
        z = out
        ldz = out.stride(0) if M > 1 else logits_stride(out.shape[1])
        if ldz % 4 != 0 or ldz < Vd:
            raise ValueError(f"out's row stride {ldz} must be a multiple of 4 and at least {Vd}")
        _on_device(dev, lm_head=lm_head_w, out=out)
    lse = torch.empty(M, dtype=torch.float32, device=dev) if with_lse else None
    d = make_dims(R=M, L=1, M=M, H=H, Vd=Vd, K=min(64, max(Vd, 1)))
    wsp, wsn = _ws(workspace, dev).get(workspace_bytes(d))
    check(load().dflash_lm_head(ctypes.byref(d), _ptr(hidden), _ptr(lm_head_w), z.data_ptr() if M else None, ldz,
                                _ptr(lse), wsp, wsn, _stream(dev)))
    return z[:, :Vd], lse


def _rows(logits: torch.Tensor):
    """(M, V_d, row stride) of a logits tensor whose rows are contiguous."""
    if not isinstance(logits, torch.Tensor) or logits.dtype != torch.float32 or logits.dim() != 2:
        raise TypeError("logits must be a float32 [M, V] tensor")
    if logits.stride(1) != 1 and logits.shape[1] > 1:
        raise ValueError("logits must have contiguous rows")
    M, Vd = logits.shape
    ldz = logits.stride(0) if M > 1 else Vd + (-Vd) % 4
    if ldz % 4 != 0 or ldz < Vd:
        raise ValueError(f"the row stride of logits ({ldz}) must be a multiple of 4 and at least {Vd}")
    return M, Vd, ldz


def row_lse(logits: torch.Tensor) -> torch.Tensor:
    M, Vd, ldz = _rows(logits)
    _on_device(logits.device)
    d = make_dims(R=M, L=1, M=M, H=8, Vd=Vd, K=min(64, max(Vd, 1)))
    lse = torch.empty(M, dtype=torch.float32, device=logits.device)
    check(load().dflash_row_lse(ctypes.byref(d), logits.data_ptr() if M else None, ldz, _ptr(lse),
                                _stream(logits.device)))
    return lse


def topk(logits: torch.Tensor, lse: torch.Tensor, top_k: int, *, d2t: Optional[torch.Tensor] = None,
         target_vocab: Optional[int] = None, workspace: Optional[Workspace] = None):
    """Part 2: (cand_idx int32 [M, K], cand_tok int64 [M, K], unary fp32 [M, K])."""
    M, Vd, ldz = _rows(logits)
    _arg(lse, "lse", _F32, (M,))
    _arg(d2t, "d2t", _I64, (Vd,), optional=True)
    dev = logits.device
    _on_device(dev, lse=lse, d2t=d2t)
    d = make_dims(R=M, L=1, M=M, H=8, Vd=Vd, Vt=target_vocab, K=top_k)
    idx = torch.empty((M, top_k), dtype=torch.int32, device=dev)
    tok = torch.empty((M, top_k), dtype=torch.int64, device=dev)
    un = torch.empty((M, top_k), dtype=torch.float32, device=dev)
    wsp, wsn = _ws(workspace, dev).get(workspace_bytes(d))
    check(load().dflash_topk(ctypes.byref(d), logits.data_ptr() if M else None, ldz, _ptr(lse), _ptr(d2t),
                             _ptr(idx), _ptr(tok), _ptr(un), wsp, wsn, _stream(dev)))
    return idx, tok, un


def _cand_args(cand_tok, unary=None):
    _arg(cand_tok, "cand_tok", _I64, (None, None))
    M, K = cand_tok.shape
    _arg(unary, "unary", _F32, (M, K), optional=True)
    return M, K


def pair_scores(cand_tok: torch.Tensor, tables: torch.Tensor, last_tok: torch.Tensor, *,
                gate_w: Optional[torch.Tensor] = None, hidden: Optional[torch.Tensor] = None,
                row_offsets: Optional[torch.Tensor] = None, block_len: Optional[int] = None) -> torch.Tensor:
    """Part 3: pair fp32 [M, K, K]."""
    M, K = _cand_args(cand_tok)
    _arg(tables, "tables", _F32, (2, None, None))
    Vt, r = tables.shape[1], tables.shape[2]
    _arg(last_tok, "last_tok", _I64, (None,))
    R = last_tok.shape[0]
    _arg(row_offsets, "row_offsets", _I32, (R + 1,), optional=True)
    _arg(hidden, "hidden", _BF16, (M, None), optional=gate_w is None)
    H = hidden.shape[1] if hidden is not None else 8
    _arg(gate_w, "gate_w", _F32, (H,), optional=True)
    dev = cand_tok.device
    L = _block_len(R, M, row_offsets, block_len)
    _check_block_len(L)
    _on_device(dev, tables=tables, last_tok=last_tok, gate_w=gate_w, hidden=hidden, row_offsets=row_offsets)
    d = make_dims(R=R, L=L, M=M, H=H, Vd=max(K, 1), Vt=Vt, K=K, r=r)
    pair = torch.empty((M, K, K), dtype=torch.float32, device=dev)
    check(load().dflash_pair_scores(ctypes.byref(d), _ptr(cand_tok), _ptr(tables), _ptr(gate_w), _ptr(hidden),
                                    _ptr(last_tok), _ptr(row_offsets), _ptr(pair), _stream(dev)))
    return pair


def _walk_args(cand_tok, unary, pair):
    M, K = _cand_args(cand_tok, unary)
    if unary is None:
        raise ValueError("unary is required")
    _arg(pair, "pair", _F32, (M, K, K))
    return M, K


def walk(cand_tok: torch.Tensor, unary: torch.Tensor, pair: torch.Tensor, R: int, *,
         row_offsets: Optional[torch.Tensor] = None, block_len: Optional[int] = None, walk="viterbi"):
    """Part 4: (tokens int64 [M], scores fp32 [R], slots int32 [M])."""
    M, K = _walk_args(cand_tok, unary, pair)
    _arg(row_offsets, "row_offsets", _I32, (R + 1,), optional=True)
    dev = cand_tok.device
    L = _block_len(R, M, row_offsets, block_len)
    _check_block_len(L)
    _on_device(dev, unary=unary, pair=pair, row_offsets=row_offsets)
    d = make_dims(R=R, L=L, M=M, H=8, Vd=max(K, 1), K=K, walk=walk)
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
    M, K = _walk_args(cand_tok, unary, pair)
    _arg(row_offsets, "row_offsets", _I32, (R + 1,), optional=True)
    _arg(uniforms, "uniforms", _F64, (M,))
    dev = cand_tok.device
    L = _block_len(R, M, row_offsets, block_len)
    _check_block_len(L)
    _on_device(dev, unary=unary, pair=pair, row_offsets=row_offsets, uniforms=uniforms)
    d = make_dims(R=R, L=L, M=M, H=8, Vd=max(K, 1), K=K)
    tokens = torch.empty(M, dtype=torch.int64, device=dev)
    scores = torch.empty(R, dtype=torch.float32, device=dev)
    slots = torch.empty(M, dtype=torch.int32, device=dev)
    q = torch.empty((M, K), dtype=torch.float64, device=dev) if with_q else None
    check(load().dflash_walk_sampled(ctypes.byref(d), _ptr(cand_tok), _ptr(unary), _ptr(pair), _ptr(row_offsets),
                                     _ptr(uniforms), float(temperature), _ptr(tokens), _ptr(scores), _ptr(slots),
                                     _ptr(q), _stream(dev)))
    return tokens, scores, slots, q


def lattice(cand_tok: torch.Tensor, unary: torch.Tensor, tables: torch.Tensor, last_tok: torch.Tensor, *,
            gate_w: Optional[torch.Tensor] = None, hidden: Optional[torch.Tensor] = None,
            row_offsets: Optional[torch.Tensor] = None, block_len: Optional[int] = None, walk="viterbi",
            workspace: Optional[Workspace] = None, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Parts 3 and 4 in one call (scorer over the packed rows, then the walk):
    (tokens int64 [M], scores fp32 [R])."""
    M, K = _cand_args(cand_tok, unary)
    if unary is None:
        raise ValueError("unary is required")
    _arg(tables, "tables", _F32, (2, None, None))
    Vt, r = tables.shape[1], tables.shape[2]
    _arg(last_tok, "last_tok", _I64, (None,))
    R = last_tok.shape[0]
    _arg(row_offsets, "row_offsets", _I32, (R + 1,), optional=True)
    _arg(hidden, "hidden", _BF16, (M, None), optional=gate_w is None)
    H = hidden.shape[1] if hidden is not None else 8
    _arg(gate_w, "gate_w", _F32, (H,), optional=True)
    dev = cand_tok.device
    tokens, scores = _outs(out, dev, [("tokens", _I64, (M,), False), ("scores", _F32, (R,), False)])
    L = _block_len(R, M, row_offsets, block_len)
    _check_block_len(L)
    _on_device(dev, unary=unary, tables=tables, last_tok=last_tok, gate_w=gate_w, hidden=hidden,
               row_offsets=row_offsets)
    d = make_dims(R=R, L=L, M=M, H=H, Vd=max(K, 1), Vt=Vt, K=K, r=r, walk=walk)
    wsp, wsn = _ws(workspace, dev).get(workspace_bytes(d))
    check(load().dflash_lattice(ctypes.byref(d), _ptr(cand_tok), _ptr(unary), _ptr(tables), _ptr(gate_w),
                                _ptr(hidden), _ptr(last_tok), _ptr(row_offsets), _ptr(tokens), _ptr(scores),
                                wsp, wsn, _stream(dev)))
    return tokens, scores


def lattice_noalloc(cand_tok: torch.Tensor, unary: torch.Tensor, tables: torch.Tensor, last_tok: torch.Tensor, *,
                    gate_w: Optional[torch.Tensor] = None, hidden: Optional[torch.Tensor] = None,
                    row_offsets: Optional[torch.Tensor] = None, block_len: Optional[int] = None, walk="viterbi",
                    out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """lattice() without a workspace: S lives in the library's static device scratch
    (at most LATTICE_NOALLOC_MAX_BYTES per GPU; overlapping calls on one GPU race).
    The outputs are allocated here unless `out` is given; the C call allocates nothing."""
    M, K = _cand_args(cand_tok, unary)
    if unary is None:
        raise ValueError("unary is required")
    _arg(tables, "tables", _F32, (2, None, None))
    Vt, r = tables.shape[1], tables.shape[2]
    _arg(last_tok, "last_tok", _I64, (None,))
    R = last_tok.shape[0]
    _arg(row_offsets, "row_offsets", _I32, (R + 1,), optional=True)
    _arg(hidden, "hidden", _BF16, (M, None), optional=gate_w is None)
    H = hidden.shape[1] if hidden is not None else 8
    _arg(gate_w, "gate_w", _F32, (H,), optional=True)
    dev = cand_tok.device
    tokens, scores = _outs(out, dev, [("tokens", _I64, (M,), False), ("scores", _F32, (R,), False)])
    L = _block_len(R, M, row_offsets, block_len)
    _check_block_len(L)
    _on_device(dev, unary=unary, tables=tables, last_tok=last_tok, gate_w=gate_w, hidden=hidden,
               row_offsets=row_offsets)
    d = make_dims(R=R, L=L, M=M, H=H, Vd=max(K, 1), Vt=Vt, K=K, r=r, walk=walk)
    with torch.cuda.device(dev):
        check(load().dflash_lattice_noalloc(ctypes.byref(d), _ptr(cand_tok), _ptr(unary), _ptr(tables),
                                            _ptr(gate_w), _ptr(hidden), _ptr(last_tok), _ptr(row_offsets),
                                            _ptr(tokens), _ptr(scores), _stream(dev)))
    return tokens, scores


def check_d2t(d2t_host, Vd: int, Vt: int) -> bool:
    """Host-side d2t check (once, at set-up): raises if a target id is out of range; returns injectivity."""
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(d2t_host, dtype=np.int64))
    if arr.shape != (Vd,):
        raise DFlashError(-1, f"d2t has shape {arr.shape}, expected ({Vd},)")
    inj = ctypes.c_int(0)
    check(load().dflash_check_d2t(arr.ctypes.data, int(Vd), int(Vt), ctypes.byref(inj)))
    return bool(inj.value)
