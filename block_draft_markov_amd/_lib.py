"""ctypes loader of libdflash_draft.so: argument types of every C entry point.

There is no fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdflash_draft.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
WALK_VITERBI, WALK_GREEDY = 0, 1
OPT_FILTER_LOGITS = 1
MAX_TOP_K, MAX_BLOCK_LEN = 64, 100
LATTICE_NOALLOC_MAX_BYTES = 16 << 20

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t


class Dims(ctypes.Structure):
    """Mirror of struct dflash_dims."""
    _fields_ = [
        ("num_requests", _I32),
        ("block_len", _I32),
        ("total_rows", _I32),
        ("hidden", _I32),
        ("draft_vocab", _I32),
        ("target_vocab", _I32),
        ("top_k", _I32),
        ("rank", _I32),
        ("walk", _I32),
        ("options", _I32),
    ]


_PD = ctypes.POINTER(Dims)

# name -> (restype, argtypes)
SIGNATURES = {
    "dflash_workspace_bytes": (_SZ, [_PD]),
    "dflash_logits_stride": (_I64, [_I32]),
    "dflash_draft_block": (ctypes.c_int, [_PD, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dflash_lm_head": (ctypes.c_int, [_PD, _P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "dflash_row_lse": (ctypes.c_int, [_PD, _P, _I64, _P, _P]),
    "dflash_topk": (ctypes.c_int, [_PD, _P, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dflash_pair_scores": (ctypes.c_int, [_PD, _P, _P, _P, _P, _P, _P, _P, _P]),
    "dflash_walk": (ctypes.c_int, [_PD, _P, _P, _P, _P, _P, _P, _P, _P]),
    "dflash_lattice": (ctypes.c_int, [_PD, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dflash_lattice_noalloc": (ctypes.c_int, [_PD, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "dflash_draft_argmax": (ctypes.c_int, [_PD, _P, _P, _P, ctypes.c_float, ctypes.c_float, _P, _P, _P, _SZ, _P]),
    "dflash_draft_dense": (ctypes.c_int, [_PD, _P, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_float, _P, _P, _P,
                                          _SZ, _P]),
    "dflash_draft_block_sampled": (ctypes.c_int, [_PD, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P,
                                                  _P, _SZ, _P]),
    "dflash_walk_sampled": (ctypes.c_int, [_PD, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P, _P]),
    "dflash_check_d2t": (ctypes.c_int, [_P, _I32, _I32, ctypes.POINTER(ctypes.c_int)]),
    "dflash_last_error": (ctypes.c_char_p, []),
}

_lib = None
_lock = threading.Lock()


class DFlashError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"dflash error {code}: {message}")
        self.code = code
        self.message = message


def load() -> ctypes.CDLL:
    """Load the HIP library (built by block_draft_markov_amd.build); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built; run `python -m block_draft_markov_amd.build`")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def check(rc: int) -> None:
    if rc != OK:
        raise DFlashError(rc, load().dflash_last_error().decode())
