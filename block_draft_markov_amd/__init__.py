"""MI355X (gfx950) draft step of DFlash/DSpark speculative decoding.

Hand-written HIP kernels behind the C ABI of include/dflash_draft.h
(libdflash_draft.so, built by ``python -m block_draft_markov_amd.build``);
this package is the thin Python binding over it.  Nothing here falls back to
a CPU path: calls fail if the library is missing.
"""
from ._lib import (DFlashError, Dims, EHIP, EINVAL, EUNSUPPORTED, EWORKSPACE, LIB_PATH, MAX_BLOCK_LEN, MAX_TOP_K,
                   OK, SIGNATURES, WALK_GREEDY, WALK_VITERBI, load)

__all__ = ["DFlashError", "Dims", "load", "LIB_PATH", "SIGNATURES", "WALK_VITERBI", "WALK_GREEDY", "OK", "EINVAL",
           "EUNSUPPORTED", "EWORKSPACE", "EHIP", "MAX_TOP_K", "MAX_BLOCK_LEN", "api"]


def __getattr__(name):
    # the torch-facing binding is imported on first use, so that loading the
    # library (and the CPU tests of the ABI) does not need torch
    if name == "api":
        import importlib
        return importlib.import_module(__name__ + ".api")
    raise AttributeError(name)
