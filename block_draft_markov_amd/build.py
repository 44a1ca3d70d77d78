"""Build libdflash_draft.so (gfx950) in-tree with hipcc.

    python -m block_draft_markov_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdflash_draft.so")
SOURCES = ["abi.hip", "lmhead.hip", "topk.hip", "lattice.hip", "dense.hip"]
ARCH = "gfx950"

# -packed-fp32-ops off: packed fp32 VALU forms are never emitted.
# -Wno-inline-asm: the LDS-DMA loads of the batched lm_head kernel set m0 in
# inline assembly, which clang flags because m0 is a reserved register; no
# compiler-generated code of those kernels uses m0 (a CPU test checks the
# generated assembly for exactly that).
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-inline-asm",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def device_asm(src: str) -> str:
    """gfx950 assembly of one source file under the library's flags (for inspection)."""
    r = subprocess.run([_hipcc()] + HIPCC_FLAGS + ["-S", "--offload-device-only", os.path.join(CSRC, src),
                                                   "-o", "-"], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(r.stderr[-4000:])
    return r.stdout


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library; returns its path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    hipcc = _hipcc()

    def compile_one(src):
        obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
        msg = _run([hipcc] + HIPCC_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
