"""Build libulys.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m ulysses_sequence_attention_amd.build`` (or call ``build()``).
Every call recompiles; the library lands next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libulys.so")
SOURCES = ["api.hip", "repack.hip", "attn.hip", "merge.hip"]
# per-source flags: the attention kernel never relies on NaN semantics (inputs
# must be finite; masked scores are -inf), so its max reductions need no
# canonicalising instructions
SOURCE_FLAGS = {"attn.hip": ["-fno-honor-nans"]}
_EXTRA: list = []

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 VALU ops stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast",
    # MFMA results in VGPRs: the softmax reads the score accumulators with VALU
    # ops, and the accumulators fit the VGPR budget (no AGPR round trips)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _compile(src: str) -> str:
    out = os.path.join(OBJ, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *_EXTRA, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = False, lib: str = LIB, extra=()) -> str:
    os.makedirs(OBJ, exist_ok=True)
    global _EXTRA
    _EXTRA = list(extra)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
