"""Build the HIP library in-tree with hipcc for gfx950.

    python -m speculative_decoding_verification_11_amd.build

produces ``speculative_decoding_verification_11_amd/_build/libspecverify.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
# verify.hip: spec_verify, spec_verify_top_p, spec_verify_top_k_top_p,
# spec_verify_early_exit (their kernels also in nucleus.hip and
# early_exit.hip, sharing verify.h); tree.hip: spec_verify_tree; lookup.hip:
# spec_prompt_lookup (common.h is the shared device header of all).
SRCS = [os.path.join(CSRC, f)
        for f in ("verify.hip", "nucleus.hip", "early_exit.hip", "tree.hip", "lookup.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "_build", "libspecverify.so")
ARCH = "gfx950"

# Packed-fp32 VALU ops stay disabled; the host pass warns that it does not
# know the feature, which is harmless.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def source_digest() -> str:
    """sha256[:16] over every kernel source file (name and bytes, sorted):
    the key that ties a committed profile to the code it measured."""
    import hashlib

    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def build_library(extra_flags=(), out: str = LIB, verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIP_FLAGS, *extra_flags, "-I", INCLUDE, "-o", tmp, *SRCS]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}) building {' '.join(SRCS)}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
