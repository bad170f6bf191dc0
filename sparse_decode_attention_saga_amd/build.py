"""Compile the HIP library libsaga.so for gfx950, in-tree, with hipcc.

Usage: python -m sparse_decode_attention_saga_amd.build
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libsaga.so")
SOURCES = [os.path.join(HERE, "csrc", "saga_api.hip")]
ARCH = "gfx950"


def source_digest() -> str:
    """sha256 over the library's sources (csrc/ and include/), in name order: names a
    build of the kernels, e.g. for measurements that are valid for one kernel only."""
    import hashlib
    h = hashlib.sha256()
    for d in (os.path.join(HERE, "csrc"), os.path.join(ROOT, "include")):
        for name in sorted(os.listdir(d)):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    """Compile libsaga.so (always recompiles) and return its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed fp32 VALU ops stay off: plain fp32 arithmetic only
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
