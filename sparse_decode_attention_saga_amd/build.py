"""Compile the HIP library libsaga.so for gfx950, in-tree, with hipcc.

Usage: python -m sparse_decode_attention_saga_amd.build
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libsaga.so")
SOURCES = [os.path.join(HERE, "csrc", n) for n in ("saga_api.hip", "saga_layer.hip", "saga_merge.hip")]
# the decode-attention kernels' sources (what a build of those kernels depends on;
# the layer's projection kernels are not among them)
LIB_FILES = [os.path.join(HERE, "csrc", n) for n in ("saga_api.hip", "saga_device.hpp", "saga_kernels.hpp")] + \
    [os.path.join(ROOT, "include", "saga.h")]
# streaming-read probe used by the benchmark (not part of the decode library)
PROBE_PATH = os.path.join(HERE, "libsaga_probe.so")
PROBE_SOURCES = [os.path.join(HERE, "csrc", "stream_probe.hip")]
ARCH = "gfx950"


def source_digest() -> str:
    """sha256 over the decode library's sources, in order: names a build of the
    kernels, e.g. for measurements that are valid for one kernel only."""
    import hashlib
    h = hashlib.sha256()
    for path in LIB_FILES:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(sources, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed fp32 VALU ops stay off: plain fp32 arithmetic only
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-o", tmp] + sources
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile libsaga.so and the benchmark's read probe (always recompiles); returns
    the library's path."""
    _compile(SOURCES, LIB_PATH, verbose)
    _compile(PROBE_SOURCES, PROBE_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
