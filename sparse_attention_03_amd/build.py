"""Build the HIP library libdsa.so for gfx950, in-tree (next to this file).

    python -m sparse_attention_03_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
SOURCES = ["api.cpp", "indexer.hip", "indexer_fp8.hip", "topk.hip", "mla.hip", "quant.hip", "merge.hip", "msa.hip"]
# Packed-FP32 VALU forms are kept out of the generated code on purpose.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA results in ordinary VGPRs: no accvgpr copies before the VALU epilogues
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-x", "hip", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("libdsa build failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))


def source_digest() -> str:
    """First 16 hex digits of the sha256 of the library sources, the public
    header and the compile flags: names the build a profile was taken on."""
    import glob
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(HERE)
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))) + [os.path.join(root, "include", "dsa.h")]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(FLAGS).encode())
    return h.hexdigest()[:16]
