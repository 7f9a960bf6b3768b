"""Build the HIP library for gfx950, in-tree (next to this file):

  libdsa.so        the release library;
  libdsa_debug.so  the same sources with DSA_DEBUG=1: every kernel notes the
                   device metadata it had to clamp or skip, read back with
                   dsa_check_debug_flag().

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
DEBUG_LIB = os.path.join(HERE, "libdsa_debug.so")
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


def _command(out: str, debug: bool) -> list:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    extra = ["-DDSA_DEBUG=1"] if debug else []
    return [hipcc(), *FLAGS, *extra, "-x", "hip", *srcs, "-o", out]


def build(verbose: bool = False, debug: bool = True) -> str:
    """Compile libdsa.so (and libdsa_debug.so unless debug=False), the two
    compilations side by side; returns the release library's path."""
    jobs = [(LIB, False)] + ([(DEBUG_LIB, True)] if debug else [])
    procs = []
    for out, dbg in jobs:
        cmd = _command(out + ".tmp", dbg)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for out, pr in procs:
        log, _ = pr.communicate()
        if pr.returncode != 0:
            sys.stderr.write(log)
            failed.append(os.path.basename(out))
        else:
            os.replace(out + ".tmp", out)
    if failed:
        raise RuntimeError("build failed: " + ", ".join(failed))
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
