"""Build libsparse_attn.so in-tree with hipcc for gfx950.

Usage: ``python -m structured_sparse_causal_amd.build`` (or
``__graft_entry__.build()``).  Objects go to ``_build/`` beside this file; the
shared library lands next to this file, where the binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsparse_attn.so")
SOURCES = ["api.hip", "prefill.hip", "skip.hip", "decode.hip", "backward.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list:
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
            # no packed-fp32 instructions in any generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # keep MFMA accumulators in ordinary VGPRs: the softmax reads every
            # score and rescales the output accumulator, so AGPR homes would
            # cost a copy per value per tile
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-Wno-unused-command-line-argument"]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [cc] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
